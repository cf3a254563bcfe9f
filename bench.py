#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

A step is one k3moe_layer call (router, top-k, permute, routed MXFP4 expert
FFN, shared bf16 experts, combine) over one batch that is already resident in
HBM.  The default workload is decode at batch 1 (d 7168, f 2048, 896 experts
top-16, 2 shared experts, the whole layer's experts resident).  Every step
uses a different token, so each step routes to a different expert set and the
routed weights come from HBM rather than from a cache warmed by the previous
step.

Printed: one JSON line with throughput (tokens/s), the roofline of the
dominant kernel (the routed gate/up MXFP4 GEMV, timed live with HIP events on
the stream it runs on) and the CPU oracle timed on a bounded sample of the same
workload on this host.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (MXFP4 bytes) at batch 1/64/4096"
PMC_FILE = os.path.join(ROOT, "profiles", "gateup_t1_decode_b1_counters.md")
GEMV_SRC = os.path.join(ROOT, "mxfp4_routed_expert_gemv_amd", "csrc", "gemv.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(GEMV_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(PMC_FILE):
        return None
    text = open(PMC_FILE).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_h or not m_t or m_h.group(1) != kernel_source_hash():
        return None
    return float(m_t.group(1))


def cpu_baseline(cfg, budget_s: float):
    """The oracle, as it stands, on consecutive tokens of the workload until
    about budget_s seconds of oracle time are spent (input generation excluded)."""
    import gen
    import oracle
    orc = oracle.default()
    wr = gen.router(cfg)
    shared = gen.shared_bank(cfg)
    spent, n = 0.0, 0
    T = cfg.T
    while spent < budget_s and n < 64:
        x = gen.x(cfg.with_tokens((n + 1) * T), n * T, (n + 1) * T)
        x64 = oracle.to_f64(x)
        t0 = time.perf_counter()
        _, idx, w = orc.route(x64, wr, cfg.k)
        spent += time.perf_counter() - t0
        experts = {int(e): gen.routed_expert(cfg, int(e)) for e in set(idx.ravel().tolist())}
        t0 = time.perf_counter()
        orc.token_outputs(x, idx, w, lambda e: experts[e], shared)
        spent += time.perf_counter() - t0
        n += 1
    return dict(value=n * T / spent, unit="tokens/s", cores=orc.threads(), kind="oracle",
                sample=f"{n} batch(es) of {T} token(s) of {cfg.name}, full layer per token "
                       f"(fp64 router, top-k, {cfg.k} MXFP4 experts, {cfg.n_shared} shared, "
                       f"combine), {spent:.1f} s of oracle time")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_b1",
                    help="decode_b1 (default), decode_b64, prefill_4096, prefill_16384_zipf")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, one device-to-device copy of this many MiB "
                         "(a known-size kernel to scale HBM counters by)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): this layer is built and measured on a single MI355X; the way it "
              "would shard across GPUs is described, not run.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gen
    import gen.device
    from mxfp4_routed_expert_gemv_amd import DIAG_COUNT, OP_LAYER, lib
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = gen.get(args.workload)
    K, W = args.steps, args.warmup
    log(f"workload {cfg.name}: T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")

    wl = gen.device.build(cfg.with_tokens(1), routed_on_device=True)
    w_router = wl.w_router
    if cfg.zipf_s is not None:
        w_router = gen.device._to_dev_bf16(gen.router(cfg), "cuda")
    layer = MoELayer(w_router, wl.routed, wl.shared, cfg.k, out_dtype=torch.bfloat16)
    T = cfg.T
    xs = gen.device.activations(cfg.with_tokens((K + W) * T))   # K+W distinct batches
    batches = [xs[i * T:(i + 1) * T] for i in range(K + W)]
    shape = layer.shape(T, xs.dtype)
    ws = layer.workspace(shape, OP_LAYER)
    out = torch.empty((T, cfg.d), dtype=torch.bfloat16, device="cuda")
    diag = torch.zeros(DIAG_COUNT, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log("weights resident; warming up")

    stream = torch.cuda.current_stream()
    for i in range(W):
        layer(batches[i], out=out, diag=diag, workspace=ws)
    torch.cuda.synchronize()

    # ---------------------------------------------------------- timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        layer(batches[W + i], out=out, diag=diag, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / K
    log(f"layer: {ms_per_step * 1e3:.1f} us/step (wall {wall / K * 1e6:.1f} us/step)")

    # ------------------------------------------- dominant kernel, HIP events
    # The routed gate/up GEMV alone: route + permute of K fresh tokens are
    # prepared first, then the K gate/up launches run back to back between two
    # events on the stream they are launched on (each launch reads its own
    # token's expert set, so the weights stream from HBM).
    prepared, touched = [], []
    for i in range(K):
        x = batches[W + i]
        idx, _, _ = layer.route(x)
        counts, offsets, sp, _ = layer.permute(idx)
        prepared.append((x, offsets, sp))
        touched.append(int((counts > 0).sum().item()))
    h = torch.empty((T * cfg.k, cfg.f), dtype=torch.float32, device="cuda")
    layer.expert_gateup(*prepared[0], h=h)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for x, offsets, sp in prepared:
        layer.expert_gateup(x, offsets, sp, h=h)
    b.record(stream)
    torch.cuda.synchronize()
    gu_ms = [a.elapsed_time(b) / K]
    per_expert_gu = lib.k3moe_mxfp4_bytes(2 * cfg.f, cfg.d)
    gu_bytes = sum(touched) / len(touched) * per_expert_gu
    gu_avg_s = sum(gu_ms) / len(gu_ms) / 1e3
    achieved = gu_bytes / gu_avg_s / 1e9
    log(f"gate/up GEMV: {gu_avg_s * 1e6:.1f} us avg, {gu_bytes / 1e6:.1f} MB/launch, "
        f"{achieved:.0f} GB/s")

    # whole-layer algorithmic bytes (MXFP4 experts touched + shared + router + x, out)
    per_expert = lib.k3moe_mxfp4_bytes(2 * cfg.f, cfg.d) + lib.k3moe_mxfp4_bytes(cfg.d, cfg.f)
    layer_bytes = (sum(touched) / len(touched) * per_expert
                   + cfg.n_shared * 3 * cfg.f_shared * cfg.d * 2 + cfg.E * cfg.d * 2
                   + 2 * T * cfg.d * 2)
    traffic = stored_traffic()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calib_copy_mib} MiB done")

    result = {
        "metric": METRIC,
        "value": T / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens_per_step": T, "d": cfg.d, "f": cfg.f,
                   "experts": cfg.E, "top_k": cfg.k, "shared_experts": cfg.n_shared,
                   "weights": "routed MXFP4 (E2M1 + E8M0/32), shared and router bf16",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gateup_t1" if T == 1 else "gateup_persistent", "bytes_per_launch": gu_bytes,
                     "avg_launch_us": gu_avg_s * 1e6},
        "layer_hbm_gbs": layer_bytes / (ms_per_step / 1e3) / 1e9,
        "layer_bytes_per_step": layer_bytes,
        "rechecked_tokens": int(diag[0].item()),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
