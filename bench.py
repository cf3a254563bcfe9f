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
dominant kernel (the routed gate/up kernel, timed live with HIP events on the
stream it runs on: HBM-bound for decode batches, bound by the scaled
FP8 x MXFP4 matrix-core instruction for large batches), per-step percentiles, and the CPU oracle timed on a bounded sample
of the same workload on this host.
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
BF16_MFMA_PEAK_TFLOPS = 2500.0     # dense bf16 matrix peak (the shared experts' format)
FP8_MFMA_PEAK_TFLOPS = 5000.0      # dense fp8 matrix peak: the rate of the scaled E4M3 x MXFP4
                                   # instruction the large-batch routed path issues
MXFP4_MFMA_PEAK_TFLOPS = 10100.0   # dense MXFP4 x MXFP4 matrix peak, for reference
X_PASSES = 2                       # E4M3 passes that carry bf16 x exactly (one MFMA each)
SPIN_CYCLES = 20_000_000           # ~10 ms of GPU spin ahead of a timed run of launches
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (MXFP4 bytes) at batch 1/64/4096"
PMC_FILE = os.path.join(ROOT, "profiles", "gateup_1tok_decode_b1_counters.md")
KERNEL_SRC = os.path.join(ROOT, "mxfp4_routed_expert_gemv_amd", "csrc", "mxscale.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as fh:
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
    """The oracle, as it stands, on consecutive tokens of the workload (chunks of
    up to 8 tokens, the workload's own router and experts) until about budget_s
    seconds of oracle time are spent (input generation excluded)."""
    import gen
    import oracle
    orc = oracle.default()
    wr = gen.router(cfg)
    shared = gen.shared_bank(cfg)
    spent, done = 0.0, 0
    chunk = min(cfg.T, 8)
    limit = cfg.T * 64
    experts = {}
    while spent < budget_s and done < limit:
        x = gen.x(cfg, done, done + chunk) if done + chunk <= cfg.T else \
            gen.x(cfg.with_tokens(done + chunk), done, done + chunk)
        x64 = oracle.to_f64(x)
        t0 = time.perf_counter()
        _, idx, w = orc.route(x64, wr, cfg.k)
        spent += time.perf_counter() - t0
        need = set(idx.ravel().tolist())
        experts = {e: experts[e] if e in experts else gen.routed_expert(cfg, int(e)) for e in need}
        t0 = time.perf_counter()
        orc.token_outputs(x, idx, w, lambda e: experts[e], shared)
        spent += time.perf_counter() - t0
        done += chunk
    return dict(value=done / spent, unit="tokens/s", cores=orc.threads(), kind="oracle",
                sample=f"first {done} token(s) of {cfg.name} in chunks of {chunk}, full layer "
                       f"per token (fp64 router, top-k, {cfg.k} MXFP4 experts, {cfg.n_shared} "
                       f"shared, combine), {spent:.1f} s of oracle time")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50 for decode workloads, 10 for prefill)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="warm-up steps (default 5 for decode workloads, 3 for prefill)")
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
    from mxfp4_routed_expert_gemv_amd import DIAG_COUNT, OP_EXPERT_FFN, OP_LAYER, k3moe_expert_ffn, lib
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = gen.get(args.workload)
    big = cfg.T >= 1024
    K = args.steps if args.steps is not None else (10 if big else 50)
    W = args.warmup if args.warmup is not None else (3 if big else 5)
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
    # K steps between two events (an event recorded after every step costs
    # about 3 us of GPU time at decode_b1, so the per-step times come from a
    # second pass over the same batches, used only for the percentiles)
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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev[0].record(stream)
    for i in range(K):
        layer(batches[W + i], out=out, workspace=ws)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    steps_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(K))

    def pct(q):
        return steps_ms[min(K - 1, int(round(q * (K - 1))))]
    log(f"layer: {ms_per_step * 1e3:.1f} us/step (wall {wall / K * 1e6:.1f} us/step; "
        f"p10 {pct(0.1) * 1e3:.1f} p50 {pct(0.5) * 1e3:.1f} p90 {pct(0.9) * 1e3:.1f} us)")

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
    # a spin kernel ahead of the first event lets the host enqueue the K
    # launches ahead of the GPU, so the events time back-to-back kernels and
    # not the host's per-call overhead
    torch.cuda._sleep(SPIN_CYCLES)
    a.record(stream)
    for x, offsets, sp in prepared:
        layer.expert_gateup(x, offsets, sp, h=h)
    b.record(stream)
    torch.cuda.synchronize()
    gu_ms = [a.elapsed_time(b) / K]
    per_expert_gu = lib.k3moe_mxfp4_bytes(2 * cfg.f, cfg.d)
    gu_bytes = sum(touched) / len(touched) * per_expert_gu
    gu_avg_s = sum(gu_ms) / len(gu_ms) / 1e3
    gu_gbs = gu_bytes / gu_avg_s / 1e9
    gu_flops = 2.0 * T * cfg.k * 2 * cfg.f * cfg.d      # useful gate/up FLOPs per launch
    gu_tflops = gu_flops / gu_avg_s / 1e12
    mfma_class = layer.path_class(T) == 1
    # the routed experts take the scaled matrix-core instruction at any batch
    # size for bf16 activations and d, f multiples of 512
    routed_scaled = cfg.x_dtype == "bf16" and cfg.d % 512 == 0 and cfg.f % 512 == 0
    # the bound of the gate/up kernel: useful FLOPs per weight byte against the
    # ridge of the instruction it issues (fp8 matrix peak / HBM peak)
    mfma_bound = routed_scaled and gu_flops / gu_bytes >= FP8_MFMA_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS
    log(f"gate/up: {gu_avg_s * 1e6:.1f} us avg, {gu_bytes / 1e6:.1f} MB/launch, "
        f"{gu_gbs:.0f} GB/s, {gu_tflops:.1f} TFLOP/s useful")

    # routed expert FFN (gate/up + down) of the same prepared batches
    y = torch.empty((T * cfg.k, cfg.d), dtype=torch.float32, device="cuda")
    fws = layer.workspace(shape, OP_EXPERT_FFN)
    torch.cuda._sleep(SPIN_CYCLES)
    a.record(stream)
    for x, offsets, sp in prepared:
        k3moe_expert_ffn(shape, layer.routed_bank, x, offsets, sp, y, fws)
    b.record(stream)
    torch.cuda.synchronize()
    ffn_ms = a.elapsed_time(b) / K
    ffn_flops = 2.0 * T * cfg.k * 3 * cfg.f * cfg.d
    per_expert_ffn = lib.k3moe_mxfp4_bytes(2 * cfg.f, cfg.d) + lib.k3moe_mxfp4_bytes(cfg.d, cfg.f)
    ffn_bytes = sum(touched) / len(touched) * per_expert_ffn
    log(f"routed FFN: {ffn_ms * 1e3:.1f} us avg, {ffn_bytes / (ffn_ms / 1e3) / 1e9:.0f} GB/s, "
        f"{ffn_flops / (ffn_ms / 1e3) / 1e12:.1f} TFLOP/s useful")

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
        "roofline": ({"bound": "mfma", "achieved": gu_tflops, "peak": FP8_MFMA_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": gu_tflops / FP8_MFMA_PEAK_TFLOPS,
                      "traffic": None, "kernel": "mx_gemm_scaled (gate/up)",
                      "flops_per_launch": gu_flops, "avg_launch_us": gu_avg_s * 1e6,
                      "issued_tflops": gu_tflops * X_PASSES,
                      "frac_of_mxfp4_peak": gu_tflops / MXFP4_MFMA_PEAK_TFLOPS,
                      "mxfp4_gbs": gu_gbs}
                     if mfma_bound else
                     {"bound": "hbm", "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": gu_gbs / HBM_PEAK_GBS, "traffic": traffic if T == 1 else None,
                      "kernel": ("gateup_1tok" if T == 1 and routed_scaled
                                 else "mx_gemm_scaled (gate/up)" if routed_scaled
                                 else "gateup_persistent"),
                      "bytes_per_launch": gu_bytes, "avg_launch_us": gu_avg_s * 1e6,
                      "useful_tflops": gu_tflops}),
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "layer_hbm_gbs": layer_bytes / (ms_per_step / 1e3) / 1e9,
        "layer_bytes_per_step": layer_bytes,
        "rechecked_tokens": int(diag[0].item()),
    }
    ffn_tflops = ffn_flops / (ffn_ms / 1e3) / 1e12
    ffn_gbs = ffn_bytes / (ffn_ms / 1e3) / 1e9
    result["routed_ffn"] = {"avg_us": ffn_ms * 1e3, "mxfp4_bytes": ffn_bytes,
                            "mxfp4_gbs": ffn_gbs, "frac_of_hbm_peak": ffn_gbs / HBM_PEAK_GBS,
                            "useful_tflops": ffn_tflops,
                            "frac_of_fp8_peak": ffn_tflops / FP8_MFMA_PEAK_TFLOPS,
                            "frac_of_mxfp4_peak": ffn_tflops / MXFP4_MFMA_PEAK_TFLOPS}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
