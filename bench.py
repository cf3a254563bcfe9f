#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

A step is one k3moe_layer call (router, top-k, permute, routed MXFP4 expert
FFN, shared bf16 experts, combine) over one batch that is already resident in
HBM.  The layer has d 7168, f 2048, 896 experts top-16 and 2 shared experts,
with the whole layer's experts resident.  One run measures the four workloads
of the metric, each with the same seeded synthetic weights:
  decode_b1           1 token a step (the headline line)
  decode_b64          64 tokens a step
  prefill_4096        4096 tokens a step
  prefill_16384_zipf  16384 tokens a step, expert popularity skewed Zipf(1.1)
and the two prefill batches again with the quantised-activation mode
(x and h in MXFP4, so the routed products run on the FP4 matrix rate): an
approximation of the layer, reported beside the exact one, never in its place;
and the decode batches with the routed experts in the pages' second format,
RVQ3 (three 256-entry codebooks per 8-weight vector, 3.00 bits per weight),
multiplied through per-token partial-dot tables; and decode at batch 1 with
the routed experts in pinned host memory, taken through an HBM cache of 128
expert slots (misses copied over PCIe on a second stream while the shared
experts run), once on uniform routing and once on Zipf(1.1)-skewed routing.
Decode steps each take fresh tokens, so every step routes to another expert
set and the routed weights stream from HBM, not from a cache warmed by the
previous step; prefill batches touch every expert at every step.

Printed: one JSON line.  Its top-level fields are the headline workload's
(decode_b1 by default): throughput in tokens/s, the roofline of the dominant
kernel (the routed gate/up kernel, timed live with HIP events on the stream it
runs on: HBM-bound for decode and prefill_4096, bound by the scaled FP8 x
MXFP4 matrix-core instruction for the skewed 16384-token batch), per-step
percentiles, and the CPU oracle timed on a bounded sample of the same
workload on this host.  "workloads" holds the same record for every workload
measured.
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
FP8_MFMA_PEAK_TFLOPS = 5000.0      # dense fp8 matrix peak: the rate of the scaled E4M3 x MXFP4
                                   # instruction the batched routed path issues
MXFP4_MFMA_PEAK_TFLOPS = 10100.0   # dense MXFP4 x MXFP4 matrix peak, for reference
X_PASSES = 2                       # E4M3 passes that carry bf16 x exactly (one MFMA each)
SPIN_CYCLES = 20_000_000           # ~10 ms of GPU spin ahead of a timed run of launches
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (MXFP4 bytes) at batch 1/64/4096"
WORKLOADS = ["decode_b1", "decode_b64", "prefill_4096", "prefill_16384_zipf",
             "prefill_4096_mxfp4act", "prefill_16384_zipf_mxfp4act", "decode_b1_rvq3",
             "decode_b64_rvq3", "decode_b1_hostcache"]
QACT = "_mxfp4act"   # suffix: the routed experts' activations quantised to MXFP4
RVQ = "_rvq3"        # suffix: the routed experts in the RVQ3 format (3.00 bits per weight)
RVQ_CODEBOOK_BYTES = 3 * 256 * 8 * 4   # per expert matrix
HOST = "_hostcache"  # suffix: routed experts in pinned host memory behind an HBM expert cache
CACHE_SLOTS = 128
PCIE_PEAK_GBS = 64.0               # PCIe 5.0 x16, one direction (the host link's published rate)
KERNEL_SRC = os.path.join(ROOT, "mxfp4_routed_expert_gemv_amd", "csrc", "mxscale.hip")
RVQ_SRC = os.path.join(ROOT, "mxfp4_routed_expert_gemv_amd", "csrc", "rvq.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pmc_file(workload: str) -> str:
    kernel = ("gateup_1tok" if workload == "decode_b1" else
              "rvq_partial" if workload.endswith(RVQ) else "mx_gemm_scaled")
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")


def kernel_source_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary of this workload, if it was taken on the current kernel source;
    else None."""
    path = pmc_file(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    src = RVQ_SRC if workload.endswith(RVQ) else KERNEL_SRC
    if not m_h or not m_t or m_h.group(1) != kernel_source_hash(src):
        return None
    return float(m_t.group(1))


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline_one_token(cfg, budget_s: float, act: str = "exact"):
    """Decode at batch 1: the oracle's whole layer (fp64 router, top-k, the
    token's experts, the shared experts, combine), one token after another,
    until about budget_s seconds of oracle time are spent."""
    import gen
    import oracle
    orc = oracle.default()
    wr = gen.router(cfg)
    shared = gen.shared_bank(cfg)
    spent, done = 0.0, 0
    while spent < budget_s and done < 64:
        x = gen.x(cfg.with_tokens(done + 1), done, done + 1)
        t0 = time.perf_counter()
        _, idx, w = orc.route(oracle.to_f64(x), wr, cfg.k)
        spent += time.perf_counter() - t0
        get = gen.rvq_expert if act == "rvq3" else gen.routed_expert
        need = {int(e): get(cfg, int(e)) for e in idx.ravel()}   # untimed
        t0 = time.perf_counter()
        orc.token_outputs(x, idx, w, lambda e: need[e], shared, act)
        spent += time.perf_counter() - t0
        done += 1
    return dict(value=done / spent, unit="tokens/s", cores=orc.threads(), kind="oracle",
                sample=f"the first {done} token(s) of {cfg.name}, one at a time through the "
                       f"whole oracle layer (fp64 router, top-k, {cfg.k} {act} experts, "
                       f"{cfg.n_shared} shared, combine); {spent:.1f} s of oracle time")


def cpu_baseline_batch(cfg, budget_s: float, act: str = "exact"):
    """A batch: the oracle's router and permute on the whole batch (timed);
    then expert FFNs of a seeded random sample of the touched experts, each
    on up to 256 of its pairs (the oracle decodes an expert's weights once for
    all its rows, then multiplies row by row), until about budget_s / 2
    seconds are spent, plus one expert on 1 and on 256 rows.  A least-squares
    line time = a + b * rows through these gives the routed estimate, the sum
    over touched experts of a + b * pairs(e).  The shared experts run on the first 64 tokens and the
    combine on the first 512, scaled by token count."""
    import numpy as np

    import gen
    import oracle
    orc = oracle.default()
    ffn = orc.expert(act)
    T = cfg.T
    x64 = oracle.to_f64(gen.x(cfg))
    wr = gen.router(cfg)
    t0 = time.perf_counter()
    _, idx, w = orc.route(x64, wr, cfg.k)
    counts, offsets, sp, pp = orc.permute(idx, cfg.E)
    t_route = time.perf_counter() - t0
    touched = np.nonzero(counts)[0]
    order = np.random.default_rng(0).permutation(touched)
    rows, secs = [], []
    # two anchors for the line: one expert on 1 row and on 256 rows
    ex = (gen.rvq_expert if act == "rvq3" else gen.routed_expert)(cfg, int(order[0]))
    for nr in (1, min(256, T)):
        t0 = time.perf_counter()
        ffn(ex, x64[:nr])
        secs.append(time.perf_counter() - t0)
        rows.append(nr)
    get = gen.rvq_expert if act == "rvq3" else gen.routed_expert
    for e in order:
        ex = get(cfg, int(e))   # untimed
        toks = sp[offsets[e]:offsets[e + 1]][:256] // cfg.k
        t0 = time.perf_counter()
        ffn(ex, x64[toks])
        secs.append(time.perf_counter() - t0)
        rows.append(len(toks))
        if sum(secs) > budget_s / 2 and len(secs) >= 2:
            break
    n = np.array(rows, dtype=np.float64)
    t = np.array(secs)
    if np.ptp(n) > 0:
        b, a = np.polyfit(n, t, 1)
        a = max(a, 0.0)
    else:
        a, b = 0.0, float(t.sum() / n.sum())
    t_routed = float(a * touched.size + b * counts[touched].sum())
    shared = gen.shared_bank(cfg)
    n_sh = min(T, 64)
    t0 = time.perf_counter()
    orc.shared_ffn(shared, x64[:n_sh])
    t_shared = (time.perf_counter() - t0) * T / n_sh
    n_c = min(T, 512)
    y = np.zeros((n_c * cfg.k, cfg.d))
    t0 = time.perf_counter()
    orc.combine(y, np.arange(n_c * cfg.k, dtype=np.int32), w[:n_c], np.zeros((n_c, cfg.d)))
    t_comb = (time.perf_counter() - t0) * T / n_c
    total = t_route + t_routed + t_shared + t_comb
    return dict(value=T / total, unit="tokens/s", cores=orc.threads(), kind="oracle",
                sample=f"{cfg.name} ({act} activations): fp64 router + permute on all {T} tokens "
                       f"({t_route:.1f} s, "
                       f"measured); routed experts: {len(secs) - 2} of the {touched.size} "
                       f"touched experts (seeded random), each on up to 256 of its pairs, and "
                       f"one on 1 and on 256 rows, "
                       f"{float(t.sum()):.1f} s, fitted as {a * 1e3:.1f} ms + "
                       f"{b * 1e3:.2f} ms per pair and summed over all touched experts "
                       f"({t_routed:.1f} s); shared experts on {n_sh} tokens and combine on "
                       f"{n_c}, scaled by token count ({t_shared:.1f} s, {t_comb:.2f} s); "
                       f"estimated whole-layer oracle time {total:.1f} s")


# --------------------------------------------------------------- GPU timing
def run_cache_workload(name, args, weights):
    """Decode at batch 1 through the expert cache: the routed bank in pinned
    host memory, CACHE_SLOTS expert slots in HBM.  A step is one
    k3moe_cache_layer call on a fresh token (route, ids to the host, misses
    copied on the copy stream while the shared experts run, routed experts on
    the slots, combine); its outputs are the resident layer's bits."""
    import torch

    import gen
    import gen.device
    import mxfp4_routed_expert_gemv_amd as k3
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer

    cfg = gen.get(name[:-len(HOST)])
    K = args.steps if args.steps is not None else 50
    W = args.warmup if args.warmup is not None else 5
    log(f"workload {name}: T={cfg.T}, {CACHE_SLOTS} slots, {K} steps after {W}")
    if "host_bank" not in weights.extra:
        log("  pinning a host copy of the routed bank")
        host = {}
        for n, t in weights.routed.items():
            host[n] = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            host[n].copy_(t)
        weights.extra["host_bank"] = host
    host = weights.extra["host_bank"]
    per_expert = sum(t[0].numel() for t in host.values())
    slot = {n: torch.empty((CACHE_SLOTS,) + tuple(t.shape[1:]), dtype=t.dtype, device="cuda")
            for n, t in host.items()}
    # the plain host-to-device rate of this link: one 1 GiB pinned copy
    probe = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    src = host["w13"].view(-1)[:1 << 30]
    probe.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    probe.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    pcie_gbs = (1 << 30) / (time.perf_counter() - t0) / 1e9
    del probe
    log(f"  pinned host-to-device copy: {pcie_gbs:.1f} GB/s")
    copy_stream = torch.cuda.Stream()
    runs = {}
    for routing in ("uniform", "zipf1.1"):
        rc = cfg if routing == "uniform" else gen.get("prefill_16384_zipf").with_tokens(1)
        w_router = (weights.w_router if routing == "uniform"
                    else gen.device._to_dev_bf16(gen.router(rc), "cuda"))
        layer = MoELayer(w_router, weights.routed, weights.shared, cfg.k,
                         out_dtype=torch.bfloat16)
        hb = k3.make_bank(k3.FMT_MXFP4, cfg.E, cfg.d, cfg.f, host["w13"], host["w13_scale"],
                          host["w2"], host["w2_scale"])
        db = k3.make_bank(k3.FMT_MXFP4, CACHE_SLOTS, cfg.d, cfg.f, slot["w13"],
                          slot["w13_scale"], slot["w2"], slot["w2_scale"])
        cache = k3.ExpertCache(layer.shape(1), hb, db)
        xs = gen.device.activations(rc.with_tokens(K + W))
        shape = layer.shape(1, xs.dtype)
        ws = torch.empty(cache.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        out = torch.empty((1, cfg.d), dtype=torch.bfloat16, device="cuda")
        for i in range(W):
            cache.layer(shape, layer.weights, xs[i:i + 1], out, workspace=ws,
                        copy_stream=copy_stream)
        torch.cuda.synchronize()
        st0 = cache.stats()
        t0 = time.perf_counter()
        for i in range(W, W + K):
            cache.layer(shape, layer.weights, xs[i:i + 1], out, workspace=ws,
                        copy_stream=copy_stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st1 = cache.stats()
        d = {n: st1[n] - st0[n] for n in st1}
        # the resident layer on the same tokens, for the cost of the cache
        t0 = time.perf_counter()
        for i in range(W, W + K):
            layer(xs[i:i + 1], out=out)
        torch.cuda.synchronize()
        resident = (time.perf_counter() - t0) / K
        runs[routing] = {
            "tokens_per_s": K / wall, "ms_per_step": wall / K * 1e3,
            "hit_rate": d["hits"] / max(d["lookups"], 1),
            "misses_per_step": d["misses"] / K, "evictions_per_step": d["evictions"] / K,
            "h2d_bytes_per_step": d["bytes_copied"] / K,
            "h2d_gbs": d["bytes_copied"] / wall / 1e9,
            "resident_layer_ms_per_step_wall": resident * 1e3,
        }
        log(f"  {routing}: {wall / K * 1e3:.2f} ms/step, hit rate "
            f"{runs[routing]['hit_rate']:.3f}, {runs[routing]['h2d_gbs']:.1f} GB/s over PCIe "
            f"(resident layer {resident * 1e3:.3f} ms/step)")
        cache.close()
        del xs, ws
    u = runs["uniform"]
    result = {
        "metric": METRIC,
        "value": u["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": u["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "tokens_per_step": cfg.T, "d": cfg.d, "f": cfg.f,
                   "experts": cfg.E, "top_k": cfg.k, "shared_experts": cfg.n_shared,
                   "weights": "routed MXFP4 in pinned host memory, shared and router bf16 in HBM",
                   "cache_slots": CACHE_SLOTS, "expert_bytes": per_expert,
                   "parallelism": "single GPU"},
        # the step is bound by the expert copies over the host link, not by a kernel
        "roofline": {"bound": "pcie", "achieved": u["h2d_gbs"], "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": u["h2d_gbs"] / PCIE_PEAK_GBS, "traffic": None,
                     "kernel": "hipMemcpyAsync host-to-device (expert misses)",
                     "measured_copy_gbs": pcie_gbs},
        "routing": runs,
    }
    del slot
    torch.cuda.empty_cache()
    return result


def run_workload(name, args, weights):
    import torch

    import gen
    import gen.device
    from mxfp4_routed_expert_gemv_amd import DIAG_COUNT, OP_EXPERT_FFN, OP_LAYER, k3moe_expert_ffn, lib
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer

    qact = name.endswith(QACT)
    rvq = name.endswith(RVQ)
    cfg = gen.get(name[:-len(QACT)] if qact else name[:-len(RVQ)] if rvq else name)
    big = cfg.T >= 1024
    K = args.steps if args.steps is not None else (10 if big else 50)
    W = args.warmup if args.warmup is not None else (3 if big else 5)
    log(f"workload {cfg.name}: T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}, "
        f"{K} steps after {W}")
    w_router = weights.w_router
    if cfg.zipf_s is not None:
        w_router = gen.device._to_dev_bf16(gen.router(cfg), "cuda")
    if rvq and "rvq" not in weights.extra:
        log("building the RVQ3 bank")
        weights.extra["rvq"] = gen.device.build_rvq(gen.get("decode_b1"))
    layer = MoELayer(w_router, weights.extra["rvq"] if rvq else weights.routed, weights.shared,
                     cfg.k, out_dtype=torch.bfloat16, act="mxfp4" if qact else "exact")
    T = cfg.T
    # decode: K + W distinct batches (fresh expert sets every step); prefill
    # batches touch every expert anyway, so two batches alternate
    nb = 2 if big else K + W
    xs = gen.device.activations(cfg.with_tokens(nb * T))
    batches = [xs[(i % nb) * T:(i % nb + 1) * T] for i in range(K + W)]
    shape = layer.shape(T, xs.dtype)
    ws = layer.workspace(shape, OP_LAYER)
    out = torch.empty((T, cfg.d), dtype=torch.bfloat16, device="cuda")
    diag = torch.zeros(DIAG_COUNT, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(W):
        layer(batches[i], out=out, diag=diag, workspace=ws)
    torch.cuda.synchronize()

    # ------------------------------------------------------ timed region
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
    log(f"  layer: {ms_per_step * 1e3:.1f} us/step (wall {wall / K * 1e6:.1f} us/step; "
        f"p10 {pct(0.1) * 1e3:.1f} p50 {pct(0.5) * 1e3:.1f} p90 {pct(0.9) * 1e3:.1f} us)")

    # -------------------------------------- dominant kernel, HIP events
    # The routed gate/up alone: route + permute of the K batches are prepared
    # first, then the K gate/up calls run back to back between two events on
    # the stream they are launched on.
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
    gu_avg_s = a.elapsed_time(b) / K / 1e3
    per_expert_gu = (2 * cfg.f * cfg.d * 3 // 8 + RVQ_CODEBOOK_BYTES if rvq
                     else lib.k3moe_mxfp4_bytes(2 * cfg.f, cfg.d))
    gu_bytes = sum(touched) / len(touched) * per_expert_gu
    gu_gbs = gu_bytes / gu_avg_s / 1e9
    gu_flops = 2.0 * T * cfg.k * 2 * cfg.f * cfg.d      # useful gate/up FLOPs per launch
    gu_tflops = gu_flops / gu_avg_s / 1e12
    # the routed experts take the scaled matrix-core instruction at any batch
    # size for bf16 activations and d, f multiples of 512
    routed_scaled = cfg.x_dtype == "bf16" and cfg.d % 512 == 0 and cfg.f % 512 == 0 and not rvq
    # the bound of the gate/up kernel: useful FLOPs per weight byte against the
    # ridge of the instruction it issues (fp8 matrix peak / HBM peak)
    mfma_bound = routed_scaled and gu_flops / gu_bytes >= FP8_MFMA_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS
    log(f"  gate/up: {gu_avg_s * 1e6:.1f} us avg, {gu_bytes / 1e6:.1f} MB/launch, "
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
    per_expert = (3 * cfg.f * cfg.d * 3 // 8 + 2 * RVQ_CODEBOOK_BYTES if rvq else
                  lib.k3moe_mxfp4_bytes(2 * cfg.f, cfg.d) + lib.k3moe_mxfp4_bytes(cfg.d, cfg.f))
    ffn_bytes = sum(touched) / len(touched) * per_expert
    ffn_tflops = ffn_flops / (ffn_ms / 1e3) / 1e12
    ffn_gbs = ffn_bytes / (ffn_ms / 1e3) / 1e9
    log(f"  routed FFN: {ffn_ms * 1e3:.1f} us avg, {ffn_gbs:.0f} GB/s, "
        f"{ffn_tflops:.1f} TFLOP/s useful")

    # whole-layer algorithmic bytes (MXFP4 experts touched + shared + router + x, out)
    layer_bytes = (ffn_bytes + cfg.n_shared * 3 * cfg.f_shared * cfg.d * 2
                   + cfg.E * cfg.d * 2 + 2 * T * cfg.d * 2)
    traffic = stored_traffic(name)
    if qact:
        # MXFP4 x MXFP4 in one pass: the matrix-core target is the FP4 peak
        roof = {"bound": "mfma", "achieved": gu_tflops, "peak": MXFP4_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": gu_tflops / MXFP4_MFMA_PEAK_TFLOPS,
                "traffic": traffic, "kernel": "mx_gemm_scaled (gate/up, MXFP4 activations)",
                "flops_per_launch": gu_flops, "avg_launch_us": gu_avg_s * 1e6,
                "bytes_per_launch": gu_bytes, "mxfp4_gbs": gu_gbs,
                "frac_of_hbm_peak": gu_gbs / HBM_PEAK_GBS}
    elif mfma_bound:
        roof = {"bound": "mfma", "achieved": gu_tflops, "peak": FP8_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": gu_tflops / FP8_MFMA_PEAK_TFLOPS, "traffic": traffic,
                "kernel": "mx_gemm_scaled (gate/up)", "flops_per_launch": gu_flops,
                "avg_launch_us": gu_avg_s * 1e6, "issued_tflops": gu_tflops * X_PASSES,
                "frac_of_mxfp4_peak": gu_tflops / MXFP4_MFMA_PEAK_TFLOPS,
                "bytes_per_launch": gu_bytes, "mxfp4_gbs": gu_gbs}
    else:
        roof = {"bound": "hbm", "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gu_gbs / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": ("rvq_partial_staged + rvq_reduce_gateup" if rvq
                           else "gateup_1tok" if T == 1 and routed_scaled
                           else "mx_gemm_scaled (gate/up)" if routed_scaled
                           else "gateup_persistent"),
                "bytes_per_launch": gu_bytes, "avg_launch_us": gu_avg_s * 1e6,
                "useful_tflops": gu_tflops}
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
        "config": {"workload": name, "tokens_per_step": T, "d": cfg.d, "f": cfg.f,
                   "experts": cfg.E, "top_k": cfg.k, "shared_experts": cfg.n_shared,
                   "weights": "routed MXFP4 (E2M1 + E8M0/32), shared and router bf16",
                   "routed_activations": "MXFP4 (quantised)" if qact else "exact",
                   "routed_format": "RVQ3 (3.00 bits/weight)" if rvq else "MXFP4",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "layer_hbm_gbs": layer_bytes / (ms_per_step / 1e3) / 1e9,
        "layer_bytes_per_step": layer_bytes,
        "experts_touched_per_step": sum(touched) / len(touched),
        "rechecked_tokens": int(diag[0].item()),
        "routed_ffn": {"avg_us": ffn_ms * 1e3, "mxfp4_bytes": ffn_bytes, "mxfp4_gbs": ffn_gbs,
                       "frac_of_hbm_peak": ffn_gbs / HBM_PEAK_GBS, "useful_tflops": ffn_tflops,
                       "frac_of_fp8_peak": ffn_tflops / FP8_MFMA_PEAK_TFLOPS,
                       "frac_of_mxfp4_peak": ffn_tflops / MXFP4_MFMA_PEAK_TFLOPS},
    }
    del xs, batches, prepared, h, y, ws, fws
    torch.cuda.empty_cache()
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50 for decode workloads, 10 for prefill)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="warm-up steps (default 5 for decode workloads, 3 for prefill)")
    ap.add_argument("--workload", default="all",
                    help="all (default: " + ", ".join(WORKLOADS) + "; the first is the "
                         "headline), or one of them")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time per workload for the CPU baseline")
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
    names = WORKLOADS if args.workload == "all" else [args.workload]
    for n in names:
        if n not in WORKLOADS:
            sys.exit(f"unknown workload {n}")

    import torch

    import gen
    import gen.device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    weights = gen.device.build(gen.get("decode_b1"), routed_on_device=True)
    torch.cuda.synchronize()
    log("weights resident")
    results = {n: (run_cache_workload if n.endswith(HOST) else run_workload)(n, args, weights)
               for n in names}
    weights.extra.pop("host_bank", None)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calib_copy_mib} MiB done")
    if not args.no_cpu_baseline:
        for n in names:
            if n.endswith(HOST):
                # the cache changes where the weights live, not what is computed:
                # the oracle's decode is the same
                base = n[:-len(HOST)]
                results[n]["cpu_baseline"] = (results[base]["cpu_baseline"] if base in results
                                              else cpu_baseline_one_token(gen.get(base),
                                                                          args.cpu_seconds))
                continue
            log(f"timing the CPU oracle on {n}")
            qact, rvq = n.endswith(QACT), n.endswith(RVQ)
            cfg = gen.get(n[:-len(QACT)] if qact else n[:-len(RVQ)] if rvq else n)
            act = "mxfp4" if qact else "rvq3" if rvq else "exact"
            results[n]["cpu_baseline"] = (cpu_baseline_one_token(cfg, args.cpu_seconds, act)
                                          if cfg.T == 1 else
                                          cpu_baseline_batch(cfg, args.cpu_seconds, act))
    line = dict(results[names[0]])
    if len(names) > 1:
        line["workloads"] = results
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
