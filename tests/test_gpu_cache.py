"""GPU tests of the expert cache (k3moe_cache_*): host-resident routed experts
streamed over PCIe into an HBM cache of a few expert slots.

The pages' contract for such a cache is that its size is a dial: the same
weights, the same top-k and the same outputs at every budget (kimi-k3-in-c
review page, memory ladder).  So every step here must equal k3moe_layer on
the resident bank bit for bit, for caches from k slots to all E experts, with
misses copied on a separate stream; the counters must add up; a prefetch of
the experts a step will use must turn all of its lookups into prefetch
hits."""
import numpy as np
import pytest
import torch

import gen
import gen.device
from gpu_util import log, require_gpu, to_np

pytestmark = pytest.mark.gpu

MED = gen.configs.LayerConfig(name="medium", T=1, d=512, f=512, E=32, k=8, n_shared=2,
                              f_shared=256, x_dtype="bf16", out_dtype="f32", scale_lo=-8,
                              scale_hi=0)


def _pinned_copy(t: torch.Tensor) -> torch.Tensor:
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def _setup(wl, cfg, slots, out_dtype=torch.float32):
    import mxfp4_routed_expert_gemv_amd as k3
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    L = MoELayer(wl.w_router, wl.routed, wl.shared, cfg.k, out_dtype=out_dtype)
    host = {n: _pinned_copy(t) for n, t in wl.routed.items()}
    dev = {n: torch.empty((slots,) + tuple(t.shape[1:]), dtype=t.dtype, device="cuda")
           for n, t in wl.routed.items()}
    hb = k3.make_bank(k3.FMT_MXFP4, cfg.E, cfg.d, cfg.f, host["w13"], host["w13_scale"],
                      host["w2"], host["w2_scale"])
    db = k3.make_bank(k3.FMT_MXFP4, slots, cfg.d, cfg.f, dev["w13"], dev["w13_scale"],
                      dev["w2"], dev["w2_scale"])
    cache = k3.ExpertCache(L.shape(1), hb, db)
    cache.keep = (host, dev)      # the banks must outlive the cache
    return L, cache, (host, dev)


def _step(L, cache, x, out_dtype, copy_stream):
    s = L.shape(x.shape[0], x.dtype, out_dtype)
    ws = torch.empty(max(cache.workspace_bytes(s), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((x.shape[0], L.d), dtype=out_dtype, device="cuda")
    cache.layer(s, L.weights, x, out, workspace=ws, copy_stream=copy_stream)
    return out


@pytest.mark.parametrize("T,slots", [(1, 8), (1, 12), (1, 32), (3, 24), (3, 28), (3, 32)])
def test_cache_matches_resident_layer(T, slots):
    require_gpu()
    cfg = MED.with_tokens(24 * T)
    wl = gen.device.build(cfg)
    L, cache, keep = _setup(wl, cfg, slots)
    cs = torch.cuda.Stream()
    log(f"case medium, {slots} slots, {T} token(s) a step")
    per_expert = sum(t[0].numel() for t in keep[0].values())
    for i in range(24):
        x = wl.x[i * T:(i + 1) * T].contiguous()
        want = L(x)
        got = _step(L, cache, x, torch.float32, cs)
        torch.cuda.synchronize()
        assert torch.equal(got, want), i
    st = cache.stats()
    log(f"  stats {st}")
    assert st["hits"] + st["misses"] == st["lookups"]
    assert st["bytes_copied"] == st["misses"] * per_expert
    assert st["prefetched"] == 0 and st["prefetch_hits"] == 0
    if slots == cfg.E:
        assert st["evictions"] == 0 and st["misses"] <= cfg.E
    else:
        assert st["evictions"] > 0


def test_cache_prefetch_turns_misses_into_hits():
    """Prefetching the experts a step routes to (a perfect lookahead) makes
    every lookup of that step a hit, and the output stays the same."""
    require_gpu()
    cfg = MED.with_tokens(6)
    wl = gen.device.build(cfg)
    L, cache, _ = _setup(wl, cfg, 16)
    cs = torch.cuda.Stream()
    fetched = 0
    for i in range(6):
        x = wl.x[i:i + 1].contiguous()
        idx, _, _ = L.route(x)
        ids = np.unique(to_np(idx))
        before = cache.stats()
        cache.prefetch(ids, copy_stream=cs)
        got = _step(L, cache, x, torch.float32, cs)
        want = L(x)
        torch.cuda.synchronize()
        assert torch.equal(got, want), i
        after = cache.stats()
        delta = {n: after[n] - before[n] for n in after}
        assert delta["misses"] == 0 and delta["hits"] == len(ids) == delta["lookups"]
        assert delta["prefetch_hits"] == delta["prefetched"]
        fetched += delta["prefetched"]
    assert fetched > 0


def test_cache_too_many_experts_for_the_slots():
    """A batch routing to more distinct experts than there are slots is
    refused (after routing, before anything else)."""
    require_gpu()
    import mxfp4_routed_expert_gemv_amd as k3
    cfg = MED.with_tokens(8)
    wl = gen.device.build(cfg)
    L, cache, _ = _setup(wl, cfg, 8)
    with pytest.raises(k3.K3moeError, match="ESHAPE"):
        _step(L, cache, wl.x, torch.float32, None)
        torch.cuda.synchronize()


def test_cache_full_size_decode(big):
    """d = 7168, 896 experts top-16: 12 decode steps through a 64-slot cache
    (1.5 GB of HBM for the routed experts instead of 21 GB), the same bits as
    the resident layer at every step."""
    cfg = gen.get("decode_b1")
    log("pinning the full-size routed bank in host memory")
    L, cache, _ = _setup(big, cfg, 64, torch.bfloat16)
    cs = torch.cuda.Stream()
    xs = gen.device.activations(cfg.with_tokens(12))
    for i in range(12):
        x = xs[i:i + 1].contiguous()
        got = _step(L, cache, x, torch.bfloat16, cs)
        want = L(x)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), i
    log(f"  stats {cache.stats()}")
