"""GPU parity of the quantised-activation mode (k3moe_shape.act = MXFP4): x
before gate/up and h before down are quantised to MXFP4 (OCP MX v1.0), so the
routed experts' products are MXFP4 x MXFP4 in one pass.

What is fixed and how it is compared:
  - x's codes and scales: a pure function of the bf16 inputs; equal to the
    oracle's quantiser byte for byte;
  - h's codes: the kernel decides them on its fp32 h, the oracle on its fp64
    h.  The two agree except where the oracle's value lies within
    ETA = 2^-10 (in units of the block's scale) of a rounding midpoint, or
    the block's largest magnitude lies within a relative ETA of a power of
    two (the scale itself could move).  Every code that differs must be such
    an element, and few may differ;
  - y (and the layer's output): the oracle's y from its own quantised h,
    within 2e-3 RMS plus, per output, the sum over the row's near elements of
    |w| 2^(E + 2) (more than any one code or scale step can move an element).
The mode's distance from the exact layer is logged, not bounded: it is an
approximation by design.
"""
import numpy as np
import pytest
import torch

import gen
import gen.device
import oracle
from gpu_util import BAR, log, oracle_expert, require_gpu, rms, to_np

pytestmark = pytest.mark.gpu

ETA = 2.0 ** -10
MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _np_decode(codes, scales):
    import oracle_pins
    return oracle_pins.np_decode(codes, scales)


def decode_q4_rows(buf: np.ndarray, rows: int, n: int):
    """Records of rows x (n / 128) stages of 80 bytes -> (codes [rows][n/2],
    scales [rows][n/32], values [rows][n])."""
    flat = np.ascontiguousarray(buf).reshape(-1).view(np.uint8)
    st = flat[:rows * (n // 128) * 80].reshape(rows, n // 128, 80)
    codes = np.ascontiguousarray(st[:, :, :64]).reshape(rows, n // 2)
    scales = np.ascontiguousarray(st[:, :, 64:68]).reshape(rows, n // 32)
    return codes, scales, _np_decode(codes, scales)


def near_mask(h: np.ndarray):
    """Elements of h (fp64, rows of blocks of 32) whose MXFP4 code could be
    decided either way by a value within ETA of it: near a rounding midpoint,
    or in a block whose largest magnitude is near a power of two; and the
    exponent E of each element's block."""
    hb = h.reshape(-1, 32)
    X = np.max(np.abs(hb), axis=1)
    with np.errstate(divide="ignore"):
        lx = np.log2(np.where(X > 0, X, 1.0))
    E = np.floor(lx) - 2
    a = np.abs(hb) / 2.0 ** E[:, None]
    near = np.min(np.abs(a[..., None] - MIDS), axis=-1) <= ETA
    frac = X / 2.0 ** np.floor(lx)
    block_near = (X > 0) & ((frac <= 1 + ETA) | (frac >= 2 * (1 - ETA)))
    near |= block_near[:, None]
    return near.reshape(h.shape), np.repeat(E, 32).reshape(h.shape)


def expected_y(orc, expert, x64):
    """Oracle y with quantised activations, the oracle's unquantised h, its
    quantised h, and the per-output allowance for h codes decided either
    way."""
    codes, scales = orc.quantize_mxfp4(x64)
    xq = orc.mxfp4_decode(codes, scales)
    _, h = orc.mxfp4_ffn(expert, xq, want_h=True)          # the qact FFN's h before quantising
    y, hq = orc.mxfp4_ffn_qact(expert, x64, want_h=True)
    near, E = near_mask(h)
    W2 = np.abs(orc.mxfp4_decode(expert["w2"], expert["w2_scale"]))
    allow = (np.where(near, 2.0 ** (E + 2), 0.0)) @ W2.T
    return y, h, hq, near, allow


def check_y(got, want, allow, name):
    scale = rms(want)
    err = np.abs(got.astype(np.float64) - want)
    over = err - BAR * scale - allow
    log(f"  {name}: max|err| {err.max():.3e} (RMS {scale:.3e}); rows with an allowance "
        f"{int(np.sum(np.any(allow > 0, axis=1)))} of {want.shape[0]}")
    assert np.all(np.isfinite(got))
    assert np.all(over <= 0), f"{name}: {int(np.sum(over > 0))} outputs beyond the bar"


def check_h(h_gpu_vals, hq, near, name):
    diff = h_gpu_vals != hq
    n = int(diff.sum())
    log(f"  {name}: {n} of {diff.size} h codes differ, {int(near.sum())} near a boundary")
    assert np.all(near[diff]), f"{name}: {int(np.sum(diff & ~near))} codes differ away from a boundary"
    assert n <= max(8, diff.size // 10000)


MED = gen.configs.LayerConfig(name="medium", T=40, d=512, f=512, E=32, k=8, n_shared=2,
                              f_shared=256, x_dtype="bf16", out_dtype="f32", scale_lo=-8,
                              scale_hi=0)


def _layer(wl, cfg, out_dtype=torch.float32, w_router=None):
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    return MoELayer(w_router if w_router is not None else wl.w_router, wl.routed, wl.shared,
                    cfg.k, out_dtype=out_dtype, act="mxfp4")


@pytest.mark.parametrize("T", [1, 5, 40, 200])
def test_qact_medium(orc, T):
    """d = 512 layer: x codes byte for byte, h codes, y and the layer output."""
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import OP_EXPERT_GATEUP, k3moe_expert_gateup
    cfg = MED.with_tokens(T)
    log(f"case {cfg.name} mxfp4 activations")
    wl = gen.device.build(cfg)
    L = _layer(wl, cfg)
    r = L.staged(wl.x)
    out = L(wl.x)
    s = L.shape(T, wl.x.dtype)
    ws = L.workspace(s, OP_EXPERT_GATEUP)
    P = T * cfg.k
    h = torch.empty((P, cfg.f), dtype=torch.float32, device="cuda")
    k3moe_expert_gateup(s, L.routed_bank, wl.x, r["offsets"], r["sorted_pair"], h, ws, None)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])
    x_host = gen.x(cfg)
    x64 = oracle.to_f64(x_host)
    # x: exact decisions, byte for byte
    gc, gs, _ = decode_q4_rows(to_np(ws), T, cfg.d)
    oc, osc = orc.quantize_mxfp4(x64)
    assert np.array_equal(gc, oc) and np.array_equal(gs, osc), "x codes or scales"
    # routing as in the exact layer
    ref = orc.layer(x_host, gen.router(cfg), oracle_expert(cfg), gen.shared_bank(cfg), cfg.k,
                    cfg.E, act="mxfp4")
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    offs, sp = ref["offsets"], ref["sorted_pair"]
    _, _, h_gpu = decode_q4_rows(to_np(h), P, cfg.f)
    y_gpu = to_np(r["y_perm"])
    allow_y = np.zeros((P, cfg.d))
    for e in np.nonzero(ref["counts"])[0]:
        lo, hi = offs[e], offs[e + 1]
        y_or, _, hq, near, allow = expected_y(orc, gen.routed_expert(cfg, int(e)),
                                              x64[sp[lo:hi] // cfg.k])
        check_h(h_gpu[lo:hi], hq, near, f"h expert {e}")
        assert np.array_equal(y_or, ref["y_perm"][lo:hi])
        allow_y[lo:hi] = allow
    check_y(y_gpu, ref["y_perm"], allow_y, "y_perm")
    # the layer output: shared + sum of w y, allowance weighted the same way
    pp = ref["pair_pos"]
    allow_out = np.zeros((T, cfg.d))
    for t in range(T):
        for sl in range(cfg.k):
            allow_out[t] += abs(ref["w"][t, sl]) * allow_y[pp[t * cfg.k + sl]]
    check_y(to_np(out), ref["out"], allow_out, "out")
    # the distance of the quantised layer from the exact one (reported only)
    exact = orc.layer(x_host, gen.router(cfg), oracle_expert(cfg), gen.shared_bank(cfg), cfg.k,
                      cfg.E)
    rel = rms(ref["y_perm"] - exact["y_perm"]) / rms(exact["y_perm"])
    log(f"  MXFP4 activations vs exact: RMS(y difference) / RMS(y) = {rel:.3e}")


def test_qact_batch_composition():
    """A token's routed outputs are the same bits alone and inside batches of
    5, 40 and 200 (the grouped GEMMs at every batch size)."""
    require_gpu()
    cfg = MED.with_tokens(200)
    wl = gen.device.build(cfg)
    L = _layer(wl, cfg)
    full = L.staged(wl.x)
    torch.cuda.synchronize()

    def rows(r, t):
        pp = to_np(r["pair_pos"])
        return to_np(r["y_perm"])[pp[t * cfg.k:(t + 1) * cfg.k]]
    for n in (1, 5, 40):
        part = L.staged(wl.x[:n].contiguous())
        torch.cuda.synchronize()
        for t in range(n):
            assert np.array_equal(rows(part, t), rows(full, t)), (n, t)
    out = L(wl.x)
    part = L(wl.x[:40].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(part, out[:40])


def _mtile_rows(cfg):
    ppe = cfg.T * cfg.k / cfg.E * 1.15
    return 16 * max(1, min(6, int((ppe + 15.0) / 16.0)))


@pytest.mark.parametrize("name", ["decode_b64", "prefill_4096", "prefill_16384_zipf"])
def test_qact_full_size(big, orc, name):
    """Full size: x codes of sampled tokens byte for byte; whole m-tiles of
    y (a tail expert, one spanning two m-tiles, the hottest expert's first
    and last) against the oracle's quantised FFN."""
    from mxfp4_routed_expert_gemv_amd import OP_EXPERT_GATEUP, k3moe_expert_gateup
    cfg = gen.get(name)
    x_host = gen.x(cfg)
    wr_host = gen.router(cfg)
    wr = gen.device._to_dev_bf16(wr_host, "cuda") if cfg.zipf_s is not None else big.w_router
    L = _layer(big, cfg, torch.bfloat16, wr)
    x = gen.device.activations(cfg)
    log(f"case {name} mxfp4 activations")
    r = L.staged(x)
    out = L(x)
    s = L.shape(cfg.T, x.dtype)
    ws = L.workspace(s, OP_EXPERT_GATEUP)
    h = torch.empty((cfg.T * cfg.k, cfg.f), dtype=torch.float32, device="cuda")
    k3moe_expert_gateup(s, L.routed_bank, x, r["offsets"], r["sorted_pair"], h, ws, None)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r["out"].view(torch.int16))
    toks = np.unique(np.linspace(0, cfg.T - 1, 16).astype(int))
    gc, gs, _ = decode_q4_rows(to_np(ws), cfg.T, cfg.d)
    oc, osc = orc.quantize_mxfp4(oracle.to_f64(x_host[toks]))
    assert np.array_equal(gc[toks], oc) and np.array_equal(gs[toks], osc), "x codes or scales"
    counts = to_np(r["counts"])
    offs = to_np(r["offsets"])
    sp = to_np(r["sorted_pair"])
    bm = _mtile_rows(cfg)
    live = np.nonzero(counts)[0]
    tail = int(live[np.argmin(counts[live])])
    ranges = [(tail, offs[tail], offs[tail + 1])]
    two = [e for e in live if bm < counts[e] <= 2 * bm]
    if two:
        e2 = int(max(two, key=lambda e: counts[e]))
        ranges.append((e2, offs[e2], offs[e2 + 1]))
    hot = int(np.argmax(counts))
    if counts[hot] > 2 * bm:
        last0 = offs[hot] + (counts[hot] - 1) // bm * bm
        ranges += [(hot, offs[hot], offs[hot] + bm), (hot, last0, offs[hot + 1])]
    y_gpu = to_np(r["y_perm"])
    _, _, h_gpu = decode_q4_rows(to_np(h), cfg.T * cfg.k, cfg.f)
    for e, lo, hi in ranges:
        x64 = oracle.to_f64(x_host[sp[lo:hi] // cfg.k])
        y_or, _, hq, near, allow = expected_y(orc, gen.routed_expert(cfg, e), x64)
        check_h(h_gpu[lo:hi], hq, near, f"h expert {e} rows {lo - offs[e]}..{hi - offs[e]}")
        check_y(y_gpu[lo:hi], y_or, allow, f"y expert {e} rows {lo - offs[e]}..{hi - offs[e]}")
