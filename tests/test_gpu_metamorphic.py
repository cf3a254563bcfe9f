"""Metamorphic identities of the routed expert FFN on the GPU.

Scaling an MXFP4 block scale by one step multiplies every weight of the block
by 2 exactly, and flipping a code's sign bit negates the weight exactly (E2M1
and E8M0 as OCP MX v1.0 defines them).  Binary floating point with
round-to-nearest-even commutes with both (no rounding is affected, nothing
overflows at these sizes), so whatever order the kernels sum in:
  - +1 on every w2 scale byte doubles y exactly;
  - flipping the sign bit of every w2 code negates y exactly;
  - +1 on every up-row scale byte doubles u, hence h = silu(g) u and y,
    exactly.
The oracle obeys the same identities (its pins); here every kernel family
the shape selects is held to them: the one-token scaled kernels, the grouped
scaled GEMMs (their h in E4M3 passes, whose codes stay and whose scales move
by one), and the vector-ALU GEMVs for fp32 x or other shapes (h in fp32).

One exception, measured on gfx950: the scaled matrix-core instruction's
internal sum does not round symmetrically under negation.  Negating every
weight leaves 5-10% of the outputs off their negated value, by up to about
1.3e-6 of the output RMS (the rounding of the partial sums, which can be far
larger than a small output, sets the size).  So on the matrix-core paths the
sign identity is held to |y(-W) + y(W)| <= 2^-14 RMS(y), and bit for bit on
the vector-ALU paths.  Scaling by a power of two stays exact on every path.
"""
import numpy as np
import pytest
import torch

import gen
import gen.device
from gpu_util import decode_scaled_h, log, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _cfg(name, T, d, f, x_dtype, E=32, k=8):
    return gen.configs.LayerConfig(name=name, T=T, d=d, f=f, E=E, k=k, n_shared=0, f_shared=0,
                                   x_dtype=x_dtype, out_dtype="f32", scale_lo=-8, scale_hi=0)


CASES = [
    # (config, h is in the scaled E4M3-pass form)
    (_cfg("tiny_gemv_T4", 4, 256, 128, "f32", E=16, k=4), False),
    (_cfg("scaled_one_token", 1, 512, 512, "bf16"), True),
    (_cfg("scaled_one_token_d3584", 1, 3584, 512, "bf16"), True),
    (_cfg("scaled_grouped_T5", 5, 512, 512, "bf16"), True),
    (_cfg("scaled_grouped_T40", 40, 512, 512, "bf16"), True),
    (_cfg("bf16_gemv_T1", 1, 768, 160, "bf16"), False),
    (_cfg("bf16_gemv_T5", 5, 768, 160, "bf16"), False),
]


@pytest.mark.parametrize("cfg,scaled", CASES, ids=[c.name for c, _ in CASES])
def test_scale_and_sign_identities(cfg, scaled):
    require_gpu()
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    log(f"case {cfg.name}")
    wl = gen.device.build(cfg)
    L = MoELayer(wl.w_router, wl.routed, {}, cfg.k, out_dtype=torch.float32)
    idx, _, _ = L.route(wl.x)
    _, offsets, sp, _ = L.permute(idx)
    P = cfg.T * cfg.k

    def run(routed):
        Lm = MoELayer(wl.w_router, routed, {}, cfg.k, out_dtype=torch.float32)
        h = Lm.expert_gateup(wl.x, offsets, sp).clone()
        y = Lm.expert_ffn(wl.x, offsets, sp).clone()
        torch.cuda.synchronize()
        return h, y

    def h_values(h):
        if scaled:
            return decode_scaled_h(to_np(h).reshape(-1), P, cfg.f)
        return to_np(h).astype(np.float64)

    h0, y0 = run(wl.routed)
    assert torch.all(torch.isfinite(y0))
    # +1 on every down scale byte: y doubles
    _, y1 = run(dict(wl.routed, w2_scale=wl.routed["w2_scale"] + 1))
    assert torch.equal(y1, 2 * y0), "w2 scale + 1"
    # sign bit of every down code flipped: y negates
    _, y2 = run(dict(wl.routed, w2=wl.routed["w2"] ^ 0x88))
    dev = (y2 + y0).abs()
    y0n = to_np(y0).astype(np.float64)
    rms = float(np.sqrt(np.mean(y0n ** 2)))
    ulps = to_np(dev).astype(np.float64) / np.spacing(np.abs(y0n).astype(np.float32))
    log(f"  sign flip: max|y(-W) + y(W)| = {float(dev.max()):.3e} "
        f"({float(dev.max()) / rms:.2e} RMS, {float(ulps.max()):.0f} ulp), "
        f"{int((dev > 0).sum())} of {dev.numel()} outputs off")
    if scaled:
        assert float(dev.max()) <= 2.0 ** -14 * rms, "w2 sign flip"
    else:
        assert torch.equal(y2, -y0), "w2 sign flip"
    # +1 on the up rows' scale bytes: h and y double
    s = wl.routed["w13_scale"].clone()
    s[:, cfg.f:, :] += 1
    h3, y3 = run(dict(wl.routed, w13_scale=s))
    assert torch.equal(y3, 2 * y0), "up scale + 1 (y)"
    assert np.array_equal(h_values(h3), 2 * h_values(h0)), "up scale + 1 (h)"
    if scaled:
        # the codes of h stay; every pass's scale byte moves up by one
        st0 = to_np(h0).reshape(-1).view(np.uint8)[:P * (cfg.f // 128) * 400]
        st3 = to_np(h3).reshape(-1).view(np.uint8)[:P * (cfg.f // 128) * 400]
        st0 = st0.reshape(P, cfg.f // 128, 400).astype(np.int64)
        st3 = st3.reshape(P, cfg.f // 128, 400).astype(np.int64)
        assert np.array_equal(st3[:, :, :384], st0[:, :, :384])
        assert np.array_equal(st3[:, :, 384:396], st0[:, :, 384:396] + 1)
