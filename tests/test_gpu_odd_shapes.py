"""bf16 activations with hidden or intermediate sizes that are not multiples
of 512: the routed experts take the vector-ALU GEMVs (one token, and the
batched persistent kernels), and the layer stays in the GEMV path class at
every batch size, shared experts included.

Checked against the oracle element by element at 1, 5 and 40 tokens, and for
batch composition: a token's output bits are the same alone and inside
batches of 31, 32 and 40 tokens (32 is where the matrix-core class would
begin for a shape that allows it)."""
import numpy as np
import pytest
import torch

import gen
import gen.device
import oracle
from gpu_util import assert_close, k3layer, log, oracle_expert, require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


# d % 512 != 0 and f % 512 != 0; shared experts 128 wide (a width the
# matrix-core shared kernels would take)
ODD = gen.configs.LayerConfig(name="odd_d768_f160", T=40, d=768, f=160, E=32, k=8, n_shared=2,
                              f_shared=256, x_dtype="bf16", out_dtype="f32", scale_lo=-8,
                              scale_hi=0)
# full hidden size with f % 512 != 0: one token takes the fused one-token
# router/shared kernels beside the routed GEMVs
WIDE = gen.configs.LayerConfig(name="odd_d7168_f1056", T=32, d=7168, f=1056, E=32, k=8,
                               n_shared=2, f_shared=2048, x_dtype="bf16", out_dtype="f32",
                               scale_lo=-10, scale_hi=-2)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_odd_shape_parity(orc, T):
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import PATH_GEMV
    cfg = ODD.with_tokens(T)
    log(f"case {cfg.name}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    assert L.path_class(T) == PATH_GEMV
    r = L.staged(wl.x)
    out = L(wl.x)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])
    bank = gen.routed_bank(cfg)
    ref = orc.layer(gen.x(cfg), gen.router(cfg), lambda e: {k: v[e] for k, v in bank.items()},
                    gen.shared_bank(cfg), cfg.k, cfg.E)
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    assert np.array_equal(to_np(r["sorted_pair"]), ref["sorted_pair"])
    assert_close(to_np(r["y_perm"]), ref["y_perm"], "y_perm")
    assert_close(to_np(r["shared_y"]), ref["shared_y"], "shared_y")
    assert_close(to_np(r["out"]), ref["out"], "out")


@pytest.mark.parametrize("base", [ODD, WIDE], ids=["d768_f160", "d7168_f1056"])
def test_odd_shape_batch_composition(orc, base):
    """One path class from 1 to 40 tokens: a token alone equals its row in
    batches of 31, 32 and 40, bit for bit; the 32-token batch also against
    the oracle (values of every token)."""
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import PATH_GEMV
    cfg = base.with_tokens(40)
    log(f"case {cfg.name}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    for n in (1, 31, 32, 40):
        assert L.path_class(n) == PATH_GEMV, n
    full = L(wl.x)
    torch.cuda.synchronize()
    for n in (31, 32):
        part = L(wl.x[:n].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(part, full[:n]), n
    for t in (0, 30, 31, 39):
        one = L(wl.x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[t]), t
    x_host = gen.x(cfg)[:32]
    _, idx, w = orc.route(oracle.to_f64(x_host), gen.router(cfg), cfg.k)
    out_ref, _, _ = orc.token_outputs(x_host, idx, w, oracle_expert(cfg), gen.shared_bank(cfg))
    assert_close(to_np(full[:32]), out_ref, "out (32 tokens)")
