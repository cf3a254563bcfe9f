"""GPU parity of the RVQ3 routed experts (WASTE article page, section
"정확성 검증과 양자화": three 256-entry codebooks per 8-weight vector, 3.00
bits per weight, multiplied through per-token partial-dot tables): the layer
and its stages against the oracle's fp64 FFN on the materialised weights,
element by element; a token's bits alone and inside a batch; dropped ids;
the full-size bank (d 7168, f 2048, 896 experts) at 1 and 64 tokens."""
import numpy as np
import pytest
import torch

import gen
import gen.device
import oracle
from gpu_util import (W_TOL, assert_close, assert_close_bf16, log, require_gpu, sample_tokens,
                      to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _small(T, x_dtype):
    return gen.configs.LayerConfig(name=f"rvq_small_{x_dtype}", T=T, d=256, f=256, E=16, k=4,
                                   n_shared=1, f_shared=128, x_dtype=x_dtype, out_dtype="f32",
                                   scale_lo=-8, scale_hi=0)


def _layer(w_router, routed, shared, k, out_dtype=torch.float32):
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    return MoELayer(w_router, routed, shared, k, out_dtype=out_dtype)


def _rvq_get(cfg):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = gen.rvq_expert(cfg, e)
        return cache[e]
    return get


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 5, 37])
def test_rvq_small_layer(orc, T, x_dtype):
    require_gpu()
    cfg = _small(T, x_dtype)
    log(f"case {cfg.name} T={T}")
    wl = gen.device.build(cfg)
    routed = gen.device.build_rvq(cfg)
    L = _layer(wl.w_router, routed, wl.shared, cfg.k)
    r = L.staged(wl.x)
    out = L(wl.x)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])
    ref = orc.layer(gen.x(cfg), gen.router(cfg), _rvq_get(cfg), gen.shared_bank(cfg), cfg.k,
                    cfg.E, act="rvq3")
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    assert np.max(np.abs(to_np(r["w"]) - ref["w"])) <= W_TOL
    assert_close(to_np(r["y_perm"]), ref["y_perm"], "y_perm")
    assert_close(to_np(r["out"]), ref["out"], "out")
    # the gate/up half: h against the oracle's
    h = L.expert_gateup(wl.x, r["offsets"], r["sorted_pair"])
    torch.cuda.synchronize()
    x64 = oracle.to_f64(gen.x(cfg))
    offs, sp = ref["offsets"], ref["sorted_pair"]
    h_ref = np.zeros((T * cfg.k, cfg.f))
    for e in np.nonzero(ref["counts"])[0]:
        _, he = orc.rvq_ffn(gen.rvq_expert(cfg, int(e)), x64[sp[offs[e]:offs[e + 1]] // cfg.k],
                            want_h=True)
        h_ref[offs[e]:offs[e + 1]] = he
    assert_close(to_np(h), h_ref, "h")


def test_rvq_batch_composition():
    """A token's routed outputs are the same bits alone and in batches."""
    require_gpu()
    cfg = _small(40, "bf16")
    wl = gen.device.build(cfg)
    routed = gen.device.build_rvq(cfg)
    L = _layer(wl.w_router, routed, wl.shared, cfg.k)
    full = L(wl.x)
    torch.cuda.synchronize()
    for n in (1, 7, 31):
        part = L(wl.x[:n].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(part, full[:n]), n
    one = L(wl.x[20:21].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(one[0], full[20])


def test_rvq_dropped_ids():
    """Pairs whose ids the permute drops are skipped by the RVQ kernels; the
    kept pairs' rows equal the oracle's."""
    require_gpu()
    cfg = _small(3, "f32")
    wl = gen.device.build(cfg)
    routed = gen.device.build_rvq(cfg)
    L = _layer(wl.w_router, routed, wl.shared, cfg.k)
    idx = torch.tensor([[0, 3, 5, 7], [2, 2, 9, 40], [15, -1, 1, 0]], dtype=torch.int32,
                       device="cuda")
    counts, offsets, sp, pp = L.permute(idx)
    y = L.expert_ffn(wl.x, offsets, sp)
    torch.cuda.synchronize()
    offs = to_np(offsets)
    spn = to_np(sp)
    x64 = oracle.to_f64(gen.x(cfg))
    yg = to_np(y)
    for e in np.nonzero(to_np(counts))[0]:
        rows = spn[offs[e]:offs[e + 1]] // cfg.k
        want = oracle.default().rvq_ffn(gen.rvq_expert(cfg, int(e)), x64[rows])
        assert_close(yg[offs[e]:offs[e + 1]], want, f"expert {e}")
    assert offs[-1] == 9


@pytest.fixture(scope="module")
def rvq_big(big):
    """The full-size RVQ3 bank (d 7168, f 2048, 896 experts: 14.8 GB of
    indices) beside the MXFP4 one."""
    cfg = gen.get("decode_b1")
    log("building the full-size RVQ3 bank on device")
    bank = gen.device.build_rvq(cfg)
    torch.cuda.synchronize()
    return bank


@pytest.mark.parametrize("T", [1, 64])
def test_rvq_full_size(big, rvq_big, orc, T):
    cfg = gen.get("decode_b64").with_tokens(T)
    log(f"case RVQ3 full size T={T}")
    L = _layer(big.w_router, rvq_big, big.shared, cfg.k, torch.bfloat16)
    x = gen.device.activations(cfg)
    r = L.staged(x)
    out = L(x)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r["out"].view(torch.int16))
    x_host = gen.x(cfg)
    _, idx, w = orc.route(oracle.to_f64(x_host), gen.router(cfg), cfg.k)
    assert np.array_equal(to_np(r["idx"]), idx)
    toks = sample_tokens(T, 4)
    out_ref, sh_ref, y_ref = orc.token_outputs(x_host[toks], idx[toks], w[toks], _rvq_get(cfg),
                                               gen.shared_bank(cfg), act="rvq3")
    pp = to_np(r["pair_pos"])
    y_rows = np.stack([to_np(r["y_perm"])[pp[t * cfg.k:(t + 1) * cfg.k]] for t in toks])
    assert_close(y_rows.reshape(-1, cfg.d), y_ref.reshape(-1, cfg.d), "y_perm (sampled)")
    assert_close_bf16(to_np(out)[toks], out_ref, "out (sampled)")
