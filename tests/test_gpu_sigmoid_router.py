"""GPU parity of the pages' K3 router: selection by sigmoid(l) + bias (the
bias bends only the selection), weights the unbiased sigmoid(l), raw or
renormalised over the chosen (kimi-k3-in-c review page, "KDA/MLA/MoE" table).

  - the router fixture (after the README's fixtures section: the bias changes
    the chosen pair in five of six rows) through real router weights: one-hot
    tokens make the logits equal the fixture's values exactly;
  - whole layers against the oracle (tiny, the matrix-core class at 40 tokens,
    full size at 1 and 64 tokens: both top-k kernels);
  - a tie in selection score at the k / k+1 boundary (same router row, same
    bias): the recheck runs and the lower id wins.
Ids are compared bit for bit, weights within 2e-6, values within 2e-3 RMS.
"""
import numpy as np
import pytest
import torch

import gen
import gen.device
import oracle
from gpu_util import (W_TOL, assert_close, assert_close_bf16, log, oracle_expert, require_gpu,
                      to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _layer(wr, routed, shared, k, out_dtype, router, bias):
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    if isinstance(wr, np.ndarray):
        wr = torch.from_numpy(np.ascontiguousarray(wr).view(np.int16)).to("cuda").view(torch.bfloat16)
    b = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias)).to("cuda")
    return MoELayer(wr, routed, shared, k, out_dtype=out_dtype, router=router, router_bias=b)


@pytest.mark.parametrize("router", ["sigmoid", "sigmoid_norm"])
def test_router_fixture_on_gpu(router):
    require_gpu()
    from conftest import golden
    from oracle_pins import sigmoid
    g = golden("sigmoid_router_fixture.json")
    logits = np.array(g["logits"], dtype=np.float64)
    T, E = logits.shape
    d = 32
    x = np.zeros((T, d), dtype=np.float32)
    x[np.arange(T), np.arange(T)] = 1.0            # token t = unit vector e_t
    wr = np.zeros((E, d), dtype=np.uint16)
    for t in range(T):
        for e in range(E):
            wr[e, t] = gen.f64_to_bf16_bits(logits[t, e])   # small integers: exact in bf16
    # any small routed bank: only the routing is checked here
    cfg = gen.configs.LayerConfig(name="fixture", T=T, d=d, f=32, E=E, k=g["k"], n_shared=0,
                                  f_shared=0, x_dtype="f32", out_dtype="f32", scale_lo=-4,
                                  scale_hi=0)
    routed = {kk: torch.from_numpy(v).to("cuda") for kk, v in gen.routed_bank(cfg).items()}
    bias = np.array(g["bias"], dtype=np.float32)
    L = _layer(wr, routed, {}, g["k"], torch.float32, router, bias)
    diag = torch.zeros(4, dtype=torch.int32, device="cuda")
    idx, w, lg = L.route(torch.from_numpy(x).to("cuda"), want_logits=True, diag=diag)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(lg), logits.astype(np.float32))
    assert to_np(idx).tolist() == g["idx_biased"]
    log(f"  diag {to_np(diag).tolist()}")
    assert to_np(diag)[0] >= 1      # row 2's tie among six equal scores is rechecked
    for t in range(T):
        s = np.array([sigmoid(logits[t, e]) for e in g["idx_biased"][t]])
        want = s if router == "sigmoid" else s / s.sum()
        assert np.max(np.abs(to_np(w)[t] - want)) <= W_TOL, (t, to_np(w)[t], want)
    # the same weights without the bias choose the unbiased pairs
    L0 = _layer(wr, routed, {}, g["k"], torch.float32, router, None)
    idx0, _, _ = L0.route(torch.from_numpy(x).to("cuda"))
    torch.cuda.synchronize()
    assert to_np(idx0).tolist() == g["idx_unbiased"]


def _check_layer(orc, cfg, wl, router, bias, out_dtype="f32"):
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    L = _layer(wl.w_router, wl.routed, wl.shared, cfg.k, dt, router, bias)
    r = L.staged(wl.x)
    out = L(wl.x)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), r["out"].view(torch.uint8))
    bank = gen.routed_bank(cfg)
    ref = orc.layer(gen.x(cfg), gen.router(cfg), lambda e: {k: v[e] for k, v in bank.items()},
                    gen.shared_bank(cfg) if cfg.n_shared else None, cfg.k, cfg.E, router, bias)
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    assert np.max(np.abs(to_np(r["w"]) - ref["w"])) <= W_TOL
    assert np.array_equal(to_np(r["sorted_pair"]), ref["sorted_pair"])
    assert_close(to_np(r["y_perm"]), ref["y_perm"], "y_perm")
    if out_dtype == "bf16":
        assert_close_bf16(to_np(r["out"]), ref["out"], "out")
    else:
        assert_close(to_np(r["out"]), ref["out"], "out")
    log(f"  diag {to_np(r['diag']).tolist()}")
    assert to_np(r["diag"])[3] == 0


@pytest.mark.parametrize("router", ["sigmoid", "sigmoid_norm"])
@pytest.mark.parametrize("name,T", [("tiny", 37), ("medium", 40), ("medium", 600)])
def test_sigmoid_router_layer(orc, router, name, T):
    require_gpu()
    if name == "tiny":
        cfg = gen.get("tiny").with_tokens(T)
    else:
        cfg = gen.configs.LayerConfig(name="medium", T=T, d=512, f=512, E=32, k=8, n_shared=2,
                                      f_shared=256, x_dtype="bf16", out_dtype="f32",
                                      scale_lo=-8, scale_hi=0)
    log(f"case {cfg.name} T={T} {router}")
    wl = gen.device.build(cfg)
    _check_layer(orc, cfg, wl, router, gen.router_bias(cfg))


@pytest.mark.parametrize("router", ["sigmoid", "sigmoid_norm"])
@pytest.mark.parametrize("T", [1, 64])
def test_sigmoid_router_full_size(big, orc, router, T):
    """d = 7168, 896 experts top-16, 2 shared: one token (the fused one-token
    top-k kernel) and 64 (the batched one, matrix-core class); ids of every
    token bit for bit, values of sampled tokens."""
    cfg = gen.get("decode_b64").with_tokens(T)
    log(f"case full size T={T} {router}")
    bias = gen.router_bias(cfg)
    L = _layer(big.w_router, big.routed, big.shared, cfg.k, torch.bfloat16, router, bias)
    x = gen.device.activations(cfg)
    r = L.staged(x)
    out = L(x)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r["out"].view(torch.int16))
    x_host = gen.x(cfg)
    _, idx, w = orc.route(oracle.to_f64(x_host), gen.router(cfg), cfg.k, router, bias)
    assert np.array_equal(to_np(r["idx"]), idx)
    assert np.max(np.abs(to_np(r["w"]) - w)) <= W_TOL
    toks = np.array(sorted({0, T // 2, T - 1}))
    out_ref, _, _ = orc.token_outputs(x_host[toks], idx[toks], w[toks], oracle_expert(cfg),
                                      gen.shared_bank(cfg))
    assert_close_bf16(to_np(out)[toks], out_ref, "out (sampled)")
    assert to_np(r["diag"])[3] == 0


@pytest.mark.parametrize("T", [1, 5])
def test_sigmoid_score_tie_rechecked(big, orc, T):
    """Token 0's k-th expert by selection score gets a twin outside its top
    k + 1 (same router row, same bias): the scores tie exactly, the
    certificate fails, the recheck runs and the lower id wins, as in the
    oracle."""
    cfg = gen.get("decode_b64").with_tokens(T)
    k = cfg.k
    x_host, wr = gen.x(cfg), gen.router(cfg).copy()
    bias = gen.router_bias(cfg).copy()
    lg = orc.router_logits(oracle.to_f64(x_host[:1]), wr)[0]
    score = 1.0 / (1.0 + np.exp(-lg)) + bias.astype(np.float64)
    order = sorted(range(cfg.E), key=lambda e: (-score[e], e))
    ek = order[k - 1]
    partner = min(e for e in order[k + 1:] if e % 64 != ek % 64)
    wr[partner] = wr[ek]
    bias[partner] = bias[ek]
    log(f"case full size T={T}: e_k {ek} twin {partner}")
    _, idx, w = orc.route(oracle.to_f64(x_host), wr, k, "sigmoid_norm", bias)
    assert (min(ek, partner) in idx[0]) and (max(ek, partner) not in idx[0])
    L = _layer(wr, big.routed, big.shared, k, torch.bfloat16, "sigmoid_norm", bias)
    x = gen.device.activations(cfg)
    diag = torch.zeros(4, dtype=torch.int32, device="cuda")
    g_idx, g_w, _ = L.route(x, diag=diag)
    ldiag = torch.zeros(4, dtype=torch.int32, device="cuda")
    L(x, diag=ldiag)
    torch.cuda.synchronize()
    log(f"  route diag {to_np(diag).tolist()}, layer diag {to_np(ldiag).tolist()}")
    assert np.array_equal(to_np(g_idx), idx)
    assert np.max(np.abs(to_np(g_w) - w)) <= W_TOL
    assert to_np(diag)[0] >= 1 and to_np(ldiag)[0] >= 1
