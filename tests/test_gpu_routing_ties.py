"""GPU parity of the routing stage where the first-pass selection cannot
decide: exact ties and near-ties at the k / k+1 boundary, and all-zero tokens.

The top-k kernels select on fp64 logits carrying a bound on their distance to
the sequential fp64 sum, certify the selection when every chosen lower bound
beats every other upper bound, and otherwise recompute the undecided logits
in the oracle's own operation order and select again
(diag[K3MOE_DIAG_RECHECKED_TOKENS] counts such tokens).  Every case here is
built so that the certificate must fail, and checks that the recheck ran and
that the chosen ids equal the oracle's bit for bit:
  - exact ties: router row e_k (the k-th best expert of the token) copied
    into a row that is not in the top k + 1, in the same lane (e_k + 64 j:
    several of one lane's entries tie) or another lane (several lanes hold
    the wave maximum at once: the lowest id must win);
  - near-ties: the copy differs from row e_k in its last element only, and
    that activation element is tiny, so the two logits differ by far less
    than the stored bound; "up" gives the higher id the larger logit (it must
    win against the tie-break), "down" the lower id; an "ulp" variant makes
    the gap a few units in the last place of the logit, below the kernels'
    own rounding;
  - a token of zeros: every logit and every bound is 0, so all E experts tie
    and the lowest k ids win with weight 1/k.
The equal-logit rule (lower id wins) is the workload's tie reading; the
hand-worked tie fixture (4 experts, top-2) is checked the same way.
"""
import numpy as np
import pytest
import torch

import gen
import gen.device
import oracle
from gpu_util import W_TOL, assert_close, assert_close_bf16, log, oracle_expert, require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


# --------------------------------------------------------------- host builders
def _bf16_bits_of(v: float) -> int:
    return gen.f64_to_bf16_bits(v)


def _ranked(logits_row: np.ndarray):
    """Expert ids by (logit desc, id asc)."""
    return sorted(range(logits_row.size), key=lambda e: (-logits_row[e], e))


def _set_tiny(x: np.ndarray, t: int, i: int, v: float):
    if x.dtype == np.uint16:
        x[t, i] = _bf16_bits_of(v)
    else:
        x[t, i] = np.float32(v)


def _bf16_neighbour(bits: int, up: bool) -> int:
    """The next bf16 above (up) or below a finite nonzero value."""
    neg = bool(bits & 0x8000)
    return bits + 1 if (up != neg) else bits - 1


def _case_holds(orc, x, wr, k, t, mode, partner, ek) -> bool:
    """The rewritten inputs do make a tie or near-tie at token t's boundary."""
    lg = orc.router_logits(oracle.to_f64(x[t:t + 1]), wr)[0]
    if mode == "zero":
        return bool(np.all(lg == 0))
    order = _ranked(lg)
    if set(order[k - 1:k + 1]) != {ek, partner}:
        return False
    gap = abs(lg[ek] - lg[partner])
    if mode in ("same_lane", "next_lane"):
        return gap == 0.0
    if mode == "near_ulp":
        return gap <= 64 * np.spacing(abs(lg[ek]))
    return 0 < gap < 1e-10 * max(1.0, abs(lg[ek]))


def _rewrite(orc, x, wr, t, k, mode, tiny_x, skip):
    """One attempt at token t: rewrite router rows (and, for near-ties, the
    token's last activation) so that its k-th choice is tied or near-tied with
    an expert outside its top k + 1; `skip` partners are passed over."""
    x = x.copy()
    wr = wr.copy()
    E, d = wr.shape
    if mode == "zero":
        x[t] = 0
        return x, wr, None, None
    near = mode.startswith("near")
    if near:
        _set_tiny(x, t, d - 1, tiny_x)
    logits = orc.router_logits(oracle.to_f64(x[t:t + 1]), wr)[0]
    order = _ranked(logits)
    ek = order[k - 1]
    outside = [e for e in order[k + 1:]]
    # preferred partners first: a higher id for "up" (it must win against the
    # tie-break), a lower one for "down" (it must lose despite it)
    if mode == "same_lane":
        cands = sorted(e for e in outside if e % 64 == ek % 64)
    elif mode in ("next_lane", "near_up", "near_ulp"):
        other = [e for e in outside if e % 64 != ek % 64]
        cands = sorted(e for e in other if e > ek) + sorted(e for e in other if e < ek)
    elif mode == "near_down":
        cands = sorted((e for e in outside if e < ek), reverse=True) + \
            sorted(e for e in outside if e > ek)
    else:
        raise ValueError(mode)
    if skip >= len(cands):
        return None
    partner = cands[skip]
    wr[partner] = wr[ek]
    if near:
        # the partner's last weight one bf16 step away from e_k's: its logit
        # moves by x[t][d-1] * step, far below the stored bound
        b = int(wr[ek, d - 1])
        if b & 0x7FFF == 0:
            b = _bf16_bits_of(0.015625)
            wr[ek, d - 1] = b
        nb = _bf16_neighbour(b, mode in ("near_up", "near_ulp"))
        wr[partner, d - 1] = nb
        if mode == "near_ulp":
            # a gap of about 4 units in the last place of the logit
            step = abs(float(oracle.to_f64(np.array([nb], np.uint16))[0]
                             - oracle.to_f64(np.array([b], np.uint16))[0]))
            ulp = np.spacing(abs(logits[ek]))
            _set_tiny(x, t, d - 1, 2.0 ** np.floor(np.log2(4 * ulp / step)))
    return x, wr, partner, ek


def make_cases(orc, x: np.ndarray, wr: np.ndarray, k: int, modes, tiny_x: float):
    """Builds the cases `modes` (a list) on tokens of one batch, in token
    order.  A rewrite for one token can disturb another's boundary (a copied
    row enters its top k), so each new case is kept only when every case
    built so far still holds; a token that admits no such rewrite is left as
    it is and the case moves to the next token.  Returns x, wr and the
    {token: mode} map."""
    cases = []
    t = 0
    for mode in modes:
        while True:
            assert t < x.shape[0], f"no token left for {mode}"
            done = False
            for skip in range(64):
                got = _rewrite(orc, x, wr, t, k, mode, tiny_x, skip)
                if got is None:
                    break
                x2, wr2, partner, ek = got
                trial = cases + [(t, mode, partner, ek)]
                if all(_case_holds(orc, x2, wr2, k, *c) for c in trial):
                    x, wr, cases, done = x2, wr2, trial, True
                    break
            t += 1
            if done:
                break
    for tt, mode, partner, ek in cases:
        lg = orc.router_logits(oracle.to_f64(x[tt:tt + 1]), wr)[0]
        gap = 0.0 if mode == "zero" else abs(lg[ek] - lg[partner])
        log(f"    token {tt} {mode}: e_k {ek} partner {partner} gap {gap:.3e}")
    return x, wr, {c[0]: c[1] for c in cases}


def _layer(wr_bits, routed, shared, k, out_dtype, dev="cuda"):
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    return MoELayer(torch.from_numpy(np.ascontiguousarray(wr_bits).view(np.int16)).to(dev)
                    .view(torch.bfloat16), routed, shared, k, out_dtype=out_dtype)


def _x_dev(x: np.ndarray, dev="cuda"):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _compare_routing(orc, L, xd, x, wr, k, E, n_forced):
    """Staged route: ids and weights against the oracle, and the recheck count."""
    diag = torch.zeros(4, dtype=torch.int32, device="cuda")
    idx, w, logits = L.route(xd, want_logits=True, diag=diag)
    torch.cuda.synchronize()
    lg, idx_ref, w_ref = orc.route(oracle.to_f64(x), wr, k)
    got = to_np(idx)
    bad = np.nonzero(np.any(got != idx_ref, axis=1))[0]
    assert bad.size == 0, f"tokens {bad.tolist()}: {got[bad]} vs {idx_ref[bad]}"
    assert np.max(np.abs(to_np(w) - w_ref)) <= W_TOL
    rechecked = int(to_np(diag)[0])
    log(f"  rechecked tokens: {rechecked} (forced {n_forced})")
    assert rechecked >= n_forced
    return idx_ref, w_ref


# ------------------------------------------------------ small layers, fp32 x
def _small_cfg(E, k, T, x_dtype="f32", d=256, f=128):
    base = gen.get("tiny")
    return gen.configs.LayerConfig(**{**base.__dict__, "E": E, "k": k, "T": T, "d": d, "f": f,
                                      "x_dtype": x_dtype, "name": f"ties_E{E}_k{k}_T{T}_{x_dtype}"})


@pytest.mark.parametrize("E,k", [(128, 8), (16, 4)])
def test_ties_small_layer(orc, E, k):
    """Vector-ALU fp64 router + the batched top-k kernel (fp32 x): one token
    per case, all in one batch, plus an untouched token."""
    require_gpu()
    modes = ["same_lane", "next_lane", "near_up", "near_down", "near_ulp", "zero"]
    if E <= 64:
        modes.remove("same_lane")
    cfg = _small_cfg(E, k, 16)
    log(f"case {cfg.name}: modes {modes}")
    x, wr, tm = make_cases(orc, gen.x(cfg), gen.router(cfg), k, modes, 2.0 ** -32)
    wl = gen.device.build(cfg)
    L = _layer(wr, wl.routed, wl.shared, k, torch.float32)
    xd = _x_dev(x)
    idx_ref, _ = _compare_routing(orc, L, xd, x, wr, k, E, len(modes))
    zero_t = [t for t, m in tm.items() if m == "zero"][0]
    assert list(idx_ref[zero_t]) == list(range(k))
    # the whole layer on the rewritten inputs: same bits as the staged calls,
    # values against the oracle
    bank = gen.routed_bank(cfg)
    ref = orc.layer(x, wr, lambda e: {kk: v[e] for kk, v in bank.items()},
                    gen.shared_bank(cfg), k, E)
    r = L.staged(xd)
    out = L(xd)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    assert_close(to_np(r["out"]), ref["out"], "out")
    assert np.all(to_np(r["w"])[zero_t] == np.float32(1.0 / k))


def test_hand_tie_fixture(orc):
    """The hand-worked tie: four experts whose logits are 0, 1, 1, 1 (top-2):
    ids 1 and 2 with weights 1/2, through the C ABI."""
    require_gpu()
    import oracle_pins
    x, wr2, experts = oracle_pins._hand_case(0)
    d = x.shape[1]
    wr = np.zeros((4, d), dtype=np.uint16)
    wr[1:, 0] = gen.BF16_ONE
    experts = experts + experts
    routed = {kk: torch.from_numpy(np.stack([e[kk] for e in experts])).to("cuda")
              for kk in experts[0]}
    L = _layer(wr, routed, {}, 2, torch.float32)
    xd = _x_dev(x)
    idx_ref, w_ref = _compare_routing(orc, L, xd, x, wr, 2, 4, 1)
    assert list(idx_ref[0]) == [1, 2] and list(w_ref[0]) == [0.5, 0.5]
    r = L.staged(xd)
    torch.cuda.synchronize()
    assert to_np(r["w"]).tolist() == [[0.5, 0.5]]
    ref = orc.layer(x, wr, lambda e: experts[e], None, 2, 4)
    assert_close(to_np(r["out"]), ref["out"], "out")


# ------------------------------ matrix-core class routers (bf16, d = 512)
@pytest.mark.parametrize("T", [40, 600])
def test_ties_mfma_router(orc, T):
    """The matrix-core class's two routers: the fp64 matrix-core logits
    (40 tokens) and, from 512 tokens, bf16 matrix-core logits whose
    candidates are refined in fp64 (600): ties, near-ties and a zero token
    inside one batch."""
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import PATH_MFMA
    E, k = 32, 8
    cfg = gen.configs.LayerConfig(name=f"ties_mfma_T{T}", T=T, d=512, f=512, E=E, k=k, n_shared=2,
                                  f_shared=256, x_dtype="bf16", out_dtype="f32", scale_lo=-8,
                                  scale_hi=0)
    modes = ["next_lane", "near_up", "near_down", "near_ulp", "zero"]
    x, wr, _ = make_cases(orc, gen.x(cfg), gen.router(cfg), k, modes, 2.0 ** -30)
    wl = gen.device.build(cfg)
    L = _layer(wr, wl.routed, wl.shared, k, torch.float32)
    assert L.path_class(T) == PATH_MFMA
    xd = _x_dev(x)
    _compare_routing(orc, L, xd, x, wr, k, E, len(modes))
    bank = gen.routed_bank(cfg)
    ref = orc.layer(oracle.to_f64(x), wr, lambda e: {kk: v[e] for kk, v in bank.items()},
                    gen.shared_bank(cfg), k, E)
    r = L.staged(xd)
    out = L(xd)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    assert_close(to_np(r["out"]), ref["out"], "out")


# ------------------------------------------------- full size, one token
@pytest.mark.parametrize("mode", ["same_lane", "next_lane", "near_up", "near_down", "near_ulp",
                                  "zero"])
def test_ties_full_size_one_token(big, orc, mode):
    """d = 7168, 896 experts, top-16, one bf16 token: both top-k kernels, the
    batched one (staged route) and the one-token one fused with the shared
    experts' gate/up (the layer call), must run the recheck and agree with
    the oracle; the layer equals the staged calls bit for bit."""
    cfg = gen.get("decode_b1")
    k = cfg.k
    log(f"case full-size T=1 {mode}")
    x, wr, _ = make_cases(orc, gen.x(cfg), gen.router(cfg), k, [mode], 2.0 ** -24)
    L = _layer(wr, big.routed, big.shared, k, torch.bfloat16)
    xd = _x_dev(x)
    idx_ref, w_ref = _compare_routing(orc, L, xd, x, wr, k, cfg.E, 1)
    diag = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = L(xd, diag=diag)
    r = L.staged(xd)
    torch.cuda.synchronize()
    log(f"  layer diag {to_np(diag).tolist()}")
    assert int(to_np(diag)[0]) == 1, "the one-token top-k kernel did not recheck"
    assert torch.equal(out.view(torch.int16), r["out"].view(torch.int16))
    if mode == "zero":
        assert list(idx_ref[0]) == list(range(k))
    out_ref, sh_ref, _ = orc.token_outputs(x, idx_ref, w_ref, oracle_expert(cfg),
                                           gen.shared_bank(cfg))
    assert_close_bf16(to_np(out), out_ref, "out")
