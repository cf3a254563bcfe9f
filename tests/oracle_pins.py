"""Pins of the CPU oracle against things other than itself.

Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle
disagrees with a fact fixed outside it: the OCP MX format tables, a closed form
worked out by hand, a library routine for a special case, brute force through
an independent numpy decode, or an exact invariant.  test_oracle_pins runs them
on the oracle; test_oracle_mutants runs them on copies of the oracle with one
plausible mistake planted each and requires that some pin fails.
"""
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import gen  # noqa: E402
from oracle import to_f64  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


# ------------------------------------------------------------- numpy helpers
def np_decode(q, s):
    """Independent MXFP4 decode: table lookup of each nibble (from the spec
    table fixture) times 2^(s-127) via ldexp; low nibble = even element."""
    table = np.array(_golden("e2m1_table.json")["values"], dtype=np.float64)
    q = np.asarray(q, dtype=np.uint8)
    codes = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = q & 0xF
    codes[..., 1::2] = q >> 4
    scale = np.ldexp(1.0, np.asarray(s, dtype=np.int64) - 127)
    scale = np.where(np.asarray(s) == 255, np.nan, scale)
    return table[codes] * np.repeat(scale, 32, axis=-1)


def np_silu(z):
    return z / (1.0 + np.exp(-z))


def tiny():
    return gen.get("tiny")


def tiny_inputs():
    c = tiny()
    bank = gen.routed_bank(c)
    return c, gen.x(c), gen.router(c), bank, gen.shared_bank(c)


def _expert(bank, e):
    return {k: v[e] for k, v in bank.items()}


def _bf16_bits(vals):
    return np.array([gen.f64_to_bf16_bits(float(v)) for v in np.ravel(vals)],
                    dtype=np.uint16).reshape(np.shape(vals))


# ------------------------------------------------------------------- formats
def pin_e2m1_table(o):
    """E2M1 codes 0..15 equal the OCP MX v1.0 FP4 table, signed zero included."""
    vals = _golden("e2m1_table.json")["values"]
    for c, v in enumerate(vals):
        got = o.e2m1(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (c, got, v)


def pin_e8m0_all(o):
    """E8M0 byte s is 2^(s-127) for s < 255 and NaN for 255 (OCP MX v1.0)."""
    for s in range(255):
        assert o.e8m0(s) == math.ldexp(1.0, s - 127), s
    assert math.isnan(o.e8m0(255))
    for s, v in _golden("e2m1_table.json")["e8m0"]["pins"]:
        assert o.e8m0(s) == v, (s, v)


def pin_decode_exhaustive(o):
    """Every (code, scale) pair: decode = table[code] * 2^(s-127), in every
    nibble position and block; row r uses scale byte r, codes 0..15 twice."""
    table = _golden("e2m1_table.json")["values"]
    q = np.zeros((256, 16), dtype=np.uint8)         # 256 rows x 32 columns
    for i in range(16):
        lo, hi = (2 * i) % 16, (2 * i + 1) % 16
        q[:, i] = lo | (hi << 4)
    s = np.arange(256, dtype=np.uint8).reshape(256, 1)
    got = o.mxfp4_decode(q, s)
    for r in range(256):
        for i in range(32):
            code = i % 16
            want = math.nan if r == 255 else table[code] * math.ldexp(1.0, r - 127)
            g = got[r, i]
            if math.isnan(want):
                assert math.isnan(g), (r, i, g)
            else:
                assert g == want, (r, i, g, want)


def pin_nibble_and_block_order(o):
    """Byte 0x21 holds element 0 = code 1 (0.5) and element 1 = code 2 (1.0);
    element i takes the scale byte of block i // 32."""
    q = np.zeros((1, 32), dtype=np.uint8)
    q[0, 0] = 0x21
    q[0, 16] = 0x43           # elements 32, 33 -> codes 3, 4
    s = np.array([[127, 129]], dtype=np.uint8)
    got = o.mxfp4_decode(q, s)[0]
    assert got[0] == 0.5 and got[1] == 1.0, got[:2]
    assert got[32] == 1.5 * 4 and got[33] == 2.0 * 4, got[32:34]
    assert np.all(got[2:32] == 0) and np.all(got[34:] == 0)


# ------------------------------------------------------------ hand example
def _hand_case(col):
    d = f = 32
    x = np.zeros((1, d), dtype=np.float32)
    x[0, col] = 1.0
    wr = np.zeros((2, d), dtype=np.uint16)
    wr[0, col] = gen.BF16_ONE
    byte, shift = col // 2, 4 * (col % 2)

    def expert(gate_code, gate_s, up_code, up_s, down_code):
        w13 = np.zeros((2 * f, d // 2), dtype=np.uint8)
        w13s = np.full((2 * f, d // 32), 127, dtype=np.uint8)
        w13[:f, byte] = gate_code << shift
        w13s[:f, col // 32] = gate_s
        w13[f:, byte] = up_code << shift
        w13s[f:, col // 32] = up_s
        w2 = np.full((d, f // 2), down_code | (down_code << 4), dtype=np.uint8)
        w2s = np.full((d, f // 32), 127, dtype=np.uint8)
        return dict(w13=w13, w13_scale=w13s, w2=w2, w2_scale=w2s)

    experts = [expert(2, 127, 4, 127, 1), expert(6, 126, 2, 128, 9)]
    return x, wr, experts


def pin_hand_two_experts(o):
    """Closed form of the hand-worked 1-token / 2-expert layer, at column 0
    (low nibble) and column 1 (high nibble)."""
    g = _golden("hand_two_experts.json")
    want = 32 * sigmoid(1) ** 2 - 64 * sigmoid(-1) * sigmoid(2)
    assert abs(want - g["out"]) <= 4e-16 * abs(want)
    for col in g["columns"]:
        x, wr, experts = _hand_case(col)
        r = o.layer(x, wr, lambda e: experts[e], None, k=2, E=2)
        assert list(r["logits"][0]) == [1.0, 0.0]
        assert list(r["idx"][0]) == [0, 1]
        assert abs(r["w"][0, 0] - sigmoid(1)) < 1e-16 and abs(r["w"][0, 1] - sigmoid(-1)) < 1e-16
        # fp64 rounding budget: ~f additions per output (u = 2^-53 each)
        y0, y1 = 32 * sigmoid(1), -64 * sigmoid(2)
        budget = lambda mag: (32 + 8) * 2.0 ** -53 * mag
        assert np.all(np.abs(r["y_perm"][0] - y0) <= budget(abs(y0)))
        assert np.all(np.abs(r["y_perm"][1] - y1) <= budget(abs(y1)))
        mag = abs(sigmoid(1) * y0) + abs(sigmoid(-1) * y1)
        assert np.all(np.abs(r["out"][0] - g["out"]) <= budget(mag)), (col, r["out"][0][:4])


def pin_hand_tie(o):
    """Equal logits: the lower expert ids win, with equal weights."""
    d = 32
    x = np.zeros((1, d), dtype=np.float32)
    x[0, 0] = 1.0
    wr = np.zeros((4, d), dtype=np.uint16)
    wr[:, 0] = gen.BF16_ONE          # all four logits are 1.0
    wr[0, 0] = 0                     # expert 0 drops to 0.0
    logits, idx, w = o.route(to_f64(x), wr, 2)
    assert list(idx[0]) == [1, 2], idx
    assert list(w[0]) == [0.5, 0.5], w


# -------------------------------------------------------------- routing
def pin_router_vs_fsum(o):
    """Router logits equal the exactly rounded dot product (math.fsum of the
    exact products) within the fp64 summation bound d * 2^-53 * sum|p|."""
    c, x, wr, _, _ = tiny_inputs()
    x64 = to_f64(x)
    w64 = to_f64(wr)
    logits = o.router_logits(x64, wr)
    for t in range(c.T):
        for e in range(c.E):
            p = x64[t] * w64[e]
            exact = math.fsum(p)
            bound = c.d * 2.0 ** -53 * np.abs(p).sum() * 1.01
            assert abs(logits[t, e] - exact) <= bound, (t, e, logits[t, e], exact)


def pin_topk_bruteforce(o):
    """Top-k = first k of a full sort by (logit desc, id asc), listed by
    ascending id; weights = softmax (scipy) of the chosen logits."""
    from scipy.special import softmax
    rng = np.random.default_rng(7)
    for T, E, k in [(5, 16, 4), (3, 9, 1), (4, 12, 12), (6, 20, 7)]:
        logits = rng.integers(-3, 4, size=(T, E)).astype(np.float64) * 0.25
        logits += rng.standard_normal((T, E)) * (rng.random((T, E)) < 0.5)
        idx, w = o.topk_softmax(logits, k)
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-logits[t, e], e))
            chosen = sorted(order[:k])
            assert list(idx[t]) == chosen, (t, list(idx[t]), chosen)
            want = softmax(logits[t, chosen])
            assert np.allclose(w[t], want, rtol=1e-14, atol=1e-300)
            assert abs(w[t].sum() - 1.0) <= 1e-15 * k


def pin_sigmoid_router_fixture(o):
    """The K3 router fixture: selection by sigmoid(l) + bias (the bias changes
    the chosen pair in five of six rows), weights the unbiased sigmoid(l),
    raw or renormalised over the chosen; without the bias the chosen pairs
    are the unbiased ones."""
    g = _golden("sigmoid_router_fixture.json")
    logits = np.array(g["logits"], dtype=np.float64)
    bias = np.array(g["bias"], dtype=np.float32)
    k = g["k"]
    idx, w_raw = o.topk_sigmoid(logits, k, bias, norm=False)
    idx2, w_norm = o.topk_sigmoid(logits, k, bias, norm=True)
    assert idx.tolist() == g["idx_biased"], idx.tolist()
    assert np.array_equal(idx2, idx)
    flips = sum(a != b for a, b in zip(g["idx_biased"], g["idx_unbiased"]))
    assert flips == 5
    idx0, _ = o.topk_sigmoid(logits, k, None)
    assert idx0.tolist() == g["idx_unbiased"], idx0.tolist()
    for t in range(logits.shape[0]):
        s = [sigmoid(logits[t, e]) for e in g["idx_biased"][t]]
        assert np.allclose(w_raw[t], s, rtol=4e-16, atol=0), (t, w_raw[t], s)
        assert np.allclose(w_norm[t], np.array(s) / sum(s), rtol=8e-16, atol=0), (t, w_norm[t])


def pin_sigmoid_router_bruteforce(o):
    """Random logits and biases: the chosen set is the first k of a full
    sort by (scipy's expit(l) + bias desc, id asc), listed by ascending id;
    the weights are expit(l); with no bias the set is the logit top-k."""
    from scipy.special import expit
    rng = np.random.default_rng(11)
    T, E, k = 40, 48, 6
    logits = rng.standard_normal((T, E)) * 2.0
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    idx, w = o.topk_sigmoid(logits, k, bias)
    for t in range(T):
        score = expit(logits[t]) + bias.astype(np.float64)
        order = sorted(range(E), key=lambda e: (-score[e], e))
        want = sorted(order[:k])
        assert idx[t].tolist() == want, (t, idx[t], want)
        assert np.allclose(w[t], expit(logits[t, want]), rtol=4e-16, atol=0)
    idx0, _ = o.topk_sigmoid(logits, k, None)
    idx_l, _ = o.topk_softmax(logits, k)
    assert np.array_equal(idx0, idx_l)


def pin_topk_full_and_single(o):
    """k = E gives the full softmax over all experts; k = 1 gives weight 1 on
    the argmax."""
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((4, 10)) * 3
    idx, w = o.topk_softmax(logits, 10)
    assert np.all(idx == np.arange(10))
    assert np.allclose(w, softmax(logits, axis=1), rtol=1e-14, atol=0)
    idx1, w1 = o.topk_softmax(logits, 1)
    assert np.all(idx1[:, 0] == np.argmax(logits, axis=1)) and np.all(w1 == 1.0)


def pin_permute_vs_stable_argsort(o):
    """Counts = bincount, offsets = exclusive scan, sorted pairs = numpy's
    stable argsort of the flattened ids, pair_pos its inverse."""
    rng = np.random.default_rng(11)
    for T, E, k in [(7, 9, 3), (33, 16, 4), (1, 5, 5)]:
        idx = np.stack([np.sort(rng.choice(E, size=k, replace=False)) for _ in range(T)])
        idx = idx.astype(np.int32)
        counts, offsets, sp, pp = o.permute(idx, E)
        flat = idx.ravel()
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(sp, order)
        inv = np.empty_like(order)
        inv[order] = np.arange(len(order))
        assert np.array_equal(pp, inv)


# ------------------------------------------------------------------ experts
def pin_ffn_bruteforce(o):
    """One expert over several rows equals numpy fp64 matmuls on weights
    decoded independently (spec table + ldexp), within 1e-12 of the output scale."""
    c, x, _, bank, _ = tiny_inputs()
    x64 = to_f64(x)
    for e in (0, 5, 15):
        ex = _expert(bank, e)
        y, h = o.mxfp4_ffn(ex, x64, want_h=True)
        w13 = np_decode(ex["w13"], ex["w13_scale"])
        w2 = np_decode(ex["w2"], ex["w2_scale"])
        g, u = x64 @ w13[:c.f].T, x64 @ w13[c.f:].T
        h_ref = np_silu(g) * u
        y_ref = h_ref @ w2.T
        assert np.max(np.abs(h - h_ref)) <= 1e-12 * np.max(np.abs(h_ref)), e
        assert np.max(np.abs(y - y_ref)) <= 1e-12 * np.max(np.abs(y_ref)), e


def pin_shared_bruteforce(o):
    """bf16 shared expert FFN equals numpy fp64 matmuls on the bf16 weights."""
    c, x, _, _, sh = tiny_inputs()
    x64 = to_f64(x)
    w13 = to_f64(sh["w13"][0])
    w2 = to_f64(sh["w2"][0])
    y = o.bf16_ffn(sh["w13"][0], sh["w2"][0], x64)
    fs = c.f_shared
    y_ref = (np_silu(x64 @ w13[:fs].T) * (x64 @ w13[fs:].T)) @ w2.T
    assert np.max(np.abs(y - y_ref)) <= 1e-12 * np.max(np.abs(y_ref))


def pin_single_expert_is_swiglu(o):
    """E = k = 1: the layer is the textbook dense SwiGLU FFN W2(silu(W1 x) * W3 x)
    of the one expert plus the shared expert (weight exactly 1)."""
    c, x, _, bank, sh = tiny_inputs()
    ex = _expert(bank, 3)
    wr = np.zeros((1, c.d), dtype=np.uint16)
    r = o.layer(x, wr, lambda e: ex, sh, k=1, E=1)
    assert np.all(r["w"] == 1.0) and np.all(r["idx"] == 0)
    x64 = to_f64(x)
    W = np_decode(ex["w13"], ex["w13_scale"])
    W2 = np_decode(ex["w2"], ex["w2_scale"])
    S13, S2 = to_f64(sh["w13"][0]), to_f64(sh["w2"][0])
    ffn = (np_silu(x64 @ W[:c.f].T) * (x64 @ W[c.f:].T)) @ W2.T
    shared = (np_silu(x64 @ S13[:c.f_shared].T) * (x64 @ S13[c.f_shared:].T)) @ S2.T
    want = shared + ffn
    assert np.max(np.abs(r["out"] - want)) <= 1e-12 * np.max(np.abs(want))


def pin_metamorphic_scales_and_signs(o):
    """Exact in binary floating point: +1 on every w2 scale doubles y; flipping
    the sign bit of every w2 code negates y; +1 on every up-row scale doubles h
    and y; +1 on the gate rows leaves u unchanged (h changes nonlinearly)."""
    c, x, _, bank, _ = tiny_inputs()
    x64 = to_f64(x)
    ex = _expert(bank, 7)
    y, h = o.mxfp4_ffn(ex, x64, want_h=True)
    ex2 = dict(ex, w2_scale=ex["w2_scale"] + 1)
    assert np.array_equal(o.mxfp4_ffn(ex2, x64), 2 * y)
    ex3 = dict(ex, w2=ex["w2"] ^ 0x88)
    assert np.array_equal(o.mxfp4_ffn(ex3, x64), -y)
    s = ex["w13_scale"].copy()
    s[c.f:] += 1
    y4, h4 = o.mxfp4_ffn(dict(ex, w13_scale=s), x64, want_h=True)
    assert np.array_equal(h4, 2 * h) and np.array_equal(y4, 2 * y)


# ------------------------------------------------ MXFP4 activation quantiser
E2M1_POS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7 (OCP MX v1.0)


def np_quantize_mxfp4(v):
    """OCP MX v1.0 MXFP4 quantiser written out independently: per block of
    32, scale 2^(floor(log2 max|v|) - 2) (X / scale in [4, 8)), each element
    the nearest E2M1 magnitude by exhaustive search (ties: the even code),
    above 6 saturating; returns the quantised values (fp64)."""
    v = np.asarray(v, dtype=np.float64).reshape(-1, 32)
    out = np.empty_like(v)
    for b in range(v.shape[0]):
        X = np.max(np.abs(v[b]))
        e = 0 if X == 0 else int(math.floor(math.log2(X))) - 2
        unit = 2.0 ** e if X > 0 else 2.0 ** -127
        for i in range(32):
            a = abs(v[b, i]) / unit
            cands = sorted(range(8), key=lambda c: (abs(a - E2M1_POS[c]), c & 1))
            out[b, i] = math.copysign(E2M1_POS[cands[0]] * unit, v[b, i])
    return out


def pin_mxfp4_quantizer_definition(o):
    """The oracle's MXFP4 quantiser against the written-out definition: random
    blocks over many magnitudes, exact midpoints (ties to the even code),
    saturation above 6, zeros of both signs, and an all-zero block."""
    rng = np.random.default_rng(3)
    blocks = [rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20) for _ in range(60)]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.9, 7.5, -0.25, -2.5, -5.0,
                     4.0, 0.0, -0.0] + [1.0] * 17)
    blocks += [mids, mids * 2.0 ** -9, np.zeros(32), -mids * 2.0 ** 30]
    v = np.concatenate(blocks)
    codes, scales = o.quantize_mxfp4(v.reshape(1, -1))
    got = o.mxfp4_decode(codes, scales).ravel()
    want = np_quantize_mxfp4(v).ravel()
    assert np.array_equal(np.signbit(got[want == 0]), np.signbit(want[want == 0]))
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]
    # the worked midpoints: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2,
    # 2.5 -> 2, 3.5 -> 4, 5 -> 4, 6.9 -> 6 (saturated), 7.5 -> 6
    m = got[60 * 32:60 * 32 + 9]
    assert m.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0], m


def pin_mxfp4_quantizer_roundtrip(o):
    """Every block that is already MXFP4 with its largest magnitude 4 or 6 (so
    the rule picks the same scale) comes back unchanged, codes and scale
    byte, over all 16 codes and many scales; a NaN block gets scale 255."""
    rng = np.random.default_rng(4)
    for s in (90, 117, 127, 128, 150):
        q = rng.integers(0, 256, size=(16, 16), dtype=np.uint8)
        q[:, 0] = (q[:, 0] & 0xF0) | np.where(np.arange(16) % 2, 7, 14)   # +6 or -4 at element 0
        sc = np.full((16, 1), s, dtype=np.uint8)
        vals = o.mxfp4_decode(q, sc)
        q2, s2 = o.quantize_mxfp4(vals)
        vals2 = o.mxfp4_decode(q2, s2)
        assert np.array_equal(s2, sc), s
        assert np.array_equal(vals2, vals), s
    bad = np.zeros(32)
    bad[5] = np.nan
    _, s3 = o.quantize_mxfp4(bad.reshape(1, 32))
    assert s3.tolist() == [[255]]


def pin_qact_ffn_dense(o):
    """The quantised-activation expert equals dense numpy: independent decode,
    x quantised by the written-out rule, gate/up, SiLU-GLU, h quantised, down."""
    c, x, _, bank, _ = tiny_inputs()
    x64 = to_f64(x)
    ex = _expert(bank, 5)
    y, h = o.mxfp4_ffn_qact(ex, x64, want_h=True)
    W13 = np_decode(ex["w13"], ex["w13_scale"])
    W2 = np_decode(ex["w2"], ex["w2_scale"])
    xq = np_quantize_mxfp4(x64).reshape(x64.shape)
    gu = xq @ W13.T
    hq = np_quantize_mxfp4(np_silu(gu[:, :c.f]) * gu[:, c.f:]).reshape(h.shape)
    assert np.array_equal(h, hq)
    want = hq @ W2.T
    assert np.max(np.abs(y - want)) <= 1e-12 * np.max(np.abs(want))


# ------------------------------------------------------------- RVQ3 experts
def _rvq_tiny():
    cfg = gen.configs.LayerConfig(name="rvq_tiny", T=3, d=256, f=128, E=4, k=2, n_shared=0,
                                  f_shared=0, x_dtype="f32", out_dtype="f32", scale_lo=-4,
                                  scale_hi=0)
    return cfg, gen.rvq_expert(cfg, 2), to_f64(gen.x(cfg))


def np_rvq_decode(idx, cb, rows, cols):
    """Independent decode: gather the three codewords of every (row, group)
    from the index layout [3][cols/128][rows][16] and add them."""
    idx = np.asarray(idx).reshape(3, cols // 128, rows, 16)
    groups = idx.transpose(0, 2, 1, 3).reshape(3, rows, cols // 8)      # [s][row][group]
    w = np.zeros((rows, cols // 8, 8))
    for st in range(3):
        w = w + cb[st].astype(np.float64)[groups[st]]
    return w.reshape(rows, cols)


def pin_rvq_decode_definition(o):
    """The oracle's RVQ3 decode equals the codeword sums gathered by numpy."""
    c, ex, _ = _rvq_tiny()
    got = o.rvq_decode(ex["w13"], ex["w13_cb"], 2 * c.f, c.d)
    assert np.array_equal(got, np_rvq_decode(ex["w13"], ex["w13_cb"], 2 * c.f, c.d))
    got2 = o.rvq_decode(ex["w2"], ex["w2_cb"], c.d, c.f)
    assert np.array_equal(got2, np_rvq_decode(ex["w2"], ex["w2_cb"], c.d, c.f))


def pin_rvq_partial_dot_tables(o):
    """The pages' evaluation, partial-dot tables: per token T_s[g][j] =
    C_s[j] . x_g, then y_r = sum over groups and stages of T_s[g][i_s[r][g]];
    it equals the oracle's FFN on the materialised weights (fp64 rounding)."""
    c, ex, x64 = _rvq_tiny()
    y, h = o.rvq_ffn(ex, x64, want_h=True)
    def table_gemv(idx, cb, rows, cols, v):
        groups = np.asarray(idx).reshape(3, cols // 128, rows, 16).transpose(0, 2, 1, 3)
        groups = groups.reshape(3, rows, cols // 8)
        out = np.zeros((v.shape[0], rows))
        for t in range(v.shape[0]):
            vg = v[t].reshape(cols // 8, 8)
            for st in range(3):
                table = vg @ cb[st].astype(np.float64).T                 # [group][entry]
                out[t] += table[np.arange(cols // 8)[None, :], groups[st]].sum(axis=1)
        return out
    gu = table_gemv(ex["w13"], ex["w13_cb"], 2 * c.f, c.d, x64)
    hh = np_silu(gu[:, :c.f]) * gu[:, c.f:]
    yy = table_gemv(ex["w2"], ex["w2_cb"], c.d, c.f, hh)
    assert np.max(np.abs(h - hh)) <= 1e-12 * np.max(np.abs(hh))
    assert np.max(np.abs(y - yy)) <= 1e-12 * np.max(np.abs(yy))


def pin_rvq_bytes_per_weight(o):
    """3 stages of 8-bit indices per 8 weights = 3.00 bits per weight; at the
    pages' expert size, 16 experts in each of 92 layers read about 17 GB per
    token."""
    g = _golden("rvq_byte_accounting.json")
    c, ex, _ = _rvq_tiny()
    assert ex["w13"].size * 8 / (2 * c.f * c.d) == g["bits_per_weight"]
    assert ex["w2"].size * 8 / (c.d * c.f) == g["bits_per_weight"]
    assert ex["w13_cb"].shape == (g["stages"], g["codebook_entries"], g["vector_dim"])
    per_token = g["experts_per_token"] * g["expert_params"] * g["bits_per_weight"] / 8
    assert abs(per_token / 2 ** 30 - g["gb_read_per_token_page"]) < 0.05


def pin_rvq_single_codeword(o):
    """Closed form: with stages 1 and 2 zero and stage 0's entry j equal to
    (j, j+1, ..., j+7) / 64, weight (r, 8g + k) is (i_0[r][g] + k) / 64."""
    c, ex, _ = _rvq_tiny()
    cb = np.zeros((3, 256, 8), dtype=np.float32)
    cb[0] = (np.arange(256)[:, None] + np.arange(8)[None, :]) / 64.0
    w = o.rvq_decode(ex["w13"], cb, 2 * c.f, c.d)
    i0 = ex["w13"][0].transpose(1, 0, 2).reshape(2 * c.f, c.d // 8)
    want = (np.repeat(i0, 8, axis=1) + np.tile(np.arange(8), c.d // 8)) / 64.0
    assert np.array_equal(w, want)


# ----------------------------------------------------------------- layer
def _layer_tiny(o, x=None, wr=None, bank=None, sh="default"):
    c, x0, wr0, bank0, sh0 = tiny_inputs()
    x = x0 if x is None else x
    wr = wr0 if wr is None else wr
    bank = bank0 if bank is None else bank
    sh = sh0 if isinstance(sh, str) else sh
    return c, o.layer(x, wr, lambda e: _expert(bank, e), sh, k=c.k, E=c.E)


def pin_weights_sum_to_one(o):
    c, r = _layer_tiny(o)
    assert np.all(np.abs(r["w"].sum(axis=1) - 1.0) <= 1e-15)
    assert np.all(np.diff(r["idx"], axis=1) > 0)


def pin_token_permutation(o):
    """Permuting the tokens permutes routing and outputs, bit for bit."""
    c, x, _, _, _ = tiny_inputs()
    perm = np.array([2, 0, 3, 1])
    _, r = _layer_tiny(o)
    _, rp = _layer_tiny(o, x=x[perm])
    assert np.array_equal(rp["idx"], r["idx"][perm])
    assert np.array_equal(rp["w"], r["w"][perm])
    assert np.array_equal(rp["out"], r["out"][perm])


def pin_batch_composition(o):
    """A token's output is the same bits alone or inside the batch."""
    c, x, _, _, _ = tiny_inputs()
    _, r = _layer_tiny(o)
    for t in range(c.T):
        _, r1 = _layer_tiny(o, x=x[t:t + 1])
        assert np.array_equal(r1["out"][0], r["out"][t])


def pin_zero_weight_expert(o):
    """A chosen expert whose weight underflows to exactly 0 contributes nothing,
    even when its weights decode to NaN (scale byte 255)."""
    c, x, wr, bank, sh = tiny_inputs()
    x = x.copy()
    x[:, 0] = 1.0
    wr = wr.copy()
    wr[:, 0] = 0
    wr[3, 0] = gen.f64_to_bf16_bits(2000.0)   # expert 3: logit ~ +2000 for every token
    wr[9, 0] = gen.f64_to_bf16_bits(1000.0)   # expert 9: logit ~ +1000 -> weight exp(-1000) = 0
    _, r = _layer_tiny(o, x=x, wr=wr)
    for t in range(c.T):
        ids = list(r["idx"][t])
        assert 3 in ids and 9 in ids, ids
        assert r["w"][t, ids.index(9)] == 0.0 and r["w"][t, ids.index(3)] == 1.0
    poisoned = {kk: v.copy() for kk, v in bank.items()}
    poisoned["w2_scale"][9] = 255
    poisoned["w13_scale"][9] = 255
    _, rp = _layer_tiny(o, x=x, wr=wr, bank=poisoned)
    assert np.all(np.isnan(rp["y_perm"][rp["offsets"][9]:rp["offsets"][10]]))
    assert np.array_equal(rp["out"], r["out"]) and np.all(np.isfinite(rp["out"]))


def pin_combine_definition(o):
    """Combine = shared + sum over slots of w * y, summed per token in slot
    order, checked against math.fsum with the fp64 bound."""
    rng = np.random.default_rng(5)
    T, k, d = 3, 4, 8
    y = rng.standard_normal((T * k, d))
    perm = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k))
    sh = rng.standard_normal((T, d))
    out = o.combine(y, perm, w, sh)
    for t in range(T):
        for j in range(d):
            terms = [sh[t, j]] + [w[t, s] * y[perm[t * k + s], j] for s in range(k)]
            assert abs(out[t, j] - math.fsum(terms)) <= 8 * 2.0 ** -53 * sum(map(abs, terms))


def pin_token_outputs_equal_layer(o):
    """The per-token path (each token alone, its chosen experts' rows gathered
    by expert, then combined in slot order) equals the batched layer's rows
    bit for bit: out, shared_y and every (token, slot) y row."""
    c, x, wr, bank, sh = tiny_inputs()
    _, r = _layer_tiny(o)
    toks = np.array([3, 0, 2])
    out, shy, y = o.token_outputs(x[toks], r["idx"][toks], r["w"][toks],
                                  lambda e: _expert(bank, e), sh)
    assert np.array_equal(out, r["out"][toks])
    assert np.array_equal(shy, r["shared_y"][toks])
    for n, t in enumerate(toks):
        for slot in range(c.k):
            assert np.array_equal(y[n, slot], r["y_perm"][r["pair_pos"][t * c.k + slot]])


ALL_PINS = [v for kname, v in sorted(globals().items()) if kname.startswith("pin_")]
