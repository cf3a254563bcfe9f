"""GPU parity of the HIP path (through the C ABI) with the CPU oracle.

Routing ids, counts, offsets, sorted pairs and positions must be equal; fp32
intermediates and outputs within 2e-3 x RMS of the oracle; bf16 outputs within
that plus one bf16 ulp; every result bit-identical run to run, between the
whole-layer call and the five staged calls, and for a token alone versus
inside a batch of the same path class.
"""
import numpy as np
import pytest
import torch

import gen
import gen.device
import oracle
from gpu_util import (W_TOL, assert_close, assert_close_bf16, check_permutation_properties,
                      decode_scaled_h, k3layer, log, oracle_expert, require_gpu, sample_tokens,
                      to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _full_oracle(cfg, orc, x_host):
    bank = gen.routed_bank(cfg)
    return orc.layer(x_host, gen.router(cfg), lambda e: {k: v[e] for k, v in bank.items()},
                     gen.shared_bank(cfg) if cfg.n_shared else None, cfg.k, cfg.E)


def _compare_full(r, ref, cfg, out_dtype):
    assert np.array_equal(to_np(r["idx"]), ref["idx"]), "expert ids differ"
    assert np.max(np.abs(to_np(r["w"]) - ref["w"])) <= W_TOL
    assert np.array_equal(to_np(r["counts"]), ref["counts"])
    assert np.array_equal(to_np(r["offsets"]), ref["offsets"])
    assert np.array_equal(to_np(r["sorted_pair"]), ref["sorted_pair"])
    assert np.array_equal(to_np(r["pair_pos"]), ref["pair_pos"])
    assert_close(to_np(r["logits"]), ref["logits"], "logits")
    assert_close(to_np(r["y_perm"]), ref["y_perm"], "y_perm")
    if cfg.n_shared:
        assert_close(to_np(r["shared_y"]), ref["shared_y"], "shared_y")
    if out_dtype == "bf16":
        assert_close_bf16(to_np(r["out"]), ref["out"], "out")
    else:
        assert_close(to_np(r["out"]), ref["out"], "out")


# ------------------------------------------------------------------ tiny layer
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_tiny_layer_parity(orc, out_dtype):
    require_gpu()
    cfg = gen.get("tiny")
    log(f"case tiny T={cfg.T} out={out_dtype}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, out_dtype)
    r = L.staged(wl.x)
    ref = _full_oracle(cfg, orc, gen.x(cfg))
    _compare_full(r, ref, cfg, out_dtype)
    # whole layer == staged, and run-to-run, bit for bit
    out1 = L(wl.x)
    out2 = L(wl.x)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.uint8), r["out"].view(torch.uint8))
    assert torch.equal(out1.view(torch.uint8), out2.view(torch.uint8))
    assert to_np(r["diag"])[1:3].tolist() == [0, 0]


@pytest.mark.parametrize("T", [1, 2, 3, 7, 64, 255, 256, 257, 600])
def test_tiny_ragged_batches(orc, T):
    """Ragged token counts across the permute chunk (256) and the token
    loops of the expert kernels (4 per step)."""
    require_gpu()
    cfg = gen.get("tiny").with_tokens(T)
    log(f"case tiny T={T}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    r = L.staged(wl.x)
    ref = _full_oracle(cfg, orc, gen.x(cfg))
    _compare_full(r, ref, cfg, "f32")


def test_tiny_batch_composition_and_order():
    """A token's output bits do not depend on the rest of the batch: alone,
    as a prefix, shuffled."""
    require_gpu()
    cfg = gen.get("tiny").with_tokens(37)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    full = L(wl.x)
    perm = torch.randperm(37, generator=torch.Generator().manual_seed(1)).to(wl.x.device)
    shuffled = L(wl.x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(shuffled, full[perm])
    for t in (0, 5, 36):
        alone = L(wl.x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(alone[0], full[t]), t
    prefix = L(wl.x[:9].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(prefix, full[:9])


# ------------------------------------------------- matrix-core (MFMA) class
# A shrunken layer with bf16 activations and d % 512 == 0, f % 512 == 0, so
# batches of 32 tokens or more take the grouped-GEMM path.  The token counts
# below select every m-tile height (16 .. 96 rows) of the kernels and every
# count of live 16-row blocks; the skewed variant gives experts several
# m-tiles and leaves others empty.
MED = gen.configs.LayerConfig(name="medium", T=200, d=512, f=512, E=32, k=8, n_shared=2,
                              f_shared=256, x_dtype="bf16", out_dtype="f32", scale_lo=-8,
                              scale_hi=0)


@pytest.mark.parametrize("T,zipf", [(32, None), (100, None), (160, None), (200, None),
                                    (260, None), (600, 1.1), (1000, 1.1)])
def test_mfma_class_parity(orc, T, zipf):
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import PATH_MFMA
    cfg = gen.configs.LayerConfig(**{**MED.__dict__, "T": T, "zipf_s": zipf,
                                     "name": f"medium_T{T}" + ("_zipf" if zipf else "")})
    log(f"case {cfg.name}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    assert L.path_class(T) == PATH_MFMA
    r = L.staged(wl.x)
    ref = _full_oracle(cfg, orc, gen.x(cfg))
    counts = ref["counts"]
    log(f"  pairs/expert max {counts.max()} min {counts.min()}")
    _compare_full(r, ref, cfg, "f32")
    out = L(wl.x)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])


def test_mfma_class_batch_composition():
    """Within the matrix-core class a token's bits do not depend on the rest
    of the batch, its position, or the m-tile height the batch size selects."""
    require_gpu()
    cfg = MED.with_tokens(200)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    full = L(wl.x)
    perm = torch.randperm(200, generator=torch.Generator().manual_seed(3)).to(wl.x.device)
    shuffled = L(wl.x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(shuffled, full[perm])
    for n in (32, 64, 150):   # m-tiles of 16, 32 and 48 rows instead of 64
        part = L(wl.x[:n].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(part, full[:n]), n


def test_shared_tiles_keep_the_bits():
    """The shared experts' matrix-core GEMMs pick their tile shape by batch
    size (64-token tiles with the waves splitting the tokens up to 64 tokens,
    64-token 2 x 2 tiles up to 256, 128-token 2 x 2 tiles up to 640, then
    8-compute-wave down tiles, and from 2048 tokens 256-token gate/up tiles),
    all on one chain per output: a batch's shared outputs equal its prefixes'
    bit for bit."""
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import OP_SHARED_FFN, k3moe_shared_ffn
    cfg = MED.with_tokens(2100)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")

    def shared(n):
        x = wl.x[:n].contiguous()
        shape = L.shape(n, x.dtype)
        y = torch.full((n, cfg.d), float("nan"), dtype=torch.float32, device=x.device)
        k3moe_shared_ffn(shape, L.shared_bank, x, y, L.workspace(shape, OP_SHARED_FFN))
        return y

    full = shared(2100)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(full).all())
    for n in (32, 64, 65, 256, 257, 640, 641, 2047):
        part = shared(n)
        torch.cuda.synchronize()
        log(f"  {n} tokens against the first {n} of 2100")
        assert torch.equal(part, full[:n]), n


def test_router_tiles_keep_the_bits():
    """The fp64 matrix-core router takes 16 x 16 tiles up to 64 tokens, 32 x 16
    up to 256 and 32 x 32 above: the same tokens get the same logits, ids and
    weights, bit for bit, at 64, 65 and 300 tokens."""
    require_gpu()
    cfg = MED.with_tokens(300)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    runs = {n: L.route(wl.x[:n].contiguous(), want_logits=True) for n in (64, 65, 300)}
    torch.cuda.synchronize()
    for n in (64, 65):
        for a, b, what in zip(runs[n], runs[300], ("idx", "w", "logits")):
            assert torch.equal(a, b[:n]), (n, what)


@pytest.mark.parametrize("d,T", [(512, 1), (512, 2), (512, 5), (512, 31), (512, 40),
                                 (3584, 1), (3584, 3)])
def test_scaled_routed_experts_any_batch(orc, d, T):
    """Routed experts on the scaled matrix-core instruction below and above 32
    tokens (one token: the one-token kernels, with 8 down fragments per wave
    at d = 512 and 7 at d = 3584; more: the grouped GEMMs): the layer against
    the oracle, the gate/up half's h (decoded from its documented form)
    against the oracle's h, and gate/up then down equal to the fused call bit
    for bit."""
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import PATH_GEMV, PATH_MFMA
    cfg = gen.configs.LayerConfig(**{**MED.__dict__, "T": T, "d": d,
                                     "name": f"medium_d{d}_T{T}"})
    log(f"case {cfg.name}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    assert L.path_class(T) == (PATH_MFMA if T >= 32 else PATH_GEMV)
    r = L.staged(wl.x)
    x_host = gen.x(cfg)
    ref = _full_oracle(cfg, orc, x_host)
    _compare_full(r, ref, cfg, "f32")
    out = L(wl.x)
    h = L.expert_gateup(wl.x, r["offsets"], r["sorted_pair"])
    y2 = L.expert_down(h, r["offsets"], T)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])
    assert torch.equal(y2, r["y_perm"])
    # h of every pair against the oracle's silu(g) * u
    P = T * cfg.k
    h_gpu = decode_scaled_h(to_np(h).reshape(-1), P, cfg.f)
    bank = gen.routed_bank(cfg)
    sp = ref["sorted_pair"]
    offs = ref["offsets"]
    h_ref = np.zeros((P, cfg.f))
    for e in range(cfg.E):
        if offs[e + 1] > offs[e]:
            toks = sp[offs[e]:offs[e + 1]] // cfg.k
            _, he = orc.mxfp4_ffn({kk: v[e] for kk, v in bank.items()},
                                  oracle.to_f64(x_host[toks]), want_h=True)
            h_ref[offs[e]:offs[e + 1]] = he
    assert_close(h_gpu, h_ref, "h (scaled form)")



@pytest.mark.parametrize("d,f,E,k", [(512, 512, 32, 8), (3584, 1024, 32, 8), (512, 512, 64, 64)])
def test_one_token_ffn_empty_ranks(d, f, E, k):
    """The one-token routed FFN with ranks left empty by a repeated and an
    out-of-range id (the kernels find no expert there and write nothing):
    k3moe_expert_ffn equals gate/up then down bit for bit on the filled
    ranks, with finite values, on two calls in a row with other experts; k up
    to 64 (every expert of E = 64)."""
    require_gpu()
    import dataclasses
    cfg = gen.configs.LayerConfig(**{**MED.__dict__, "T": 1, "d": d, "f": f, "E": E, "k": k,
                                     "name": f"ffn1_d{d}_E{E}_k{k}"})
    log(f"case {cfg.name}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    rng = np.random.default_rng(d + E + k)
    for trial in range(2):
        ids = rng.permutation(E)[:k].astype(np.int32)
        ids[1] = ids[0]        # repeated: dropped
        ids[k - 1] = E + 3     # out of range: dropped
        x = gen.device.activations(dataclasses.replace(cfg, seed=300 + trial))
        idx = torch.from_numpy(ids[None, :].copy()).to("cuda")
        _, offsets, sp, _ = L.permute(idx)
        y = L.expert_ffn(x, offsets, sp)
        h = L.expert_gateup(x, offsets, sp)
        y2 = L.expert_down(h, offsets, 1)
        torch.cuda.synchronize()
        n = int(to_np(offsets)[-1])
        assert n == k - 2, n
        assert torch.isfinite(y[:n]).all(), trial
        assert torch.equal(y[:n], y2[:n]), trial

def _e4m3_rne(v: np.ndarray):
    """OCP E4M3 code of each value rounded to nearest even (|v| <= 448), and
    the value the code stands for; written from the format's definition."""
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    sub = a < 2.0 ** -6
    n = np.round(a * 512.0)                                   # half to even
    e = np.floor(np.log2(np.where(sub, 1.0, a)))
    mant = np.round((a / 2.0 ** e - 1.0) * 8.0)
    e = np.where(mant == 8, e + 1, e)
    mant = np.where(mant == 8, 0, mant)
    code = np.where(sub, n, (e + 7) * 8 + mant).astype(np.int64)
    q = np.where(sub, n / 512.0, (1.0 + mant / 8.0) * 2.0 ** e)
    return code | sign, np.where(np.signbit(v), -q, q)


def test_activation_split_is_exact_rne():
    """The batched gate/up first writes x as 2 E4M3 passes per 128-element
    stage (272-byte records in the workspace): every code and scale byte equals
    the split written out here from its definition (scale so that the block's
    largest magnitude lies in [2^7, 2^8), round to nearest even, remainder
    times 32), and the two passes give back bf16 x exactly for every element
    down to 2^-15 of its block's largest magnitude."""
    require_gpu()
    import ctypes
    from mxfp4_routed_expert_gemv_amd import OP_EXPERT_GATEUP, k3moe_expert_gateup
    cfg = MED.with_tokens(5)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    T, d = cfg.T, cfg.d
    idx, _, _ = L.route(wl.x)
    _, offsets, sp, _ = L.permute(idx)
    s = L.shape(T, wl.x.dtype)
    ws = L.workspace(s, OP_EXPERT_GATEUP)
    h = torch.empty((T * cfg.k, cfg.f), dtype=torch.float32, device=wl.x.device)
    k3moe_expert_gateup(s, L.routed_bank, wl.x, offsets, sp, h, ws, None)
    torch.cuda.synchronize()
    xq = to_np(ws)[:T * (d // 128) * 272].reshape(T, d // 128, 272)
    xb = to_np(wl.x.view(torch.int16)).astype(np.int64) & 0xFFFF
    bits = (xb << 16).astype(np.uint32)
    x64 = bits.view(np.float32).astype(np.float64).reshape(T, d // 32, 32)
    mb = (bits & 0x7FFFFFFF).reshape(T, d // 32, 32).max(axis=2).astype(np.int64)
    sb0 = np.maximum((mb >> 23) - 7, 5)
    v = x64 * 2.0 ** (127 - sb0)[..., None]
    v0 = v.copy()
    back = np.zeros_like(v)
    for p in range(2):
        code, q = _e4m3_rne(v)
        got = xq[:, :, 128 * p:128 * (p + 1)].reshape(T, d // 32, 32)
        assert np.array_equal(got, code), f"pass {p} codes"
        back += q * 2.0 ** (-5 * p)
        v = (v - q) * 32.0
    scales = xq[:, :, 256:264].reshape(T, d // 128, 2, 4).astype(np.int64)
    want = np.stack([sb0.reshape(T, d // 128, 4) - 5 * p for p in range(2)], axis=2)
    assert np.array_equal(scales, want), "scale bytes"
    assert np.all(xq[:, :, 264:272] == 0)
    # exact down to 2^-7 in the scaled units (2^-15 of the block's largest
    # magnitude); below, within half the second pass's finest step
    err = np.abs(back - v0)
    assert np.all(err[np.abs(v0) >= 2.0 ** -7] == 0), "2 passes are not exact"
    assert np.all(err <= 2.0 ** -15)


def test_routed_bits_do_not_depend_on_batch_size():
    """A token's routed expert outputs are the same bits alone (one-token
    kernels), in small batches (grouped GEMMs, GEMV class) and in large ones
    (matrix-core class)."""
    require_gpu()
    cfg = MED.with_tokens(200)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    full = L.staged(wl.x)

    def rows(r, t):
        pp = to_np(r["pair_pos"])
        return to_np(r["y_perm"])[pp[t * cfg.k:(t + 1) * cfg.k]]
    for n in (1, 2, 7, 31, 64):
        part = L.staged(wl.x[:n].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(to_np(part["idx"]), to_np(full["idx"])[:n])
        for t in range(n):
            assert np.array_equal(rows(part, t), rows(full, t)), (n, t)
    for t in (5, 77, 199):   # single tokens from inside the batch
        one = L.staged(wl.x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(rows(one, 0), rows(full, t)), t


def test_hand_worked_two_experts(orc):
    """The closed-form 1-token / 2-expert layer (hand-worked fixture), both
    nibble positions, through the C ABI."""
    require_gpu()
    import oracle_pins
    from conftest import golden
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    g = golden("hand_two_experts.json")
    for col in g["columns"]:
        x, wr, experts = oracle_pins._hand_case(col)
        dev = "cuda"
        routed = {k: torch.from_numpy(np.stack([e[k] for e in experts])).to(dev)
                  for k in experts[0]}
        L = MoELayer(torch.from_numpy(wr.view(np.int16)).to(dev).view(torch.bfloat16), routed, {},
                     k=2, out_dtype=torch.float32)
        r = L.staged(torch.from_numpy(x).to(dev))
        out = to_np(r["out"])
        assert np.array_equal(to_np(r["idx"]), [[0, 1]])
        assert np.allclose(out, g["out"], rtol=1e-5, atol=0), (col, out[0, :4])


def test_edge_ids_and_empty_batch():
    """Permute drops ids outside [0, E) and repeated ids (counted in diag,
    position -1); an empty batch is a no-op."""
    require_gpu()
    cfg = gen.get("tiny")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    idx = torch.tensor([[0, 3, 5, 7], [2, 2, 9, 40], [15, -1, 1, 0]], dtype=torch.int32,
                       device="cuda")
    diag = torch.zeros(4, dtype=torch.int32, device="cuda")
    counts, offsets, sp, pp = L.permute(idx, diag=diag)
    torch.cuda.synchronize()
    assert to_np(diag)[2] == 3
    ppn = to_np(pp)
    assert ppn[5] == -1 and ppn[7] == -1 and ppn[9] == -1 and ppn[4] >= 0
    valid = [(p, e) for p, e in enumerate(idx.cpu().numpy().ravel()) if ppn[p] >= 0]
    assert to_np(offsets)[-1] == len(valid) == 9
    order = sorted(valid, key=lambda pe: (pe[1], pe[0]))
    assert to_np(sp)[:9].tolist() == [p for p, _ in order]
    assert to_np(sp)[9:].tolist() == [-1, -1, -1]
    empty = L(wl.x[:0])
    assert empty.shape == (0, cfg.d)


def test_k_equals_E_and_k_one(orc):
    require_gpu()
    base = gen.get("tiny")
    for k in (1, base.E):
        cfg = gen.configs.LayerConfig(**{**base.__dict__, "k": k, "name": f"tiny_k{k}"})
        wl = gen.device.build(cfg)
        L = k3layer(wl, "f32")
        r = L.staged(wl.x)
        ref = _full_oracle(cfg, orc, gen.x(cfg))
        _compare_full(r, ref, cfg, "f32")


@pytest.mark.parametrize("E,k,T", [(96, 24, 300), (40, 16, 700), (64, 64, 70)])
def test_wide_routing_chunked_permute(orc, E, k, T):
    """More experts per token than the decode shapes: exercises both chunk
    sizes of the large-batch permute (256 tokens for k <= 16, 64 above)."""
    require_gpu()
    base = gen.get("tiny")
    cfg = gen.configs.LayerConfig(**{**base.__dict__, "E": E, "k": k, "T": T,
                                     "name": f"tiny_E{E}_k{k}_T{T}"})
    log(f"case {cfg.name}")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    r = L.staged(wl.x)
    ref = _full_oracle(cfg, orc, gen.x(cfg))
    _compare_full(r, ref, cfg, "f32")


def test_zero_weight_expert_contributes_nothing(orc):
    """An expert whose routing weight underflows to 0 is skipped, even with
    NaN weights (scale byte 255)."""
    require_gpu()
    cfg = gen.get("tiny")
    x = gen.x(cfg).copy()
    x[:, 0] = 1.0
    wr = gen.router(cfg).copy()
    wr[:, 0] = 0
    wr[3, 0] = gen.f64_to_bf16_bits(2000.0)
    wr[9, 0] = gen.f64_to_bf16_bits(1000.0)
    bank = gen.routed_bank(cfg)
    bank["w2_scale"][9] = 255
    bank["w13_scale"][9] = 255
    sh = gen.shared_bank(cfg)
    ref = orc.layer(x, wr, lambda e: {k: v[e] for k, v in bank.items()}, sh, cfg.k, cfg.E)
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    dev = "cuda"
    L = MoELayer(torch.from_numpy(wr.view(np.int16)).to(dev).view(torch.bfloat16),
                 {k: torch.from_numpy(v).to(dev) for k, v in bank.items()},
                 {k: torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
                  for k, v in sh.items()}, cfg.k, out_dtype=torch.float32)
    r = L.staged(torch.from_numpy(x).to(dev))
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    out = to_np(r["out"])
    assert np.all(np.isfinite(out))
    assert_close(out, ref["out"], "out with a NaN expert at weight 0")


@pytest.mark.parametrize("T", [1, 40])
def test_scaled_nan_expert_at_weight_zero(orc, T):
    """On the scaled path (one-token kernels at T = 1, grouped GEMMs at 40) an
    expert with NaN scales (byte 255) whose routing weight underflows to 0
    leaves every output finite and equal to the oracle's."""
    require_gpu()
    cfg = MED.with_tokens(T)
    x = gen.x(cfg).copy()
    x[:, 0] = gen.f64_to_bf16_bits(1.0)
    wr = gen.router(cfg).copy()
    wr[:, 0] = 0
    wr[3, 0] = gen.f64_to_bf16_bits(2000.0)
    wr[9, 0] = gen.f64_to_bf16_bits(1000.0)
    bank = gen.routed_bank(cfg)
    bank["w2_scale"][9] = 255
    bank["w13_scale"][9] = 255
    sh = gen.shared_bank(cfg)
    ref = orc.layer(oracle.to_f64(x), wr, lambda e: {k: v[e] for k, v in bank.items()}, sh,
                    cfg.k, cfg.E)
    assert np.all(ref["counts"][[3, 9]] == T)   # both experts chosen by every token
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    dev = "cuda"
    L = MoELayer(torch.from_numpy(wr.view(np.int16)).to(dev).view(torch.bfloat16),
                 {k: torch.from_numpy(v).to(dev) for k, v in bank.items()},
                 {k: torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
                  for k, v in sh.items()}, cfg.k, out_dtype=torch.float32)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    r = L.staged(xd)
    out = L(xd)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(r["idx"]), ref["idx"])
    y = to_np(r["y_perm"])
    o9 = ref["offsets"]
    assert np.all(np.isnan(y[o9[9]:o9[10]])), "the NaN expert's own rows are NaN"
    assert np.all(np.isfinite(to_np(out)))
    assert torch.equal(out, r["out"])
    assert_close(to_np(out), ref["out"], "out with a NaN expert at weight 0")


def test_scaled_nonfinite_activation_stays_in_its_token():
    """An infinite activation element on the scaled path turns its block's
    codes into E4M3 NaN: the token's own routed rows become NaN, and every
    other token's outputs keep their bits."""
    require_gpu()
    cfg = MED.with_tokens(40)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    base = L.staged(wl.x)
    x = wl.x.clone()
    x[7, 100] = float("inf")
    r = L.staged(x)
    torch.cuda.synchronize()
    k = cfg.k
    pp = to_np(r["pair_pos"])
    y = to_np(r["y_perm"])
    assert np.all(~np.isfinite(y[pp[7 * k:8 * k]])), "token 7's routed rows"
    others = np.array([t for t in range(cfg.T) if t != 7])
    assert np.array_equal(to_np(r["out"])[others], to_np(base["out"])[others])
    # the same token alone (one-token kernels)
    one = L.staged(x[7:8].contiguous())
    torch.cuda.synchronize()
    assert np.all(~np.isfinite(to_np(one["y_perm"])))


def test_nonfinite_logits_are_counted():
    require_gpu()
    cfg = gen.get("tiny")
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    x = wl.x.clone()
    x[1, 5] = float("inf")
    diag = torch.zeros(4, dtype=torch.int32, device="cuda")
    L.route(x, diag=diag)
    torch.cuda.synchronize()
    assert to_np(diag)[1] > 0


def test_nonfinite_logits_bf16_route():
    """From 512 tokens the matrix-core class routes on bf16 logits: a token
    with an infinite activation has every expert re-evaluated in fp64 (its
    logits are not finite and are counted), and every other token keeps the
    ids of the clean batch."""
    require_gpu()
    cfg = MED.with_tokens(600)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    clean, _, _ = L.route(wl.x)
    x = wl.x.clone()
    x[1, 5] = float("inf")
    diag = torch.zeros(4, dtype=torch.int32, device="cuda")
    idx, _, _ = L.route(x, diag=diag)
    torch.cuda.synchronize()
    assert to_np(diag)[1] > 0
    others = np.array([t for t in range(cfg.T) if t != 1])
    assert np.array_equal(to_np(idx)[others], to_np(clean)[others])


def test_device_generator_matches_host():
    """The device fill of the routed bank equals the host generator byte for
    byte (sampled experts of the full-size bank)."""
    require_gpu()
    cfg = gen.get("decode_b1")
    sz = gen.routed_sizes(cfg)
    for e in (0, 447, 895):
        host = gen.routed_expert(cfg, e)
        for name, n in sz.items():
            buf = torch.empty(n, dtype=torch.uint8, device="cuda")
            kk = gen.key(cfg.seed, gen._routed_streams(cfg)[name])
            lib = gen._load_dev()
            if name.endswith("scale"):
                rc = lib.k3gen_dev_scales(kk, e * n, n, cfg.scale_lo, cfg.scale_hi, buf.data_ptr(), 0)
            else:
                rc = lib.k3gen_dev_bytes(kk, e * n, n, buf.data_ptr(), 0)
            assert rc == 0
            torch.cuda.synchronize()
            assert np.array_equal(buf.cpu().numpy(), host[name].ravel()), (e, name)


# ------------------------------------------------------------- full-size layer
def _mtile_rows(cfg) -> int:
    """Rows per m-tile of the routed grouped GEMMs at this batch: 16 per
    block, blocks from the expected pairs per expert with 15% headroom, at
    most 6 (the launch rule of the scaled grouped GEMMs)."""
    ppe = cfg.T * cfg.k / cfg.E * 1.15
    return 16 * max(1, min(6, int((ppe + 15.0) / 16.0)))


def _check_whole_experts(r, cfg, orc, x_host, counts, offsets, sp):
    """y_perm of whole m-tiles against the oracle: the expert with the fewest
    pairs (a tail tile), an expert spanning two m-tiles, and the first and
    last m-tiles of the hottest expert (the ragged last one included)."""
    bm = _mtile_rows(cfg)
    live = np.nonzero(counts)[0]
    tail = int(live[np.argmin(counts[live])])
    two = [e for e in live if bm < counts[e] <= 2 * bm]
    hot = int(np.argmax(counts))
    ranges = [(tail, offsets[tail], offsets[tail + 1])]
    if two:
        e2 = int(max(two, key=lambda e: counts[e]))
        ranges.append((e2, offsets[e2], offsets[e2 + 1]))
    if counts[hot] > 2 * bm:
        last0 = offsets[hot] + (counts[hot] - 1) // bm * bm
        ranges += [(hot, offsets[hot], offsets[hot] + bm), (hot, last0, offsets[hot + 1])]
    y_gpu = to_np(r["y_perm"])
    for e, lo, hi in ranges:
        toks = sp[lo:hi] // cfg.k
        want = orc.mxfp4_ffn(gen.routed_expert(cfg, e), oracle.to_f64(x_host[toks]))
        assert_close(y_gpu[lo:hi], want,
                     f"y_perm expert {e} rows {lo - offsets[e]}..{hi - offsets[e]} of {counts[e]}")


def _run_big(big, cfg, orc, n_sample, whole_experts=False):
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    x_host = gen.x(cfg)
    x = gen.device.activations(cfg)
    wr_host = gen.router(cfg)
    wr = gen.device._to_dev_bf16(wr_host, "cuda") if cfg.zipf_s is not None else big.w_router
    L = MoELayer(wr, big.routed, big.shared, cfg.k, out_dtype=torch.bfloat16)
    log(f"case {cfg.name}: T={cfg.T} path={L.path_class(cfg.T)}")
    r = L.staged(x)
    out_layer = L(x)
    torch.cuda.synchronize()
    assert torch.equal(out_layer.view(torch.int16), r["out"].view(torch.int16))
    log(f"  diag = {to_np(r['diag']).tolist()}")
    assert to_np(r["diag"])[1:3].tolist() == [0, 0]

    # routing: every token's ids against the oracle, bit for bit
    logits, idx, w = orc.route(oracle.to_f64(x_host), wr_host, cfg.k)
    g_idx = to_np(r["idx"])
    assert np.array_equal(g_idx, idx), f"{int(np.sum(np.any(g_idx != idx, axis=1)))} tokens differ"
    assert np.max(np.abs(to_np(r["w"]) - w)) <= W_TOL
    assert_close(to_np(r["logits"]), logits, "logits")
    counts, offsets, sp, pp = orc.permute(idx, cfg.E)
    assert np.array_equal(to_np(r["counts"]), counts)
    assert np.array_equal(to_np(r["offsets"]), offsets)
    assert np.array_equal(to_np(r["sorted_pair"]), sp)
    assert np.array_equal(to_np(r["pair_pos"]), pp)
    nz = counts[counts > 0]
    log(f"  experts touched {nz.size}, pairs/expert max {nz.max()} min {nz.min()}")

    # values: sampled tokens, every stage, against the oracle; the layer's
    # fp32 output (before any rounding to bf16) under the strict bar
    toks = sample_tokens(cfg.T, n_sample)
    out_ref, sh_ref, y_ref = orc.token_outputs(x_host[toks], idx[toks], w[toks],
                                               oracle_expert(cfg), gen.shared_bank(cfg))
    y_gpu = to_np(r["y_perm"])
    pp_g = to_np(r["pair_pos"])
    y_rows = np.stack([y_gpu[pp_g[t * cfg.k:(t + 1) * cfg.k]] for t in toks])
    assert_close(y_rows.reshape(-1, cfg.d), y_ref.reshape(-1, cfg.d), "y_perm (sampled)")
    assert_close(to_np(r["shared_y"])[toks], sh_ref, "shared_y (sampled)")
    assert_close_bf16(to_np(r["out"])[toks], out_ref, "out (sampled)")
    out32 = L(x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(to_np(out32)[toks], out_ref, "out fp32 (sampled)")
    if whole_experts:
        _check_whole_experts(r, cfg, orc, x_host, counts, offsets, sp)
    return r, L, x


def test_decode_b1(big, orc):
    _run_big(big, gen.get("decode_b1"), orc, 1)


def test_decode_layer_in_a_graph(big):
    """The one-token layer records into a graph (no memset, copy, allocation
    or host synchronisation inside the library): every replay, with eager
    layers run between replays, equals the eager result bit for bit."""
    import dataclasses
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    cfg = gen.get("decode_b1")
    L = MoELayer(big.w_router, big.routed, big.shared, cfg.k, out_dtype=torch.bfloat16)
    xs = [gen.device.activations(dataclasses.replace(cfg, seed=200 + i)) for i in range(3)]
    eager = [L(x) for x in xs]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for x in xs:
            L(x)
    torch.cuda.current_stream().wait_stream(side)
    graphs, outs = [], []
    for x in xs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            outs.append(L(x))
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, g in enumerate(graphs):
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(outs[i].view(torch.int16), eager[i].view(torch.int16)), (rep, i)
            L(xs[(i + 1) % 3])
            torch.cuda.synchronize()


def test_decode_b64(big, orc):
    r, L, x = _run_big(big, gen.get("decode_b64"), orc, 16)
    # batch composition inside the matrix-core class: the first 32 tokens
    # alone equal the same tokens of the batch of 64, bit for bit
    part = L(x[:32].contiguous())
    full = L(x)
    torch.cuda.synchronize()
    assert torch.equal(part.view(torch.int16), full[:32].view(torch.int16))
    # a ragged batch in the small-batch shared-expert regime: the first 50
    # tokens alone equal their rows of the batch of 64, bit for bit
    part50 = L(x[:50].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(part50.view(torch.int16), full[:50].view(torch.int16))
    # the routed outputs of single tokens (one-token kernels) equal their rows
    # of the batch (grouped GEMMs), bit for bit
    k = gen.get("decode_b64").k
    pp = to_np(r["pair_pos"])
    y = to_np(r["y_perm"])
    for t in (0, 63):
        one = L.staged(x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(to_np(one["idx"])[0], to_np(r["idx"])[t])
        assert np.array_equal(to_np(one["y_perm"]), y[pp[t * k:(t + 1) * k]]), t


def test_prefill_4096(big, orc):
    _run_big(big, gen.get("prefill_4096"), orc, 8, whole_experts=True)


@pytest.mark.parametrize("T", [8, 33, 1025, 4095])
def test_full_size_other_batches(big, orc, T):
    """Full size at 8 tokens (the vector-ALU router and shared experts beside
    the scaled grouped GEMMs), 33 (16 x 16 router tiles, the small-batch
    shared kernels with a ragged token count), 1025 (48-row grouped tiles,
    128-token shared tiles, 32 x 32 router tiles) and 4095 (ragged 96-row
    tiles): full oracle routing and permutation, and the values of sampled
    tokens."""
    _run_big(big, gen.get("prefill_4096").with_tokens(T), orc, 3)


def test_prefill_16384_zipf(big, orc):
    r, _, _ = _run_big(big, gen.get("prefill_16384_zipf"), orc, 8, whole_experts=True)
    counts = to_np(r["counts"])
    srt = np.sort(counts)
    gini = 1 - 2 * np.sum(np.cumsum(srt) / srt.sum()) / srt.size + 1 / srt.size
    log(f"  zipf histogram: max {counts.max()} min {counts.min()} gini {gini:.3f}")
    assert counts.max() > 1000


@pytest.mark.parametrize("name,T", [("tiny", 4), ("medium", 40), ("medium", 1)])
def test_expert_ffn_shared_mode(orc, name, T):
    """k3moe_expert_ffn with a BF16 bank and no sorted pairs is the shared
    experts' FFN (every token through every expert, summed in bank order):
    equal to k3moe_shared_ffn bit for bit, and to the oracle."""
    require_gpu()
    from mxfp4_routed_expert_gemv_amd import OP_SHARED_FFN, k3moe_expert_ffn
    cfg = (gen.get("tiny") if name == "tiny" else MED).with_tokens(T)
    wl = gen.device.build(cfg)
    L = k3layer(wl, "f32")
    want = L.shared_ffn(wl.x)
    s = L.shape(T, wl.x.dtype)
    y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    k3moe_expert_ffn(s, L.shared_bank, wl.x, None, None, y, L.workspace(s, OP_SHARED_FFN))
    torch.cuda.synchronize()
    assert torch.equal(y, want)
    ref = orc.shared_ffn(gen.shared_bank(cfg), oracle.to_f64(gen.x(cfg)))
    assert_close(to_np(y), ref, "shared mode")
