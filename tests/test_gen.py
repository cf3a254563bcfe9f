"""The seeded input generator: determinism, regeneration of any slice alone,
value distributions of the five workloads, and the skewed-routing targets."""
import math

import numpy as np

import gen


def test_stream_is_splitmix64():
    # SplitMix64 reference values: state 0 advanced by the golden gamma once
    # gives 0xE220A8397B1DCDAF (Vigna's splitmix64.c with x = 0).
    assert gen.draw(0, 0) == 0xE220A8397B1DCDAF


def test_regeneration_matches_full_bank():
    c = gen.get("tiny")
    bank = gen.routed_bank(c)
    for e in (0, 7, 15):
        ex = gen.routed_expert(c, e)
        for k in bank:
            assert np.array_equal(ex[k], bank[k][e])


def test_deterministic_and_prefix_property():
    c1, c2 = gen.get("decode_b1"), gen.get("decode_b64")
    a = gen.x(c2)
    assert np.array_equal(gen.x(c1)[0], a[0])
    assert np.array_equal(gen.x(c2, 10, 12), a[10:12])
    assert np.array_equal(gen.router(c1), gen.router(c2))


def test_distributions_tiny():
    c = gen.get("tiny")
    x = gen.x(c)
    assert x.dtype == np.float32 and x.shape == (4, 256)
    assert abs(x.mean()) < 0.15 and 0.85 < x.std() < 1.15
    wr = (gen.router(c).astype(np.uint32) << 16).view(np.float32)
    assert 0.018 < wr.std() < 0.022
    bank = gen.routed_bank(c)
    s = np.concatenate([bank["w13_scale"].ravel(), bank["w2_scale"].ravel()])
    assert s.min() == 127 - 8 and s.max() == 127
    codes = np.concatenate([bank["w13"].ravel() & 15, bank["w13"].ravel() >> 4])
    hist = np.bincount(codes, minlength=16)
    assert hist.min() > 0.9 * hist.mean() and hist.max() < 1.1 * hist.mean()


def test_big_scale_range():
    c = gen.get("decode_b1")
    ex = gen.routed_expert(c, 123)
    assert ex["w13"].shape == (4096, 3584) and ex["w13_scale"].shape == (4096, 224)
    assert ex["w2"].shape == (7168, 1024) and ex["w2_scale"].shape == (7168, 64)
    s = ex["w13_scale"]
    assert s.min() == 117 and s.max() == 125


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even (1.0)
    assert gen.f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80
    assert gen.f64_to_bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82   # tie -> even 1 + 2^-6
    assert gen.f64_to_bf16_bits(-2.0) == 0xC000


def test_zipf_targets():
    c = gen.get("prefill_16384_zipf")
    n = gen.zipf_target_counts(c)
    assert abs(n.sum() - c.T * c.k) < 1e-6 * c.T * c.k
    assert n.max() == c.T and np.all(np.diff(n) <= 0)
    r = gen.zipf_ranking(c)
    assert sorted(r.tolist()) == list(range(c.E))
    b = gen.zipf_bias(c)
    assert np.all(np.diff(b[r]) <= 0)            # bias falls with rank
    x = gen.x(c, 0, 2)
    assert np.all(x[:, c.d - 1] == gen.BF16_ONE)
    sigma_l = c.router_sigma * math.sqrt(c.d - 1)
    assert b.max() > 4 * sigma_l
