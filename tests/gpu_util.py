"""Helpers of the GPU parity tests: device workloads, oracle expectations and
the comparison bars.

Bars (written here once, used by every GPU test):
  - integers (expert ids, counts, offsets, sorted pairs, positions): equal;
  - fp32 tensors: max |gpu - oracle| <= 2e-3 * RMS(oracle) over the tensor;
  - bf16 outputs: compared with the oracle value, allowing 2e-3 * RMS plus
    one bf16 ulp of the element (the output rounding itself);
  - routing weights: |gpu - oracle| <= 2e-6 (fp32 storage of values in [0, 1]).
"""
import math
import sys

import numpy as np
import torch

import gen
import gen.device
import oracle

BAR = 2e-3
W_TOL = 2e-6


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16) \
            .view(np.float32).astype(np.float64)
    return t.cpu().numpy()


def rms(a: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def assert_close(got: np.ndarray, want: np.ndarray, name: str, scale: float = None):
    scale = rms(want) if scale is None else scale
    err = float(np.max(np.abs(got.astype(np.float64) - want))) if want.size else 0.0
    log(f"  {name}: max|err| = {err:.3e}, RMS = {scale:.3e}, ratio = {err / max(scale, 1e-300):.2e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= BAR * scale, f"{name}: max|err| {err:.3e} > {BAR} * RMS {scale:.3e}"


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1e-38)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))


def assert_close_bf16(got: np.ndarray, want: np.ndarray, name: str, scale: float = None):
    scale = rms(want) if scale is None else scale
    allow = BAR * scale + ulp_bf16(want)
    err = np.abs(got - want)
    log(f"  {name} (bf16): max|err| = {err.max():.3e}, RMS = {scale:.3e}")
    assert np.all(err <= allow), f"{name}: {int(np.sum(err > allow))} elements beyond the bf16 bar"


def oracle_expert(cfg):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = gen.routed_expert(cfg, e)
        return cache[e]
    return get


def k3layer(wl: gen.device.DeviceWorkload, out_dtype=None):
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype or wl.cfg.out_dtype]
    return MoELayer(wl.w_router, wl.routed, wl.shared, wl.cfg.k, out_dtype=dt)


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = set([0, T - 1])
    while len(s) < n:
        s.add(int(rng.integers(0, T)))
    return np.array(sorted(s))


def check_permutation_properties(idx: np.ndarray, counts, offsets, sp, pp, E: int):
    """Properties that fix the permutation of any id matrix: counts are the
    histogram, offsets its exclusive scan, sorted pairs the stable argsort,
    pair_pos the inverse."""
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(sp, order)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(pp, inv)


def float_ok(x):
    return x is not None and math.isfinite(x)


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 (FN) code -> value: bias 7, subnormals m/8 * 2^-6, 0x7F/0xFF NaN."""
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def decode_scaled_h(buf: np.ndarray, rows: int, f: int) -> np.ndarray:
    """The gate/up buffer in its scaled form (rows of f/128 stages of 400
    bytes: 3 passes of 128 E4M3 codes, then byte 4p + b = E8M0 scale of pass p,
    32-feature block b) -> fp64 values [rows][f]."""
    st = buf.view(np.uint8)[:rows * (f // 128) * 400].reshape(rows, f // 128, 400)
    out = np.zeros((rows, f // 128, 128))
    for p in range(3):
        sc = st[:, :, 384 + 4 * p:388 + 4 * p].astype(np.float64)          # [rows][stages][4]
        out += e4m3_value(st[:, :, 128 * p:128 * (p + 1)]) * np.repeat(2.0 ** (sc - 127), 32, axis=2)
    return out.reshape(rows, f)
