"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This package only makes input bytes; it holds none of the layer's arithmetic.
Every tensor is a pure function of (seed, tensor id, element index) through the
counter-based stream documented in csrc/k3gen.h, so any expert can be
regenerated alone on the host (for the oracle) or filled in place in device
memory (for the HIP path).

Tensors (all row-major):
  x         [T][d]          fp32 (tiny) or bf16 bits, N(0, 1)
  w_router  [E][d]          bf16 bits, N(0, router_sigma)
  w13       [E][2f][d/2]    packed E2M1 codes; rows 0..f-1 gate, f..2f-1 up
  w13_scale [E][2f][d/32]   E8M0 bytes, 127 + U{scale_lo..scale_hi}
  w2        [E][d][f/2]     packed E2M1 codes
  w2_scale  [E][d][f/32]    E8M0 bytes
  shared w13 [S][2f_s][d], shared w2 [S][d][f_s]  bf16 bits, N(0, shared_sigma)
  router_bias [E]           fp32, N(0, 0.05) (the sigmoid router's selection bias)
Byte i of a packed row holds element 2i in its low nibble and 2i+1 in its high
nibble; each 32-element block shares one scale byte.

Skewed routing (zipf_s set): a constant bias channel x[:, d-1] = 1 with
w_router[e, d-1] = b_e, where b_e comes from a closed-form threshold model so
that expert e's share of the token-expert pairs follows rank^-s over a seeded
random ranking, capped at T pairs per expert.  The realized histogram is
whatever the router then produces; it is measured, not assumed.
"""
import ctypes
import math
import os

import numpy as np

from .configs import CONFIGS, ORDER, LayerConfig, get  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))

(T_X, T_ROUTER, T_W13, T_W13S, T_W2, T_W2S, T_SH13, T_SH2, T_ZIPF, T_RBIAS, T_RVQ13, T_RVQ2,
 T_RVQCB13, T_RVQCB2) = range(1, 15)

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        from . import build as _b
        if not os.path.exists(_b.HOST_LIB):
            _b.build_host()
        lib = ctypes.CDLL(_b.HOST_LIB)
        u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        lib.k3gen_key.restype = u64
        lib.k3gen_key.argtypes = [u64, u64]
        lib.k3gen_draw.restype = u64
        lib.k3gen_draw.argtypes = [u64, u64]
        lib.k3gen_bytes.argtypes = [u64, u64, u64, vp]
        lib.k3gen_scales.argtypes = [u64, u64, u64, i32, i32, vp]
        lib.k3gen_normal_bf16.argtypes = [u64, u64, u64, ctypes.c_double, vp]
        lib.k3gen_normal_f32.argtypes = [u64, u64, u64, ctypes.c_double, vp]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (bind to the HIP runtime torch loaded; see the binding)
        from . import build as _b
        if not os.path.exists(_b.DEV_LIB):
            raise RuntimeError(f"{_b.DEV_LIB} is not built; run gen.build.build()")
        lib = ctypes.CDLL(_b.DEV_LIB)
        u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        lib.k3gen_dev_bytes.restype = i32
        lib.k3gen_dev_bytes.argtypes = [u64, u64, u64, vp, vp]
        lib.k3gen_dev_scales.restype = i32
        lib.k3gen_dev_scales.argtypes = [u64, u64, u64, i32, i32, vp, vp]
        _dev = lib
    return _dev


def key(seed: int, tensor_id: int) -> int:
    return _load_host().k3gen_key(seed, tensor_id)


def draw(k: int, i: int) -> int:
    return _load_host().k3gen_draw(k, i)


def _bytes(k, start, n):
    out = np.empty(n, dtype=np.uint8)
    if n:
        _load_host().k3gen_bytes(k, start, n, out.ctypes.data)
    return out


def _scales(k, start, n, lo, hi):
    out = np.empty(n, dtype=np.uint8)
    if n:
        _load_host().k3gen_scales(k, start, n, lo, hi, out.ctypes.data)
    return out


def _normal_bf16(k, start, n, sigma):
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load_host().k3gen_normal_bf16(k, start, n, sigma, out.ctypes.data)
    return out


def _normal_f32(k, start, n, sigma):
    out = np.empty(n, dtype=np.float32)
    if n:
        _load_host().k3gen_normal_f32(k, start, n, sigma, out.ctypes.data)
    return out


BF16_ONE = 0x3F80


def f64_to_bf16_bits(v: float) -> int:
    """Round one fp64 value to bf16 bits, nearest-even (normal range)."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    m, e = math.frexp(v)
    q = math.ldexp(round(math.ldexp(m, 8)), e - 8)   # Python round() is half-even
    return int(np.array([q], dtype=np.float32).view(np.uint32)[0] >> 16)


# ----------------------------------------------------------------- activations
def x(cfg: LayerConfig, t0: int = 0, t1: int = None) -> np.ndarray:
    """Tokens t0..t1-1 of the activation matrix; token t is the same vector in
    every workload that shares cfg's seed and d (a prefix of a bigger batch)."""
    t1 = cfg.T if t1 is None else t1
    n = (t1 - t0) * cfg.d
    kx = key(cfg.seed, T_X)
    if cfg.x_dtype == "f32":
        a = _normal_f32(kx, t0 * cfg.d, n, 1.0).reshape(t1 - t0, cfg.d)
        if cfg.zipf_s is not None:
            a[:, cfg.d - 1] = 1.0
        return a
    a = _normal_bf16(kx, t0 * cfg.d, n, 1.0).reshape(t1 - t0, cfg.d)
    if cfg.zipf_s is not None:
        a[:, cfg.d - 1] = BF16_ONE
    return a


# ---------------------------------------------------------------------- router
def zipf_ranking(cfg: LayerConfig) -> np.ndarray:
    """Seeded random permutation: ranking[r] = expert id of popularity rank r."""
    kz = key(cfg.seed, T_ZIPF)
    perm = np.arange(cfg.E, dtype=np.int64)
    for i in range(cfg.E - 1, 0, -1):           # Fisher-Yates, draw i
        j = ((draw(kz, i) >> 32) * (i + 1)) >> 32
        perm[i], perm[j] = perm[j], perm[i]
    return perm


def zipf_target_counts(cfg: LayerConfig) -> np.ndarray:
    """Pairs per popularity rank: min(T, c r^-s) with c chosen so they sum to T k."""
    r = np.arange(1, cfg.E + 1, dtype=np.float64)
    base = r ** (-cfg.zipf_s)
    lo, hi = 0.0, float(cfg.T * cfg.k) * 10
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(cfg.T, c * base).sum() < cfg.T * cfg.k:
            lo = c
        else:
            hi = c
    return np.minimum(cfg.T, hi * base)


def zipf_bias(cfg: LayerConfig) -> np.ndarray:
    """Per-expert bias b_e (fp64) of the threshold model: expert e is chosen when
    its unbiased logit z_e ~ N(0, sigma_l^2) plus b_e exceeds 0, so
    P(chosen) = Phi(b_e / sigma_l) is set to target_pairs / T."""
    from scipy.special import ndtri
    sigma_l = cfg.router_sigma * math.sqrt(cfg.d - 1)
    p = np.clip(zipf_target_counts(cfg) / cfg.T, 1e-9, 1.0 - 1e-6)
    b_rank = sigma_l * ndtri(p)
    b = np.empty(cfg.E, dtype=np.float64)
    b[zipf_ranking(cfg)] = b_rank
    return b


def router(cfg: LayerConfig) -> np.ndarray:
    """w_router [E][d] as bf16 bits."""
    w = _normal_bf16(key(cfg.seed, T_ROUTER), 0, cfg.E * cfg.d, cfg.router_sigma)
    w = w.reshape(cfg.E, cfg.d)
    if cfg.zipf_s is not None:
        b = zipf_bias(cfg)
        w[:, cfg.d - 1] = np.array([f64_to_bf16_bits(v) for v in b], dtype=np.uint16)
    return w


def router_bias(cfg: LayerConfig, sigma: float = 0.05) -> np.ndarray:
    """Per-expert selection bias [E] fp32, N(0, sigma), for the sigmoid router
    (the pages give no distribution for it)."""
    return _normal_f32(key(cfg.seed, T_RBIAS), 0, cfg.E, sigma)


# --------------------------------------------------------------- routed experts
def routed_sizes(cfg: LayerConfig) -> dict:
    """Bytes per expert of each routed tensor."""
    return dict(w13=2 * cfg.f * cfg.d // 2, w13_scale=2 * cfg.f * cfg.d // 32,
                w2=cfg.d * cfg.f // 2, w2_scale=cfg.d * cfg.f // 32)


def _routed_streams(cfg):
    return dict(w13=T_W13, w13_scale=T_W13S, w2=T_W2, w2_scale=T_W2S)


def routed_expert(cfg: LayerConfig, e: int) -> dict:
    """Expert e's packed tensors, regenerated on the host."""
    return routed_experts(cfg, e, e + 1, squeeze=True)


def routed_experts(cfg: LayerConfig, e0: int, e1: int, squeeze: bool = False) -> dict:
    sz = routed_sizes(cfg)
    out = {}
    for name, tid in _routed_streams(cfg).items():
        kk = key(cfg.seed, tid)
        n = sz[name]
        if name.endswith("scale"):
            a = _scales(kk, e0 * n, (e1 - e0) * n, cfg.scale_lo, cfg.scale_hi)
        else:
            a = _bytes(kk, e0 * n, (e1 - e0) * n)
        rows = 2 * cfg.f if name.startswith("w13") else cfg.d
        a = a.reshape(e1 - e0, rows, -1)
        out[name] = a[0] if squeeze else a
    return out


def routed_bank(cfg: LayerConfig) -> dict:
    """All E experts on the host: w13 [E][2f][d/2], w13_scale [E][2f][d/32], ..."""
    return routed_experts(cfg, 0, cfg.E)


def fill_routed_bank_device(cfg: LayerConfig, ptrs: dict, stream: int = 0):
    """Write all E experts into device buffers (dict name -> device address)."""
    lib = _load_dev()
    sz = routed_sizes(cfg)
    for name, tid in _routed_streams(cfg).items():
        kk = key(cfg.seed, tid)
        n = sz[name] * cfg.E
        if name.endswith("scale"):
            rc = lib.k3gen_dev_scales(kk, 0, n, cfg.scale_lo, cfg.scale_hi, ptrs[name], stream)
        else:
            rc = lib.k3gen_dev_bytes(kk, 0, n, ptrs[name], stream)
        if rc != 0:
            raise RuntimeError(f"device fill of {name} failed with HIP error {rc}")


# ------------------------------------------------------------- RVQ3 experts
RVQ_SIGMA = (0.05, 0.0125, 0.003)   # codebook spread per stage (residual stages shrink)


def rvq_sizes(cfg: LayerConfig) -> dict:
    """Bytes per expert of each RVQ3 tensor: 3 index bytes per 8 weights
    (3.00 bits per weight) and three [256][8] fp32 codebooks per matrix."""
    return dict(w13=3 * 2 * cfg.f * cfg.d // 8, w2=3 * cfg.d * cfg.f // 8, w13_cb=3 * 256 * 8 * 4,
                w2_cb=3 * 256 * 8 * 4)


def rvq_codebooks(cfg: LayerConfig, e0: int, e1: int, which: str) -> np.ndarray:
    """Codebooks [e1-e0][3][256][8] fp32 of matrix `which` ("w13" or "w2"):
    stage s ~ N(0, RVQ_SIGMA[s])."""
    k = key(cfg.seed, T_RVQCB13 if which == "w13" else T_RVQCB2)
    out = np.empty((e1 - e0, 3, 256, 8), dtype=np.float32)
    for e in range(e0, e1):
        for st in range(3):
            out[e - e0, st] = _normal_f32(k, (e * 3 + st) * 2048, 2048,
                                          RVQ_SIGMA[st]).reshape(256, 8)
    return out


def rvq_expert(cfg: LayerConfig, e: int) -> dict:
    """Expert e of the RVQ3 bank: w13 [3][d/128][2f][16] u8 indices (rows 0..f-1
    gate, f..2f-1 up), w2 [3][f/128][d][16], and their codebooks."""
    sz = rvq_sizes(cfg)
    w13 = _bytes(key(cfg.seed, T_RVQ13), e * sz["w13"], sz["w13"])
    w2 = _bytes(key(cfg.seed, T_RVQ2), e * sz["w2"], sz["w2"])
    return dict(w13=w13.reshape(3, cfg.d // 128, 2 * cfg.f, 16),
                w2=w2.reshape(3, cfg.f // 128, cfg.d, 16),
                w13_cb=rvq_codebooks(cfg, e, e + 1, "w13")[0],
                w2_cb=rvq_codebooks(cfg, e, e + 1, "w2")[0])


def fill_rvq_bank_device(cfg: LayerConfig, ptrs: dict, stream: int = 0):
    """Write all E experts' RVQ3 indices into device buffers (name -> address);
    the codebooks come from rvq_codebooks (host)."""
    lib = _load_dev()
    sz = rvq_sizes(cfg)
    for name, tid in (("w13", T_RVQ13), ("w2", T_RVQ2)):
        rc = lib.k3gen_dev_bytes(key(cfg.seed, tid), 0, sz[name] * cfg.E, ptrs[name], stream)
        if rc != 0:
            raise RuntimeError(f"device fill of rvq {name} failed with HIP error {rc}")


# --------------------------------------------------------------- shared experts
def shared_bank(cfg: LayerConfig) -> dict:
    """Shared experts as bf16 bits: w13 [S][2f_s][d] (gate rows then up rows),
    w2 [S][d][f_s]."""
    S, fs, d = cfg.n_shared, cfg.f_shared, cfg.d
    w13 = _normal_bf16(key(cfg.seed, T_SH13), 0, S * 2 * fs * d, cfg.shared_sigma)
    w2 = _normal_bf16(key(cfg.seed, T_SH2), 0, S * d * fs, cfg.shared_sigma)
    return dict(w13=w13.reshape(S, 2 * fs, d), w2=w2.reshape(S, d, fs))
