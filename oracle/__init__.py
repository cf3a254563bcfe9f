"""CPU oracle of the routed MoE FFN layer — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library (mxfp4_routed_expert_gemv_amd)
and never imports it.  The arithmetic lives in oracle.c (fp64, fixed ascending
order, no FMA contraction); this module only marshals numpy arrays and walks
the stages in order:

  route    logits = x Wr^T; top-k by (logit desc, id asc); ids ascending;
           softmax over the chosen logits            (router of the pages' MoE
           layer: 16 of 896 experts per token — review page "at a glance");
           or the pages' K3 router: top-k by sigmoid(l) + bias, weights the
           unbiased sigmoid(l), raw or renormalised (review page,
           "KDA/MLA/MoE" table)
  permute  stable counting sort of (token, slot) pairs by expert
  experts  per pair: y = Wd (silu(Wg x) * (Wu x)) on exactly decoded MXFP4
           weights (the pages multiply the 4-bit experts directly — README,
           "shard census"; explainer, "reduction one")
  shared   the always-on bf16 shared experts, summed in order
  combine  out = shared + sum over chosen experts, ascending id, of w * y
"""
import ctypes
import os

import numpy as np

from . import build as _build

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int


def _ptr(a: np.ndarray):
    return a.ctypes.data if a is not None else None


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 copy of fp32 values or of bf16 bits (uint16)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported activation dtype {a.dtype}")


class Oracle:
    def __init__(self, lib_path: str = None):
        if lib_path is None:
            lib_path = _build.LIB
            if not os.path.exists(lib_path):
                _build.build()
        lib = ctypes.CDLL(lib_path)
        lib.oracle_e2m1.restype = ctypes.c_double
        lib.oracle_e2m1.argtypes = [_I32]
        lib.oracle_e8m0.restype = ctypes.c_double
        lib.oracle_e8m0.argtypes = [_I32]
        lib.oracle_mxfp4_decode.argtypes = [_I64, _I64, _I32, _P, _P, _P]
        lib.oracle_router_logits.argtypes = [_I64, _I32, _I32, _P, _P, _P]
        lib.oracle_topk_softmax.argtypes = [_I64, _I32, _I32, _P, _P, _P]
        lib.oracle_topk_sigmoid.argtypes = [_I64, _I32, _I32, _P, _P, _I32, _P, _P]
        lib.oracle_permute.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P]
        lib.oracle_mxfp4_ffn.argtypes = [_I32, _I32, _P, _P, _P, _P, _I64, _P, _P, _P]
        lib.oracle_quantize_mxfp4.argtypes = [_I64, _P, _P, _P]
        lib.oracle_mxfp4_ffn_qact.argtypes = [_I32, _I32, _P, _P, _P, _P, _I64, _P, _P, _P]
        lib.oracle_rvq_decode.argtypes = [_I64, _I64, _I64, _I32, _P, _P, _P]
        lib.oracle_rvq_ffn.argtypes = [_I32, _I32, _P, _P, _P, _P, _I64, _P, _P, _P]
        lib.oracle_bf16_ffn.argtypes = [_I32, _I32, _P, _P, _I64, _P, _P]
        lib.oracle_combine.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P]
        lib.oracle_threads.restype = _I32
        lib.oracle_threads.argtypes = []
        self.lib = lib

    def threads(self) -> int:
        return self.lib.oracle_threads()

    # ------------------------------------------------------------ formats
    def e2m1(self, code: int) -> float:
        return self.lib.oracle_e2m1(code)

    def e8m0(self, s: int) -> float:
        return self.lib.oracle_e8m0(s)

    def mxfp4_decode(self, q: np.ndarray, s: np.ndarray) -> np.ndarray:
        """[rows][cols/2] codes + [rows][cols/32] scales -> [rows][cols] fp64."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint8)
        rows, cols = q.shape[0], q.shape[1] * 2
        out = np.empty((rows, cols), dtype=np.float64)
        self.lib.oracle_mxfp4_decode(0, rows, cols, _ptr(q), _ptr(s), _ptr(out))
        return out

    # ------------------------------------------------------------- router
    def router_logits(self, x64: np.ndarray, w_router: np.ndarray) -> np.ndarray:
        x64 = np.ascontiguousarray(x64, dtype=np.float64)
        wr = np.ascontiguousarray(w_router, dtype=np.uint16)
        T, d = x64.shape
        E = wr.shape[0]
        assert wr.shape[1] == d
        out = np.empty((T, E), dtype=np.float64)
        self.lib.oracle_router_logits(T, d, E, _ptr(x64), _ptr(wr), _ptr(out))
        return out

    def topk_softmax(self, logits: np.ndarray, k: int):
        logits = np.ascontiguousarray(logits, dtype=np.float64)
        T, E = logits.shape
        idx = np.empty((T, k), dtype=np.int32)
        w = np.empty((T, k), dtype=np.float64)
        self.lib.oracle_topk_softmax(T, E, k, _ptr(logits), _ptr(idx), _ptr(w))
        return idx, w

    def topk_sigmoid(self, logits: np.ndarray, k: int, bias: np.ndarray = None,
                     norm: bool = False):
        """The pages' K3 router: select by sigmoid(l) + bias, weights from the
        unbiased sigmoid(l), optionally renormalised over the chosen."""
        logits = np.ascontiguousarray(logits, dtype=np.float64)
        T, E = logits.shape
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        assert b is None or b.shape == (E,)
        idx = np.empty((T, k), dtype=np.int32)
        w = np.empty((T, k), dtype=np.float64)
        self.lib.oracle_topk_sigmoid(T, E, k, _ptr(logits), _ptr(b), 1 if norm else 0, _ptr(idx),
                                     _ptr(w))
        return idx, w

    def route(self, x64, w_router, k, router: str = "softmax", bias=None):
        """router: "softmax" (softmax over the chosen logits), "sigmoid" (the
        pages' K3 router, raw sigmoid weights) or "sigmoid_norm" (the same,
        weights renormalised over the chosen)."""
        logits = self.router_logits(x64, w_router)
        if router == "softmax":
            assert bias is None, "the softmax router takes no bias"
            idx, w = self.topk_softmax(logits, k)
        else:
            assert router in ("sigmoid", "sigmoid_norm"), router
            idx, w = self.topk_sigmoid(logits, k, bias, norm=router == "sigmoid_norm")
        return logits, idx, w

    # ------------------------------------------------------------ permute
    def permute(self, idx: np.ndarray, E: int):
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, k = idx.shape
        counts = np.empty(E, dtype=np.int32)
        offsets = np.empty(E + 1, dtype=np.int32)
        sorted_pair = np.empty(T * k, dtype=np.int32)
        pair_pos = np.empty(T * k, dtype=np.int32)
        self.lib.oracle_permute(T, E, k, _ptr(idx), _ptr(counts), _ptr(offsets),
                                _ptr(sorted_pair), _ptr(pair_pos))
        return counts, offsets, sorted_pair, pair_pos

    # ------------------------------------------------------------ experts
    def mxfp4_ffn(self, expert: dict, x64: np.ndarray, want_h: bool = False):
        """One MXFP4 expert (dict w13, w13_scale, w2, w2_scale) over rows x64."""
        x64 = np.ascontiguousarray(x64, dtype=np.float64)
        n, d = x64.shape
        w13 = np.ascontiguousarray(expert["w13"], dtype=np.uint8)
        w13s = np.ascontiguousarray(expert["w13_scale"], dtype=np.uint8)
        w2 = np.ascontiguousarray(expert["w2"], dtype=np.uint8)
        w2s = np.ascontiguousarray(expert["w2_scale"], dtype=np.uint8)
        f = w13.shape[0] // 2
        assert w13.shape == (2 * f, d // 2) and w2.shape == (d, f // 2)
        assert w13s.shape == (2 * f, d // 32) and w2s.shape == (d, f // 32)
        y = np.empty((n, d), dtype=np.float64)
        h = np.empty((n, f), dtype=np.float64) if want_h else None
        self.lib.oracle_mxfp4_ffn(d, f, _ptr(w13), _ptr(w13s), _ptr(w2), _ptr(w2s), n,
                                  _ptr(x64), _ptr(y), _ptr(h))
        return (y, h) if want_h else y

    def quantize_mxfp4(self, v: np.ndarray):
        """OCP MX quantisation to MXFP4 of rows whose length is a multiple of
        32: [..., n] fp64 -> (codes [..., n/2] u8 packed, scales [..., n/32] u8)."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        assert v.shape[-1] % 32 == 0
        nblk = v.size // 32
        codes = np.empty(v.shape[:-1] + (v.shape[-1] // 2,), dtype=np.uint8)
        scales = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), dtype=np.uint8)
        self.lib.oracle_quantize_mxfp4(nblk, _ptr(v), _ptr(codes), _ptr(scales))
        return codes, scales

    def mxfp4_ffn_qact(self, expert: dict, x64: np.ndarray, want_h: bool = False):
        """One MXFP4 expert with activations quantised to MXFP4 (x before
        gate/up, h before down)."""
        x64 = np.ascontiguousarray(x64, dtype=np.float64)
        n, d = x64.shape
        w13 = np.ascontiguousarray(expert["w13"], dtype=np.uint8)
        w13s = np.ascontiguousarray(expert["w13_scale"], dtype=np.uint8)
        w2 = np.ascontiguousarray(expert["w2"], dtype=np.uint8)
        w2s = np.ascontiguousarray(expert["w2_scale"], dtype=np.uint8)
        f = w13.shape[0] // 2
        y = np.empty((n, d), dtype=np.float64)
        h = np.empty((n, f), dtype=np.float64) if want_h else None
        self.lib.oracle_mxfp4_ffn_qact(d, f, _ptr(w13), _ptr(w13s), _ptr(w2), _ptr(w2s), n,
                                       _ptr(x64), _ptr(y), _ptr(h))
        return (y, h) if want_h else y

    def rvq_decode(self, idx: np.ndarray, cb: np.ndarray, rows: int, cols: int) -> np.ndarray:
        """RVQ3 matrix (idx [3][cols/128][rows][16] u8, cb [3][256][8] fp32) ->
        [rows][cols] fp64, each weight the sum of its three codeword entries."""
        idx = np.ascontiguousarray(idx, dtype=np.uint8)
        cb = np.ascontiguousarray(cb, dtype=np.float32)
        assert idx.size == 3 * rows * cols // 8 and cb.shape == (3, 256, 8)
        out = np.empty((rows, cols), dtype=np.float64)
        self.lib.oracle_rvq_decode(0, rows, rows, cols, _ptr(idx), _ptr(cb), _ptr(out))
        return out

    def rvq_ffn(self, expert: dict, x64: np.ndarray, want_h: bool = False):
        """One RVQ3 expert (dict w13, w13_cb, w2, w2_cb) over rows x64."""
        x64 = np.ascontiguousarray(x64, dtype=np.float64)
        n, d = x64.shape
        w13 = np.ascontiguousarray(expert["w13"], dtype=np.uint8)
        w13c = np.ascontiguousarray(expert["w13_cb"], dtype=np.float32)
        w2 = np.ascontiguousarray(expert["w2"], dtype=np.uint8)
        w2c = np.ascontiguousarray(expert["w2_cb"], dtype=np.float32)
        f = w13.size * 8 // 3 // d // 2
        assert w13.size == 3 * 2 * f * d // 8 and w2.size == 3 * d * f // 8
        y = np.empty((n, d), dtype=np.float64)
        h = np.empty((n, f), dtype=np.float64) if want_h else None
        self.lib.oracle_rvq_ffn(d, f, _ptr(w13), _ptr(w13c), _ptr(w2), _ptr(w2c), n, _ptr(x64),
                                _ptr(y), _ptr(h))
        return (y, h) if want_h else y

    def bf16_ffn(self, w13: np.ndarray, w2: np.ndarray, x64: np.ndarray):
        x64 = np.ascontiguousarray(x64, dtype=np.float64)
        n, d = x64.shape
        w13 = np.ascontiguousarray(w13, dtype=np.uint16)
        w2 = np.ascontiguousarray(w2, dtype=np.uint16)
        f = w13.shape[0] // 2
        assert w13.shape == (2 * f, d) and w2.shape == (d, f)
        y = np.empty((n, d), dtype=np.float64)
        self.lib.oracle_bf16_ffn(d, f, _ptr(w13), _ptr(w2), n, _ptr(x64), _ptr(y))
        return y

    def shared_ffn(self, shared: dict, x64: np.ndarray):
        """Sum of the shared experts in order: ((s_0 + s_1) + ...)."""
        acc = None
        for j in range(shared["w13"].shape[0]):
            s = self.bf16_ffn(shared["w13"][j], shared["w2"][j], x64)
            acc = s if acc is None else acc + s
        return acc

    def expert(self, act: str):
        """The expert FFN of a mode: "exact" (MXFP4 experts, activations as
        given), "mxfp4" (MXFP4 experts, x and h quantised to MXFP4) or "rvq3"
        (RVQ3 experts)."""
        return {"exact": self.mxfp4_ffn, "mxfp4": self.mxfp4_ffn_qact, "rvq3": self.rvq_ffn}[act]

    def routed_ffn(self, x64, get_expert, counts, offsets, sorted_pair, k, act="exact"):
        """y_perm [P][d]: row p = expert e's output on the token of pair
        sorted_pair[p], for the experts e with counts[e] > 0."""
        d = x64.shape[1]
        ffn = self.expert(act)
        y = np.zeros((len(sorted_pair), d), dtype=np.float64)
        for e in np.nonzero(counts)[0]:
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            toks = sorted_pair[lo:hi] // k
            y[lo:hi] = ffn(get_expert(int(e)), x64[toks])
        return y

    # ------------------------------------------------------------ combine
    def combine(self, y_perm, pair_pos, w, shared_y=None):
        T, k = w.shape
        d = y_perm.shape[1]
        y_perm = np.ascontiguousarray(y_perm, dtype=np.float64)
        pair_pos = np.ascontiguousarray(pair_pos, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
        sh = None if shared_y is None else np.ascontiguousarray(shared_y, dtype=np.float64)
        out = np.empty((T, d), dtype=np.float64)
        self.lib.oracle_combine(T, d, k, _ptr(y_perm), _ptr(pair_pos), _ptr(w), _ptr(sh),
                                _ptr(out))
        return out

    # -------------------------------------------------------------- layer
    def layer(self, x, w_router, get_expert, shared, k, E, router="softmax", bias=None,
              act="exact"):
        """All stages on the full batch.  x: fp32 or bf16 bits [T][d];
        get_expert(e) -> dict of expert e's packed tensors; shared: dict of
        bf16 banks or None; router and bias as for route(); act: the routed
        experts' activation mode (expert()).  Returns every intermediate in
        fp64/int32."""
        x64 = to_f64(x)
        logits, idx, w = self.route(x64, w_router, k, router, bias)
        counts, offsets, sorted_pair, pair_pos = self.permute(idx, E)
        y_perm = self.routed_ffn(x64, get_expert, counts, offsets, sorted_pair, k, act)
        shared_y = self.shared_ffn(shared, x64) if shared is not None else None
        out = self.combine(y_perm, pair_pos, w, shared_y)
        return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                    sorted_pair=sorted_pair, pair_pos=pair_pos, y_perm=y_perm,
                    shared_y=shared_y, out=out)

    def token_outputs(self, x_rows, idx_rows, w_rows, get_expert, shared, act="exact"):
        """out for a few tokens alone (each token's output depends only on its own
        activation row, chosen experts and weights): x_rows [n][d] activations,
        idx_rows/w_rows [n][k] their routing.  Sums in the same order as
        combine().  Returns (out [n][d], shared_y [n][d] or None, y [n][k][d])."""
        x64 = to_f64(x_rows)
        n, k = idx_rows.shape
        d = x64.shape[1]
        y = np.zeros((n, k, d), dtype=np.float64)
        ffn = self.expert(act)
        for e in np.unique(idx_rows):
            rows, slots = np.nonzero(idx_rows == e)
            y[rows, slots] = ffn(get_expert(int(e)), x64[rows])
        shared_y = self.shared_ffn(shared, x64) if shared is not None else None
        pair_pos = np.arange(n * k, dtype=np.int32)
        out = self.combine(y.reshape(n * k, d), pair_pos, np.asarray(w_rows, np.float64),
                           shared_y)
        return out, shared_y, y


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default

