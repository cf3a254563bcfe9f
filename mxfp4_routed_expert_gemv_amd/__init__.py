"""Python binding of libk3moe: the routed MoE FFN layer on MXFP4 experts for
MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions keep the C names (k3moe_route, k3moe_permute,
k3moe_expert_ffn, k3moe_shared_ffn, k3moe_combine, k3moe_layer); tensors are
torch device tensors (or raw device addresses), the stream defaults to torch's
current stream, and a non-OK status raises K3moeError.  PyTorch provides device
memory and streams only.

If libk3moe.so is not built this module raises on import: there is no other
implementation to fall back to.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libk3moe.so")

F32, BF16 = 0, 1
FMT_MXFP4, FMT_BF16, FMT_RVQ3 = 0, 1, 2
(OP_ROUTE, OP_PERMUTE, OP_EXPERT_FFN, OP_SHARED_FFN, OP_COMBINE, OP_LAYER,
 OP_EXPERT_GATEUP) = range(7)
PATH_GEMV, PATH_MFMA = 0, 1
ROUTER_SOFTMAX, ROUTER_SIGMOID, ROUTER_SIGMOID_NORM = 0, 1, 2
ROUTERS = {"softmax": ROUTER_SOFTMAX, "sigmoid": ROUTER_SIGMOID,
           "sigmoid_norm": ROUTER_SIGMOID_NORM}
DIAG_RECHECKED_TOKENS, DIAG_NONFINITE_LOGITS, DIAG_BAD_EXPERT_IDS = 0, 1, 2
DIAG_SCORE_NEAR_TIES = 3
ACT_EXACT, ACT_MXFP4 = 0, 1
ACTS = {"exact": ACT_EXACT, "mxfp4": ACT_MXFP4}
DIAG_COUNT = 4

STATUS = {0: "K3MOE_OK", 1: "K3MOE_EINVAL", 2: "K3MOE_ESHAPE", 3: "K3MOE_EALIGN",
          4: "K3MOE_EWORKSPACE", 5: "K3MOE_EUNSUPPORTED", 6: "K3MOE_EHIP"}
EXPORTS = ["k3moe_workspace_bytes", "k3moe_mxfp4_bytes", "k3moe_path_class", "k3moe_route",
           "k3moe_permute", "k3moe_expert_ffn", "k3moe_expert_gateup", "k3moe_expert_down",
           "k3moe_shared_ffn", "k3moe_combine", "k3moe_layer", "k3moe_layer_noalloc",
           "k3moe_status_str", "k3moe_last_error", "k3moe_cache_create", "k3moe_cache_destroy",
           "k3moe_cache_workspace_bytes", "k3moe_cache_layer", "k3moe_cache_prefetch",
           "k3moe_cache_plan", "k3moe_cache_stats_get"]
NOALLOC_SCRATCH_BYTES = 64 << 20


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("f_shared", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("router", ctypes.c_int32),
                ("act", ctypes.c_int32), ("routed_format", ctypes.c_int32)]


class ExpertBank(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("routed", ExpertBank), ("shared", ExpertBank),
                ("router_bias", ctypes.c_void_p)]


class CacheStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("lookups", "hits", "misses", "prefetched",
                                              "prefetch_hits", "evictions", "bytes_copied")]


class K3moeError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def _load():
    # torch's HIP runtime first: when torch is used in the same process,
    # libk3moe must bind to the runtime torch already loaded (same soname)
    # rather than bring a second copy that then finds no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                          "the layer has no implementation other than the HIP library")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    SP = ctypes.POINTER(Shape)
    lib.k3moe_workspace_bytes.restype = S
    lib.k3moe_workspace_bytes.argtypes = [SP, ctypes.c_int]
    lib.k3moe_mxfp4_bytes.restype = ctypes.c_uint64
    lib.k3moe_mxfp4_bytes.argtypes = [I64, I64]
    lib.k3moe_path_class.restype = ctypes.c_int
    lib.k3moe_path_class.argtypes = [SP]
    lib.k3moe_route.restype = ctypes.c_int
    lib.k3moe_route.argtypes = [SP, P, P, P, P, P, P, P, P, S, P]
    lib.k3moe_permute.restype = ctypes.c_int
    lib.k3moe_permute.argtypes = [SP, P, P, P, P, P, P, P, S, P]
    lib.k3moe_expert_ffn.restype = ctypes.c_int
    lib.k3moe_expert_ffn.argtypes = [SP, ctypes.POINTER(ExpertBank), P, P, P, P, P, S, P]
    lib.k3moe_expert_gateup.restype = ctypes.c_int
    lib.k3moe_expert_gateup.argtypes = [SP, ctypes.POINTER(ExpertBank), P, P, P, P, P, S, P]
    lib.k3moe_expert_down.restype = ctypes.c_int
    lib.k3moe_expert_down.argtypes = [SP, ctypes.POINTER(ExpertBank), P, P, P, P]
    lib.k3moe_shared_ffn.restype = ctypes.c_int
    lib.k3moe_shared_ffn.argtypes = [SP, ctypes.POINTER(ExpertBank), P, P, P, S, P]
    lib.k3moe_combine.restype = ctypes.c_int
    lib.k3moe_combine.argtypes = [SP, P, P, P, P, P, P]
    lib.k3moe_layer.restype = ctypes.c_int
    lib.k3moe_layer.argtypes = [SP, ctypes.POINTER(LayerWeights), P, P, P, P, S, P]
    lib.k3moe_layer_noalloc.restype = ctypes.c_int
    lib.k3moe_layer_noalloc.argtypes = [SP, ctypes.POINTER(LayerWeights), P, P, P, P]
    BP = ctypes.POINTER(ExpertBank)
    lib.k3moe_cache_create.restype = ctypes.c_int
    lib.k3moe_cache_create.argtypes = [SP, BP, BP, ctypes.POINTER(P)]
    lib.k3moe_cache_destroy.restype = None
    lib.k3moe_cache_destroy.argtypes = [P]
    lib.k3moe_cache_workspace_bytes.restype = S
    lib.k3moe_cache_workspace_bytes.argtypes = [SP, I32]
    lib.k3moe_cache_layer.restype = ctypes.c_int
    lib.k3moe_cache_layer.argtypes = [P, SP, ctypes.POINTER(LayerWeights), P, P, P, P, S, P, P]
    lib.k3moe_cache_prefetch.restype = ctypes.c_int
    lib.k3moe_cache_prefetch.argtypes = [P, P, I32, P]
    lib.k3moe_cache_plan.restype = ctypes.c_int
    lib.k3moe_cache_plan.argtypes = [P, P, I32, P]
    lib.k3moe_cache_stats_get.restype = ctypes.c_int
    lib.k3moe_cache_stats_get.argtypes = [P, ctypes.POINTER(CacheStats)]
    lib.k3moe_status_str.restype = ctypes.c_char_p
    lib.k3moe_status_str.argtypes = [ctypes.c_int]
    lib.k3moe_last_error.restype = ctypes.c_char_p
    lib.k3moe_last_error.argtypes = []
    return lib


lib = _load()


def _addr(t):
    """Device address of a torch tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _check(status):
    if status != 0:
        raise K3moeError(status, lib.k3moe_last_error().decode())


# ----------------------------------------------------------------- C wrappers
def k3moe_workspace_bytes(shape: Shape, op: int) -> int:
    return lib.k3moe_workspace_bytes(ctypes.byref(shape), op)


def k3moe_mxfp4_bytes(rows: int, cols: int) -> int:
    return lib.k3moe_mxfp4_bytes(rows, cols)


def k3moe_path_class(shape: Shape) -> int:
    return lib.k3moe_path_class(ctypes.byref(shape))


def k3moe_route(shape, x, w_router, topk_idx, topk_w, logits=None, diag=None, workspace=None,
                stream=None, router_bias=None):
    wp, wb = _ws(workspace)
    _check(lib.k3moe_route(ctypes.byref(shape), _addr(x), _addr(w_router), _addr(router_bias),
                           _addr(topk_idx), _addr(topk_w), _addr(logits), _addr(diag), wp, wb,
                           _stream(stream)))


def k3moe_permute(shape, topk_idx, counts, offsets, sorted_pair, pair_pos, diag=None,
                  workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(lib.k3moe_permute(ctypes.byref(shape), _addr(topk_idx), _addr(counts),
                             _addr(offsets), _addr(sorted_pair), _addr(pair_pos), _addr(diag),
                             wp, wb, _stream(stream)))


def k3moe_expert_ffn(shape, bank: ExpertBank, x, offsets, sorted_pair, y, workspace=None,
                     stream=None):
    wp, wb = _ws(workspace)
    _check(lib.k3moe_expert_ffn(ctypes.byref(shape), ctypes.byref(bank), _addr(x),
                                _addr(offsets), _addr(sorted_pair), _addr(y), wp, wb,
                                _stream(stream)))


def k3moe_expert_gateup(shape, bank: ExpertBank, x, offsets, sorted_pair, h, workspace=None,
                        stream=None):
    wp, wb = _ws(workspace)
    _check(lib.k3moe_expert_gateup(ctypes.byref(shape), ctypes.byref(bank), _addr(x),
                                   _addr(offsets), _addr(sorted_pair), _addr(h), wp, wb,
                                   _stream(stream)))


def k3moe_expert_down(shape, bank: ExpertBank, h, offsets, y, stream=None):
    _check(lib.k3moe_expert_down(ctypes.byref(shape), ctypes.byref(bank), _addr(h),
                                 _addr(offsets), _addr(y), _stream(stream)))


def k3moe_shared_ffn(shape, bank: ExpertBank, x, y, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(lib.k3moe_shared_ffn(ctypes.byref(shape), ctypes.byref(bank), _addr(x), _addr(y),
                                wp, wb, _stream(stream)))


def k3moe_combine(shape, y_perm, pair_pos, topk_w, shared_y, out, stream=None):
    _check(lib.k3moe_combine(ctypes.byref(shape), _addr(y_perm), _addr(pair_pos),
                             _addr(topk_w), _addr(shared_y), _addr(out), _stream(stream)))


def k3moe_layer(shape, weights: LayerWeights, x, out, diag=None, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(lib.k3moe_layer(ctypes.byref(shape), ctypes.byref(weights), _addr(x), _addr(out),
                           _addr(diag), wp, wb, _stream(stream)))


def k3moe_layer_noalloc(shape, weights: LayerWeights, x, out, diag=None, stream=None):
    """The whole layer on the library's fixed device scratch buffer (no
    workspace, no allocation)."""
    _check(lib.k3moe_layer_noalloc(ctypes.byref(shape), ctypes.byref(weights), _addr(x),
                                   _addr(out), _addr(diag), _stream(stream)))


class ExpertCache:
    """An HBM cache of host-resident routed experts (k3moe_cache_*): host_bank
    holds pinned host tensors, slot_bank device tensors of `slots` experts;
    the caller keeps both alive while the cache lives."""

    def __init__(self, shape: Shape, host_bank: ExpertBank, slot_bank: ExpertBank):
        self.handle = ctypes.c_void_p()
        _check(lib.k3moe_cache_create(ctypes.byref(shape), ctypes.byref(host_bank),
                                      ctypes.byref(slot_bank), ctypes.byref(self.handle)))
        self.slots = slot_bank.n_experts

    def close(self):
        if self.handle:
            lib.k3moe_cache_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        self.close()

    def workspace_bytes(self, shape: Shape) -> int:
        return lib.k3moe_cache_workspace_bytes(ctypes.byref(shape), self.slots)

    def layer(self, shape, weights: LayerWeights, x, out, diag=None, workspace=None,
              stream=None, copy_stream=None):
        wp, wb = _ws(workspace)
        cs = None if copy_stream is None else _stream(copy_stream)
        _check(lib.k3moe_cache_layer(self.handle, ctypes.byref(shape), ctypes.byref(weights),
                                     _addr(x), _addr(out), _addr(diag), wp, wb, _stream(stream),
                                     cs))

    def prefetch(self, ids, copy_stream=None):
        import numpy as np
        a = np.ascontiguousarray(ids, dtype=np.int32)
        cs = None if copy_stream is None else _stream(copy_stream)
        _check(lib.k3moe_cache_prefetch(self.handle, a.ctypes.data, a.size, cs))

    def plan(self, ids):
        import numpy as np
        a = np.ascontiguousarray(ids, dtype=np.int32)
        out = np.empty(a.size, dtype=np.int32)
        _check(lib.k3moe_cache_plan(self.handle, a.ctypes.data, a.size, out.ctypes.data))
        return out

    def stats(self) -> dict:
        st = CacheStats()
        _check(lib.k3moe_cache_stats_get(self.handle, ctypes.byref(st)))
        return {n: getattr(st, n) for n, _ in CacheStats._fields_}


# --------------------------------------------------------- struct builders
def make_shape(T, d, f, E, k, n_shared, f_shared, x_dtype, out_dtype, router=ROUTER_SOFTMAX,
               act=ACT_EXACT, routed_format=FMT_MXFP4) -> Shape:
    return Shape(T, d, f, E, k, n_shared, f_shared, x_dtype, out_dtype, router, act,
                 routed_format)


def make_bank(fmt, n, d, f, w13, w13_scale, w2, w2_scale) -> ExpertBank:
    return ExpertBank(fmt, n, d, f, _addr(w13), _addr(w13_scale), _addr(w2), _addr(w2_scale))


def make_weights(w_router, routed: ExpertBank, shared: ExpertBank,
                 router_bias=None) -> LayerWeights:
    return LayerWeights(_addr(w_router), routed, shared, _addr(router_bias))
