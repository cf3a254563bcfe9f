"""Torch-facing convenience over the C ABI: holds a layer's device weights,
allocates outputs and workspaces with torch, and calls the library.  Every
computation happens in libk3moe's kernels; this file only marshals."""
import torch

from . import (BF16, DIAG_COUNT, F32, FMT_BF16, FMT_MXFP4, FMT_RVQ3, OP_EXPERT_FFN, OP_EXPERT_GATEUP,
               OP_LAYER, OP_PERMUTE, OP_ROUTE, OP_SHARED_FFN, ACTS, ROUTERS, k3moe_combine,
               k3moe_expert_down,
               k3moe_expert_ffn, k3moe_expert_gateup, k3moe_layer, k3moe_path_class,
               k3moe_permute, k3moe_route, k3moe_shared_ffn, k3moe_workspace_bytes, make_bank, make_shape, make_weights)

_DT = {torch.float32: F32, torch.bfloat16: BF16}


class MoELayer:
    """One routed MoE FFN layer.  routed: dict of uint8 tensors w13 [E][2f][d/2],
    w13_scale [E][2f][d/32], w2 [E][d][f/2], w2_scale [E][d][f/32] (MXFP4), or
    w13 [E][3][d/128][2f][16], w2 [E][3][f/128][d][16] uint8 indices with fp32
    codebooks w13_cb, w2_cb [E][3][256][8] (RVQ3); shared:
    dict of bf16 tensors w13 [S][2fs][d], w2 [S][d][fs] (or empty); router:
    "softmax", "sigmoid" or "sigmoid_norm", with router_bias an fp32 [E]
    tensor (or None) for the sigmoid routers; act: "exact" or "mxfp4" (the
    routed experts' activations quantised to MXFP4)."""

    def __init__(self, w_router, routed: dict, shared: dict, k: int,
                 out_dtype=torch.bfloat16, router: str = "softmax", router_bias=None,
                 act: str = "exact"):
        self.w_router = w_router
        self.routed = routed
        self.shared = shared
        if "w13_cb" in routed:     # RVQ3: [E][3][d/128][2f][16]
            self.fmt = FMT_RVQ3
            self.E, _, nsl, two_f, _ = routed["w13"].shape
            self.f, self.d = two_f // 2, nsl * 128
        else:
            self.fmt = FMT_MXFP4
            self.E, two_f, half_d = routed["w13"].shape
            self.f, self.d = two_f // 2, half_d * 2
        self.k = k
        self.n_shared = shared["w13"].shape[0] if shared else 0
        self.f_shared = shared["w13"].shape[1] // 2 if shared else 0
        self.out_dtype = out_dtype
        self.router = ROUTERS[router]
        self.router_bias = router_bias
        self.act = ACTS[act]
        if self.fmt == FMT_RVQ3:
            self.routed_bank = make_bank(FMT_RVQ3, self.E, self.d, self.f, routed["w13"],
                                         routed["w13_cb"], routed["w2"], routed["w2_cb"])
        else:
            self.routed_bank = make_bank(FMT_MXFP4, self.E, self.d, self.f, routed["w13"],
                                         routed["w13_scale"], routed["w2"], routed["w2_scale"])
        self.shared_bank = make_bank(FMT_BF16, self.n_shared, self.d, self.f_shared,
                                     shared.get("w13"), None, shared.get("w2"), None)
        self.weights = make_weights(w_router, self.routed_bank, self.shared_bank, router_bias)

    # ------------------------------------------------------------ helpers
    def shape(self, T: int, x_dtype=torch.bfloat16, out_dtype=None):
        out_dtype = self.out_dtype if out_dtype is None else out_dtype
        return make_shape(T, self.d, self.f, self.E, self.k, self.n_shared, self.f_shared,
                          _DT[x_dtype], _DT[out_dtype], self.router, self.act, self.fmt)

    def workspace(self, shape, op):
        n = k3moe_workspace_bytes(shape, op)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.w_router.device)

    def path_class(self, T: int, x_dtype=torch.bfloat16) -> int:
        return k3moe_path_class(self.shape(T, x_dtype))

    def _dev(self):
        return self.w_router.device

    # ------------------------------------------------------------- stages
    def route(self, x, want_logits=False, diag=None, stream=None):
        T = x.shape[0]
        s = self.shape(T, x.dtype)
        idx = torch.empty((T, self.k), dtype=torch.int32, device=self._dev())
        w = torch.empty((T, self.k), dtype=torch.float32, device=self._dev())
        logits = torch.empty((T, self.E), dtype=torch.float32, device=self._dev()) if want_logits else None
        k3moe_route(s, x, self.w_router, idx, w, logits, diag, self.workspace(s, OP_ROUTE), stream,
                    router_bias=self.router_bias)
        return idx, w, logits

    def permute(self, idx, diag=None, stream=None):
        T = idx.shape[0]
        s = self.shape(T)
        P = T * self.k
        counts = torch.empty(self.E, dtype=torch.int32, device=self._dev())
        offsets = torch.empty(self.E + 1, dtype=torch.int32, device=self._dev())
        sp = torch.empty(max(P, 1), dtype=torch.int32, device=self._dev())
        pp = torch.empty(max(P, 1), dtype=torch.int32, device=self._dev())
        k3moe_permute(s, idx, counts, offsets, sp, pp, diag, self.workspace(s, OP_PERMUTE), stream)
        return counts, offsets, sp[:P], pp[:P]

    def expert_ffn(self, x, offsets, sorted_pair, stream=None):
        T = x.shape[0]
        s = self.shape(T, x.dtype)
        y = torch.empty((max(T * self.k, 1), self.d), dtype=torch.float32, device=self._dev())
        k3moe_expert_ffn(s, self.routed_bank, x, offsets, sorted_pair, y,
                         self.workspace(s, OP_EXPERT_FFN), stream)
        return y[:T * self.k]

    def expert_gateup(self, x, offsets, sorted_pair, h=None, stream=None):
        T = x.shape[0]
        s = self.shape(T, x.dtype)
        if h is None:
            h = torch.empty((max(T * self.k, 1), self.f), dtype=torch.float32, device=self._dev())
        k3moe_expert_gateup(s, self.routed_bank, x, offsets, sorted_pair, h,
                            self.workspace(s, OP_EXPERT_GATEUP), stream)
        return h[:T * self.k]

    def expert_down(self, h, offsets, T, y=None, stream=None, x_dtype=torch.bfloat16):
        s = self.shape(T, x_dtype)
        if y is None:
            y = torch.empty((max(T * self.k, 1), self.d), dtype=torch.float32, device=self._dev())
        k3moe_expert_down(s, self.routed_bank, h, offsets, y, stream)
        return y[:T * self.k]

    def shared_ffn(self, x, stream=None):
        T = x.shape[0]
        s = self.shape(T, x.dtype)
        y = torch.empty((max(T, 1), self.d), dtype=torch.float32, device=self._dev())
        k3moe_shared_ffn(s, self.shared_bank, x, y, self.workspace(s, OP_SHARED_FFN), stream)
        return y[:T]

    def combine(self, y_perm, pair_pos, topk_w, shared_y, out_dtype=None, stream=None):
        T = topk_w.shape[0]
        s = self.shape(T, torch.bfloat16, out_dtype)
        dt = self.out_dtype if out_dtype is None else out_dtype
        out = torch.empty((max(T, 1), self.d), dtype=dt, device=self._dev())
        k3moe_combine(s, y_perm, pair_pos, topk_w, shared_y, out, stream)
        return out[:T]

    def __call__(self, x, out_dtype=None, diag=None, workspace=None, stream=None, out=None):
        T = x.shape[0]
        s = self.shape(T, x.dtype, out_dtype)
        dt = self.out_dtype if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty((max(T, 1), self.d), dtype=dt, device=self._dev())
        if workspace is None:
            workspace = self.workspace(s, OP_LAYER)
        k3moe_layer(s, self.weights, x, out, diag, workspace, stream)
        return out[:T]

    def staged(self, x, out_dtype=None, stream=None):
        """The five stages called one by one (route, permute, routed experts,
        shared experts, combine); returns every intermediate."""
        diag = torch.zeros(DIAG_COUNT, dtype=torch.int32, device=self._dev())
        idx, w, logits = self.route(x, want_logits=True, diag=diag, stream=stream)
        counts, offsets, sp, pp = self.permute(idx, diag=diag, stream=stream)
        y = self.expert_ffn(x, offsets, sp, stream=stream)
        sh = self.shared_ffn(x, stream=stream) if self.n_shared else None
        out = self.combine(y, pp, w, sh, out_dtype=out_dtype, stream=stream)
        return dict(idx=idx, w=w, logits=logits, counts=counts, offsets=offsets, sorted_pair=sp,
                    pair_pos=pp, y_perm=y, shared_y=sh, out=out, diag=diag)
