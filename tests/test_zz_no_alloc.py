"""k3moe_layer_noalloc, the whole layer on the library's fixed device scratch
buffer (no workspace argument, no allocation), against k3moe_layer with a
caller's workspace: the same bits, on two calls in a row, the second with a
smaller batch (so it runs on what the first left in the buffer)."""
import pytest
import torch

import gen
import gen.device
from gpu_util import log, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _noalloc(L, x, out_dtype):
    from mxfp4_routed_expert_gemv_amd import DIAG_COUNT, k3moe_layer_noalloc
    T = x.shape[0]
    out = torch.empty((T, L.d), dtype=out_dtype, device="cuda")
    diag = torch.zeros(DIAG_COUNT, dtype=torch.int32, device="cuda")
    k3moe_layer_noalloc(L.shape(T, x.dtype, out_dtype), L.weights, x, out, diag)
    return out, diag


def _check_sequence(L, xs, out_dtype):
    from mxfp4_routed_expert_gemv_amd import DIAG_COUNT
    for x in xs:
        got, gdiag = _noalloc(L, x, out_dtype)
        wdiag = torch.zeros(DIAG_COUNT, dtype=torch.int32, device="cuda")
        want = L(x, out_dtype=out_dtype, diag=wdiag)
        torch.cuda.synchronize()
        log(f"  T={x.shape[0]}: diag {to_np(gdiag).tolist()}")
        assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), x.shape[0]
        assert torch.equal(gdiag, wdiag)


def test_noalloc_tiny_then_smaller():
    require_gpu()
    cfg = gen.get("tiny").with_tokens(37)
    wl = gen.device.build(cfg)
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    L = MoELayer(wl.w_router, wl.routed, wl.shared, cfg.k, out_dtype=torch.float32)
    log("case tiny: 37 then 5 tokens")
    _check_sequence(L, [wl.x, wl.x[:5].contiguous()], torch.float32)


def test_noalloc_full_size_then_smaller(big):
    """d = 7168, 896 experts top-16: 64 tokens (matrix-core class), then one
    token (the one-token kernels), then 103, the largest batch the buffer
    holds; a 104-token call is refused before anything is enqueued."""
    from mxfp4_routed_expert_gemv_amd import K3moeError
    from mxfp4_routed_expert_gemv_amd.layer import MoELayer
    cfg = gen.get("decode_b64")
    L = MoELayer(big.w_router, big.routed, big.shared, cfg.k, out_dtype=torch.bfloat16)
    x = gen.device.activations(cfg.with_tokens(104))
    log("case full size: 64, 1, 103 tokens")
    _check_sequence(L, [x[:64].contiguous(), x[64:65].contiguous(), x[:103].contiguous()],
                    torch.bfloat16)
    with pytest.raises(K3moeError, match="EWORKSPACE"):
        _noalloc(L, x, torch.bfloat16)
