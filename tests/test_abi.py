"""The C ABI on the CPU: the library loads, exports every function the header
declares, sizes workspaces, and rejects every invalid argument with the
documented status before launching anything (no device is touched)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, golden

k3 = pytest.importorskip("mxfp4_routed_expert_gemv_amd")

HEADER = os.path.join(ROOT, "include", "k3moe.h")

EINVAL, ESHAPE, EALIGN, EWORKSPACE, EUNSUPPORTED = 1, 2, 3, 4, 5
FAKE = 0x10000   # an aligned address that is never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(k3moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(k3.lib, n), n
    assert sorted(k3.EXPORTS) == names


def big_shape(T=1, **kw):
    a = dict(T=T, d=7168, f=2048, E=896, k=16, n_shared=2, f_shared=2048, x_dtype=k3.BF16,
             out_dtype=k3.BF16)
    a.update(kw)
    return k3.make_shape(**a)


def test_mxfp4_bytes_matches_pages_accounting():
    g = golden("pages_byte_accounting.json")
    # the pages' expert: 33,030,144 weights at 0.53125 B each = 17,547,264 B
    assert g["expert_params"] * g["bytes_per_weight"] == g["expert_bytes"]
    # an MXFP4 matrix whose element count is the pages' expert parameter count
    assert k3.k3moe_mxfp4_bytes(1, g["expert_params"]) == g["expert_bytes"]
    assert k3.k3moe_mxfp4_bytes(3 * 7168, 1536) == g["expert_bytes"]   # 3 x d x f', d = 7168
    assert g["experts_per_layer"] * g["moe_layers"] == g["experts_total"]
    # the census prints 1.447 TB for 1.44646e12 B: within one unit of its last digit
    assert abs(g["experts_total"] * g["expert_bytes"] / 1e12 - g["routed_set_tb"]) < 1e-3
    assert abs(g["experts_per_token"] * g["expert_bytes"] / 1e9 - g["ladder_row1_gb_read"]) < 5e-3
    # this layer's expert: gate/up [2f][d] + down [d][f]
    per_expert = k3.k3moe_mxfp4_bytes(2 * 2048, 7168) + k3.k3moe_mxfp4_bytes(7168, 2048)
    assert per_expert == 23_396_352
    assert 16 * per_expert == 374_341_632


def test_workspace_sizes():
    s = big_shape(T=1)
    for op in range(7):
        n = k3.k3moe_workspace_bytes(s, op)
        assert n % 256 == 0
    assert k3.k3moe_workspace_bytes(s, k3.OP_LAYER) >= 16 * 7168 * 4
    assert k3.k3moe_workspace_bytes(s, k3.OP_COMBINE) == 0
    assert k3.k3moe_workspace_bytes(big_shape(T=0), k3.OP_LAYER) == 0
    assert k3.k3moe_workspace_bytes(big_shape(d=100), k3.OP_LAYER) == 0
    assert k3.k3moe_workspace_bytes(s, 99) == 0
    # gate/up alone: the activations in two E4M3 passes, 272 bytes per token
    # and 128-element stage, wherever the routed experts take the scaled
    # matrix-core instruction (bf16 x, d % 512 == 0, f % 512 == 0, any T);
    # nothing for the fp32 GEMV
    assert k3.k3moe_workspace_bytes(s, k3.OP_EXPERT_GATEUP) == 15360
    assert k3.k3moe_workspace_bytes(big_shape(T=1, x_dtype=k3.F32), k3.OP_EXPERT_GATEUP) == 0
    assert k3.k3moe_workspace_bytes(big_shape(T=1, f=2048 + 256), k3.OP_EXPERT_GATEUP) == 0
    big = big_shape(T=4096)
    xq = 4096 * (7168 // 128) * 272
    assert k3.k3moe_workspace_bytes(big, k3.OP_EXPERT_GATEUP) == (xq + 255) // 256 * 256
    assert k3.k3moe_workspace_bytes(big, k3.OP_EXPERT_FFN) >= 4096 * 16 * 2048 * 4 + xq


def test_gateup_workspace_validation():
    bank = k3.make_bank(k3.FMT_MXFP4, 896, 7168, 2048, FAKE, FAKE, FAKE, FAKE)

    def gateup(shape, ws, nbytes):
        return k3.lib.k3moe_expert_gateup(ctypes.byref(shape), ctypes.byref(bank), FAKE, FAKE,
                                          FAKE, FAKE, ws, nbytes, None)
    big = big_shape(T=64)
    assert gateup(big, None, 0) == EWORKSPACE
    need = k3.k3moe_workspace_bytes(big, k3.OP_EXPERT_GATEUP)
    assert gateup(big, FAKE * 256, need - 256) == EWORKSPACE
    assert gateup(big, FAKE * 256 + 16, need) == EALIGN


def _route(shape, x=FAKE, wr=FAKE, idx=FAKE, w=FAKE, ws=(FAKE * 256, 1 << 40), bias=None):
    return k3.lib.k3moe_route(ctypes.byref(shape), x, wr, bias, idx, w, None, None, ws[0], ws[1],
                              None)


def test_route_validation():
    assert _route(big_shape(T=-1)) == EINVAL
    assert k3.lib.k3moe_route(None, FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, 1,
                              None) == EINVAL
    assert _route(big_shape(d=7170)) == ESHAPE
    assert _route(big_shape(d=16)) == ESHAPE
    assert _route(big_shape(f=2050)) == ESHAPE
    assert _route(big_shape(k=0)) == ESHAPE
    assert _route(big_shape(k=897)) == ESHAPE
    assert _route(big_shape(E=2000)) == ESHAPE
    assert _route(big_shape(T=1 << 28)) == ESHAPE          # T * k >= 2^31
    assert _route(big_shape(x_dtype=7)) == EUNSUPPORTED
    assert _route(big_shape(out_dtype=3)) == EUNSUPPORTED
    # router modes: an unknown one, a bias given to the softmax router, a
    # misaligned bias
    assert _route(big_shape(router=3)) == EUNSUPPORTED
    assert _route(big_shape(), bias=FAKE) == EINVAL
    assert _route(big_shape(router=k3.ROUTER_SIGMOID), bias=FAKE + 4) == EALIGN
    assert _route(big_shape(router=k3.ROUTER_SIGMOID_NORM, T=0), bias=FAKE) == 0
    assert _route(big_shape(), x=None) == EINVAL
    assert _route(big_shape(), wr=FAKE + 8) == EALIGN
    assert _route(big_shape(), ws=(None, 0)) == EWORKSPACE
    assert _route(big_shape(), ws=(FAKE * 256, 16)) == EWORKSPACE
    assert _route(big_shape(), ws=(FAKE * 256 + 64, 1 << 40)) == EALIGN
    assert "workspace" in k3.lib.k3moe_last_error().decode()
    assert _route(big_shape(T=0)) == 0                     # empty batch: nothing to do


def test_bank_and_layer_validation():
    s = big_shape()
    good = k3.make_bank(k3.FMT_MXFP4, 896, 7168, 2048, FAKE, FAKE, FAKE, FAKE)
    bf = k3.make_bank(k3.FMT_BF16, 896, 7168, 2048, FAKE, FAKE, FAKE, FAKE)
    wrong_n = k3.make_bank(k3.FMT_MXFP4, 895, 7168, 2048, FAKE, FAKE, FAKE, FAKE)
    no_scale = k3.make_bank(k3.FMT_MXFP4, 896, 7168, 2048, FAKE, None, FAKE, FAKE)

    def ffn(bank):
        return k3.lib.k3moe_expert_ffn(ctypes.byref(s), ctypes.byref(bank), FAKE, FAKE, FAKE,
                                       FAKE, FAKE * 256, 1 << 40, None)
    assert ffn(bf) == EUNSUPPORTED          # a BF16 bank takes no sorted_pair
    assert ffn(wrong_n) == EINVAL
    assert ffn(no_scale) == EINVAL
    assert k3.lib.k3moe_expert_ffn(ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, FAKE * 256,
                                   1 << 40, None) == EINVAL
    sh_ok = k3.make_bank(k3.FMT_BF16, 2, 7168, 2048, FAKE, None, FAKE, None)
    sh_bad = k3.make_bank(k3.FMT_MXFP4, 2, 7168, 2048, FAKE, FAKE, FAKE, FAKE)
    assert k3.lib.k3moe_shared_ffn(ctypes.byref(s), ctypes.byref(sh_bad), FAKE, FAKE,
                                   FAKE * 256, 1 << 40, None) == EUNSUPPORTED
    # shared mode of k3moe_expert_ffn: a BF16 bank and sorted_pair NULL; an
    # MXFP4 bank needs sorted_pair
    def ffn_shared(bank, sp=None, shape=s, y=FAKE, ws=(FAKE * 256, 1 << 40)):
        return k3.lib.k3moe_expert_ffn(ctypes.byref(shape), ctypes.byref(bank), FAKE, None, sp,
                                       y, ws[0], ws[1], None)
    assert ffn_shared(good) == EUNSUPPORTED
    assert ffn_shared(bf) == EINVAL                        # 896 experts: not the 2 shared ones
    assert ffn_shared(sh_ok, y=None) == EINVAL
    assert ffn_shared(sh_ok, ws=(None, 0)) == EWORKSPACE
    assert ffn_shared(sh_ok, shape=big_shape(T=0)) == 0
    assert ffn_shared(sh_ok, shape=big_shape(n_shared=0, f_shared=0)) == EINVAL
    w_ok = k3.make_weights(FAKE, good, sh_ok)

    def layer(weights, x=FAKE, out=FAKE, ws=(FAKE * 256, 1 << 40), shape=s):
        return k3.lib.k3moe_layer(ctypes.byref(shape), ctypes.byref(weights), x, out, None,
                                  ws[0], ws[1], None)
    assert layer(k3.make_weights(None, good, sh_ok)) == EINVAL
    assert layer(k3.make_weights(FAKE, good, sh_ok, router_bias=FAKE)) == EINVAL   # softmax
    assert layer(k3.make_weights(FAKE, bf, sh_ok)) == EUNSUPPORTED
    assert layer(k3.make_weights(FAKE, good, k3.make_bank(k3.FMT_BF16, 1, 7168, 2048, FAKE, None, FAKE, None))) == EINVAL
    assert layer(w_ok, out=None) == EINVAL
    assert layer(w_ok, x=FAKE + 4) == EALIGN
    assert layer(w_ok, ws=(FAKE * 256, 1024)) == EWORKSPACE
    assert layer(w_ok, shape=big_shape(T=0)) == 0
    assert k3.lib.k3moe_layer(ctypes.byref(s), None, FAKE, FAKE, None, FAKE * 256, 1 << 40,
                              None) == EINVAL


def test_noalloc_layer_validation():
    """The no-allocation layer validates like k3moe_layer before touching any
    device, and refuses a call whose workspace would not fit its buffer."""
    good = k3.make_bank(k3.FMT_MXFP4, 896, 7168, 2048, FAKE, FAKE, FAKE, FAKE)
    sh_ok = k3.make_bank(k3.FMT_BF16, 2, 7168, 2048, FAKE, None, FAKE, None)
    w = k3.make_weights(FAKE, good, sh_ok)

    def call(shape, weights=w, x=FAKE, out=FAKE):
        return k3.lib.k3moe_layer_noalloc(ctypes.byref(shape), ctypes.byref(weights), x, out,
                                          None, None)
    assert k3.k3moe_workspace_bytes(big_shape(T=103), k3.OP_LAYER) <= k3.NOALLOC_SCRATCH_BYTES
    assert k3.k3moe_workspace_bytes(big_shape(T=104), k3.OP_LAYER) > k3.NOALLOC_SCRATCH_BYTES
    assert call(big_shape(T=104)) == EWORKSPACE
    assert "workspace" in k3.lib.k3moe_last_error().decode()
    assert call(big_shape(T=4096)) == EWORKSPACE
    assert call(big_shape(T=1), x=None) == EINVAL
    assert call(big_shape(T=1), out=FAKE + 4) == EALIGN
    assert call(big_shape(T=1), weights=k3.make_weights(None, good, sh_ok)) == EINVAL
    assert call(big_shape(T=1, d=7000)) == ESHAPE
    assert call(big_shape(T=0)) == 0


def test_rvq_validation():
    """RVQ3 experts: the shape names the routed format, which the bank must
    match; d and f multiples of 128; exact activations only; the down half
    alone is refused (its slice partial sums need k3moe_expert_ffn's
    workspace); the expert workspace holds the partial sums."""
    rvq = k3.make_bank(k3.FMT_RVQ3, 896, 7168, 2048, FAKE, FAKE, FAKE, FAKE)
    mx = k3.make_bank(k3.FMT_MXFP4, 896, 7168, 2048, FAKE, FAKE, FAKE, FAKE)
    s_rvq = big_shape(routed_format=k3.FMT_RVQ3)

    def ffn(shape, bank):
        return k3.lib.k3moe_expert_ffn(ctypes.byref(shape), ctypes.byref(bank), FAKE, FAKE, FAKE,
                                       FAKE, FAKE * 256, 1 << 40, None)
    assert ffn(big_shape(), rvq) == EINVAL            # bank RVQ3, shape MXFP4
    assert ffn(s_rvq, mx) == EINVAL
    assert ffn(big_shape(routed_format=7), rvq) == EUNSUPPORTED
    assert ffn(big_shape(routed_format=k3.FMT_RVQ3, d=7168 + 64), rvq) == ESHAPE
    assert ffn(big_shape(routed_format=k3.FMT_RVQ3, act=k3.ACT_MXFP4), rvq) == EUNSUPPORTED
    assert k3.lib.k3moe_expert_down(ctypes.byref(s_rvq), ctypes.byref(rvq), FAKE, FAKE, FAKE,
                                    None) == EUNSUPPORTED
    # h (16 pairs x f fp32) and 16 pairs x 2f rows x d/128 slice sums of 4 bytes
    assert k3.k3moe_workspace_bytes(s_rvq, k3.OP_EXPERT_FFN) >= 16 * 2048 * 4 + 16 * 4096 * 56 * 4


def test_permute_and_combine_validation():
    s = big_shape(T=4)
    assert k3.lib.k3moe_permute(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, None, FAKE * 256,
                                1 << 40, None) == EINVAL
    assert k3.lib.k3moe_permute(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                                None) == EWORKSPACE
    assert k3.lib.k3moe_combine(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None) == EINVAL
    assert k3.lib.k3moe_combine(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE + 2, FAKE, None) == EALIGN


def test_status_strings_and_path_class():
    for code in range(7):
        assert k3.lib.k3moe_status_str(code)
    assert k3.k3moe_path_class(big_shape(T=1)) == k3.PATH_GEMV
    assert k3.k3moe_path_class(big_shape(T=31)) == k3.PATH_GEMV
    assert k3.k3moe_path_class(big_shape(T=32)) == k3.PATH_MFMA
    assert k3.k3moe_path_class(big_shape(T=4096)) == k3.PATH_MFMA
    # the matrix-core class needs bf16 activations and d % 512, f % 512
    assert k3.k3moe_path_class(big_shape(T=4096, x_dtype=k3.F32)) == k3.PATH_GEMV
    assert k3.k3moe_path_class(big_shape(T=4096, d=7168 + 128)) == k3.PATH_GEMV
    assert k3.k3moe_path_class(big_shape(T=4096, f=2048 + 64)) == k3.PATH_GEMV
    assert k3.k3moe_path_class(big_shape(T=4096, f=2048 + 256)) == k3.PATH_GEMV
    assert k3.k3moe_path_class(big_shape(T=4096, d=0)) == k3.PATH_GEMV
    # shapes of the GEMV class at any batch size, whatever the shared width
    assert k3.k3moe_path_class(big_shape(T=32, f=1056)) == k3.PATH_GEMV
    assert k3.k3moe_path_class(big_shape(T=32, d=768, f_shared=256)) == k3.PATH_GEMV


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it exits with a message,
    before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
