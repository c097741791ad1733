"""The C-ABI library loads, exports every function include/libbfp.h declares, and rejects
bad arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

import block_float_quantized_amd as bfq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "libbfp.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(bfp_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert "bfp_gemm" in names and "bfp_quantize" in names and "bfp_moe_forward" in names
    handle = ctypes.CDLL(bfq.library_path())
    for name in names:
        assert hasattr(handle, name), name
    # the binding knows every declared function
    assert set(names) <= set(bfq._SIGS)


def test_status_strings_and_sizes():
    lib = bfq.lib()
    assert lib.bfp_status_str(0) == b"ok"
    assert lib.bfp_status_str(4).startswith(b"non-finite")
    assert lib.bfp_status_str(99) == b"unknown status"
    assert lib.bfp_exp_bytes(5120, 17408) == 5120 * 1088
    assert lib.bfp_code_bytes(4, 5120, 17408) == 5120 * 8704
    assert lib.bfp_code_bytes(8, 2048, 2048) == 2048 * 2048
    assert lib.bfp_code_bytes(5, 16, 16) == 0


def _tensor(fmt=4, n=32, k=64, exp=16, code=16):
    return bfq._Tensor(fmt, n, k, exp, code)


def test_host_validation_before_any_launch():
    lib = bfq.lib()
    # quantize
    assert lib.bfp_quantize(5, 16, 4, 16, 16, 16, 16, None) == 1      # unknown format
    assert lib.bfp_quantize(4, None, 4, 16, 16, 16, 16, None) == 1     # null pointer
    assert lib.bfp_quantize(4, 16, 4, 24, 24, 16, 16, None) == 2       # k % 16
    assert lib.bfp_quantize(4, 16, 0, 16, 16, 16, 16, None) == 2       # n = 0
    assert lib.bfp_quantize(4, 16, 4, 32, 16, 16, 16, None) == 2       # row stride below k
    assert lib.bfp_quantize(4, 18, 4, 16, 16, 16, 16, None) == 3       # misaligned input
    assert lib.bfp_quantize(4, 16, 4, 16, 18, 16, 16, None) == 3       # row stride not 16-byte aligned
    # dequantize
    t = _tensor(k=40)
    assert lib.bfp_dequantize(ctypes.byref(t), 0, 16, None) == 2
    t = _tensor(code=24)
    assert lib.bfp_dequantize(ctypes.byref(t), 0, 16, None) == 3
    t = _tensor()
    assert lib.bfp_dequantize(ctypes.byref(t), 7, 16, None) == 1
    # gemm
    w = _tensor()
    assert lib.bfp_gemm(ctypes.byref(w), None, 0, 16, 1, 0, 64, 16, 0, 32, None, 0, None) == 2     # m = 0
    assert lib.bfp_gemm(ctypes.byref(w), None, 0, 16, 1, 33, 64, 16, 0, 32, None, 0, None) == 2    # m > 32
    assert lib.bfp_gemm(ctypes.byref(w), None, 0, 16, 1, 1, 32, 16, 0, 32, None, 0, None) == 2     # ldx < k
    assert lib.bfp_gemm(ctypes.byref(w), None, 0, 16, 1, 1, 68, 16, 0, 32, None, 0, None) == 3     # ldx*2 % 16
    assert lib.bfp_gemm(ctypes.byref(w), None, 1, 16, 1, 1, 64, 16, 0, 32, None, 0, None) != 0     # SwiGLU without up
    u = _tensor(n=16)
    assert lib.bfp_gemm(ctypes.byref(w), ctypes.byref(u), 1, 16, 1, 1, 64, 16, 0, 32, None, 0, None) == 2
    u = _tensor(fmt=8)
    assert lib.bfp_gemm(ctypes.byref(w), ctypes.byref(u), 1, 16, 1, 1, 64, 16, 0, 32, None, 0, None) == 1
    assert lib.bfp_gemm(ctypes.byref(w), ctypes.byref(w), 0, 16, 1, 1, 64, 16, 0, 32, None, 0, None) == 1
    assert lib.bfp_gemm(ctypes.byref(w), None, 3, 16, 1, 1, 64, 16, 0, 32, None, 0, None) == 1
    # a shape that is cut into K slices needs the workspace it reports
    big = _tensor(n=64, k=16384)
    need = lib.bfp_gemm_workspace_bytes(ctypes.byref(big), None, 2)
    assert need > 0
    assert lib.bfp_gemm(ctypes.byref(big), None, 0, 16, 1, 2, 16384, 16, 0, 64, None, 0, None) == 5
    assert lib.bfp_gemm(ctypes.byref(big), None, 0, 16, 1, 2, 16384, 16, 0, 64, 16, need - 1, None) == 5
    assert lib.bfp_gemm_workspace_bytes(ctypes.byref(big), None, 0) == 0             # m out of range
    # greedy argmax: candidates per row of x need workspace even for one row
    lm = _tensor(fmt=8, n=151936, k=2048)
    need = lib.bfp_gemm_argmax_workspace_bytes(ctypes.byref(lm), 1)
    assert need >= 151936 // 64 * 8
    assert lib.bfp_gemm_argmax_workspace_bytes(ctypes.byref(lm), 33) == 0
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 0, 2048, 0, 16, 16, 16, need, None) == 2      # m = 0
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 33, 2048, 0, 16, 16, 16, need, None) == 2     # m > 32
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 0, 1, 2048, 0, 16, 16, 16, need, None) == 7      # fp32 x
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 2, 1, 2048, 0, 16, 16, 16, need, None) == 1      # bad dtype
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 1, 2040, 0, 16, 16, 16, need, None) == 2      # ldx < k
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 24, 1, 1, 2048, 0, 16, 16, 16, need, None) == 3      # misaligned x
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 1, 2048, 0, None, 16, 16, need, None) == 1    # no idx
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 1, 2048, 0, 16, 16, None, need, None) == 1    # no workspace
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 1, 2048, 0, 16, 16, 16, need - 1, None) == 5  # too small
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 1, 2048, 0, 16, 16, 24, need, None) == 3      # misaligned ws
    assert lib.bfp_gemm_argmax(ctypes.byref(lm), 16, 1, 1, 2048, 2, 16, 16, 16, need, None) == 1      # unknown flag
    # batch-invariant flag: other high bits of the epilogue are rejected; the workspace query
    # covers the matrix-core kernel at m = 1
    assert lib.bfp_gemm(ctypes.byref(w), None, 0x200, 16, 1, 1, 64, 16, 0, 32, None, 0, None) == 1
    assert lib.bfp_gemm(ctypes.byref(big), None, 0x100, 16, 1, 1, 16384, 16, 0, 64, None, 0, None) == 5
    assert lib.bfp_gemm_workspace_bytes(ctypes.byref(big), None, 1) > 0


def _fake_layer(hidden, inter, n_exp=256, top_k=8):
    t = lambda n, k: bfq._Tensor(4, n, k, 16, 16)
    return bfq._MoeLayer(n_exp, top_k, hidden, inter, 16, None, t(n_exp * inter, hidden), t(n_exp * inter, hidden),
                         t(n_exp * hidden, inter), t(inter, hidden), t(inter, hidden), t(hidden, inter), 16)


def test_moe_host_validation():
    """Shapes the many-token kernels cannot address with 32-bit offsets are refused on the
    host (BFP_E_UNSUPPORTED) before the routing or dispatch kernels are queued."""
    lib = bfq.lib()
    L = _fake_layer(2048, 14592)          # (8192 * 8 + 8192) * 14592 * 2 B of h >= 2^31
    assert lib.bfp_moe_forward(ctypes.byref(L), 16, 8192, 16, None, None, 16, 1 << 40, None) == 7
    assert lib.bfp_moe_forward(ctypes.byref(L), 16, 32, 16, None, None, None, 0, None) == 5   # decode: workspace
    L = _fake_layer(2048, 96)             # inter not a multiple of the 128-value K step
    assert lib.bfp_moe_forward(ctypes.byref(L), 16, 64, 16, None, None, 16, 1 << 40, None) == 7
    L = _fake_layer(2048, 512)
    assert lib.bfp_moe_forward(ctypes.byref(L), 16, 8193, 16, None, None, 16, 1 << 40, None) == 2  # m
    assert lib.bfp_moe_forward(ctypes.byref(L), 24, 4, 16, None, None, 16, 1 << 40, None) == 3    # x alignment
    bad = _fake_layer(2048, 512, top_k=9)
    assert lib.bfp_moe_forward(ctypes.byref(bad), 16, 4, 16, None, None, 16, 1 << 40, None) == 2
    # the no-allocation decode variant: decode sizes only, and a layer whose decode workspace
    # fits the static scratch
    L = _fake_layer(2048, 512)
    assert lib.bfp_moe_forward_noalloc(ctypes.byref(L), 16, 33, 16, None, None, None) == 7
    assert lib.bfp_moe_workspace_bytes(ctypes.byref(L), 32) <= bfq.MOE_NOALLOC_SCRATCH_BYTES
    big = _fake_layer(8192, 512)
    assert lib.bfp_moe_workspace_bytes(ctypes.byref(big), 32) > bfq.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.bfp_moe_forward_noalloc(ctypes.byref(big), 16, 32, 16, None, None, None) == 5
    assert lib.bfp_moe_forward_noalloc(ctypes.byref(L), 24, 4, 16, None, None, None) == 3
    huge = bfq._Tensor(4, 1 << 31, 64, 16, 16)      # rows beyond the kernels' int range
    assert lib.bfp_dequantize(ctypes.byref(huge), 0, 16, None) == 2


def test_kv_cache_host_validation():
    lib = bfq.lib()
    c = bfq._KvCache(2, 256, 100, 16, 16, 16, 16)
    assert lib.bfp_kv_append(ctypes.byref(c), 16, 16, 0, 90, 11, None) == 2                   # past the slots
    assert lib.bfp_kv_append(ctypes.byref(c), 16, 16, 5, 0, 1, None) == 1                     # bad dtype
    assert lib.bfp_kv_append(ctypes.byref(c), 24, 16, 0, 0, 1, None) == 3                    # misaligned k
    bad = bfq._KvCache(2, 96, 100, 16, 16, 16, 16)
    assert lib.bfp_kv_append(ctypes.byref(bad), 16, 16, 0, 0, 1, None) == 2                   # head_dim
    fmt = bfq._KvCache(2, 256, 100, 16, 16, 16, 16, 2)
    assert lib.bfp_kv_append(ctypes.byref(fmt), 16, 16, 0, 0, 1, None) == 1                   # v_format
    assert lib.bfp_attn_decode_workspace_bytes(ctypes.byref(fmt), 16, 100) == 0
    rot = bfq._KvCache(2, 256, 100, 16, 16, 16, 16, bfq.KV_V_BFP4_HADAMARD)
    assert lib.bfp_attn_decode_workspace_bytes(ctypes.byref(rot), 16, 100) > 0
    assert lib.bfp_kv_append(ctypes.byref(rot), 16, 16, 0, 90, 11, None) == 2
    need = lib.bfp_attn_decode_workspace_bytes(ctypes.byref(c), 16, 100)
    assert need > 0 and lib.bfp_attn_decode_workspace_bytes(ctypes.byref(c), 16, 101) == 0
    assert lib.bfp_attn_decode(ctypes.byref(c), 16, 0, 16, 0, 1.0, 16, 16, need, None) == 2   # seq_len 0
    assert lib.bfp_attn_decode(ctypes.byref(c), 16, 0, 6, 10, 1.0, 16, 16, need, None) == 7   # group 3
    assert lib.bfp_attn_decode(ctypes.byref(c), 16, 0, 5, 10, 1.0, 16, 16, need, None) == 2   # not a multiple
    assert lib.bfp_attn_decode(ctypes.byref(c), 16, 0, 16, 100, 1.0, 16, 16, need - 1, None) == 5
    assert lib.bfp_attn_decode(ctypes.byref(c), 16, 0, 16, 100, float("nan"), 16, 16, need, None) == 1
    assert lib.bfp_attn_decode(ctypes.byref(c), 16, 0, 16, 100, 1.0, 20, 16, need, None) == 3  # misaligned out


def test_python_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bfq, "_LIB", None)
    monkeypatch.setattr(bfq, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        bfq.lib()


def test_kv_cache_planes_and_format():
    """Plane sizes of both cache formats (host tensors; no device call) and the format field
    handed to the C struct."""
    for fmt, vbytes in ((bfq.KV_V_BFP8, 256), (bfq.KV_V_BFP4_HADAMARD, 128)):
        c = bfq.KvCache.empty(2, 256, 10, device="cpu", v_format=fmt)
        assert c.k_exp.numel() == c.v_exp.numel() == 2 * 10 * 16
        assert c.k_code.numel() == 2 * 10 * 256 and c.v_code.numel() == 2 * 10 * vbytes
        with pytest.raises(ValueError):                 # the binding takes device memory only
            c.view()
        assert bfq._KvCache(2, 256, 10, 16, 16, 16, 16, fmt).v_format == fmt
    # 26 / 34 of the BFP8 cache's bytes (the 27B card's 26,624 vs 34,816 bytes per token)
    a = bfq.KvCache.empty(4, 256, 16, device="cpu").nbytes
    b = bfq.KvCache.empty(4, 256, 16, device="cpu", v_format=bfq.KV_V_BFP4_HADAMARD).nbytes
    assert b * 34 == a * 26
