"""Python binding of libbfp: BFP4/BFP8 weight-streaming matmuls for AMD MI355X (gfx950).

A thin ctypes layer over the C ABI declared in ``include/libbfp.h``. It only marshals
arguments: every step of the computation runs in the HIP kernels of ``libbfp.so``. PyTorch
provides device memory and streams. There is no CPU fallback: if ``libbfp.so`` is missing or
fails to load, every call raises.

Functions keep the C names (``bfp_quantize``, ``bfp_dequantize``, ``bfp_gemm``,
``bfp_gemm_argmax``, ``bfp_kv_append``, ``bfp_attn_decode``, ``bfp_moe_route``, ``bfp_moe_dispatch``, ``bfp_moe_workspace_bytes``, ``bfp_moe_forward``)
and take torch tensors where the C call takes device pointers.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "BFP4", "BFP8", "BfpError", "BfpMatrix", "MoeLayer", "lib", "library_path",
    "bfp_quantize", "bfp_dequantize", "bfp_gemm", "bfp_gemm_workspace_bytes", "bfp_gemm_argmax",
    "bfp_gemm_argmax_workspace_bytes", "bfp_moe_route", "bfp_moe_dispatch", "KvCache", "KV_V_BFP8", "KV_V_BFP4_HADAMARD", "bfp_kv_append",
    "bfp_attn_decode", "bfp_attn_decode_workspace_bytes",
    "bfp_moe_workspace_bytes", "bfp_moe_forward", "bfp_moe_forward_noalloc", "MOE_NOALLOC_SCRATCH_BYTES",
    "exp_bytes", "code_bytes",
]

BFP4 = 4
BFP8 = 8
DT_F32 = 0
DT_BF16 = 1
EPI_NONE = 0
EPI_SWIGLU = 1
BATCH_INVARIANT = 0x100

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libbfp.so")


class BfpError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


class _Tensor(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("exp", ctypes.c_void_p), ("code", ctypes.c_void_p)]


class _MoeLayer(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", _Tensor), ("up", _Tensor), ("down", _Tensor),
                ("sh_gate", _Tensor), ("sh_up", _Tensor), ("sh_down", _Tensor),
                ("sh_gate_w", ctypes.c_void_p)]


class _KvCache(ctypes.Structure):
    _fields_ = [("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("max_tokens", ctypes.c_int64),
                ("k_exp", ctypes.c_void_p), ("k_code", ctypes.c_void_p), ("v_exp", ctypes.c_void_p),
                ("v_code", ctypes.c_void_p), ("v_format", ctypes.c_int32)]


_LIB = None

# name -> (restype, argtypes)
_SIGS = {
    "bfp_version": (ctypes.c_int32, []),
    "bfp_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "bfp_exp_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "bfp_code_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64]),
    "bfp_quantize": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "bfp_dequantize": (ctypes.c_int32, [ctypes.POINTER(_Tensor), ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "bfp_gemm_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                                  ctypes.c_int64]),
    "bfp_gemm": (ctypes.c_int32, [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]),
    "bfp_gemm_argmax_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Tensor), ctypes.c_int64]),
    "bfp_gemm_argmax": (ctypes.c_int32, [ctypes.POINTER(_Tensor), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "bfp_kv_append": (ctypes.c_int32, [ctypes.POINTER(_KvCache), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "bfp_attn_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_KvCache), ctypes.c_int32, ctypes.c_int64]),
    "bfp_attn_decode": (ctypes.c_int32, [ctypes.POINTER(_KvCache), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "bfp_moe_route_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_MoeLayer), ctypes.c_int64]),
    "bfp_moe_route": (ctypes.c_int32, [ctypes.POINTER(_MoeLayer), ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]),
    "bfp_moe_dispatch": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "bfp_moe_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_MoeLayer), ctypes.c_int64]),
    "bfp_moe_forward": (ctypes.c_int32, [ctypes.POINTER(_MoeLayer), ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "bfp_moe_forward_noalloc": (ctypes.c_int32, [ctypes.POINTER(_MoeLayer), ctypes.c_void_p, ctypes.c_int64,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]),
}


def lib() -> ctypes.CDLL:
    """Load libbfp.so (once). Raises if it is missing: there is no fallback path."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libbfp.so not built ({path}); run `python -m block_float_quantized_amd.build`")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise BfpError(fn, status, lib().bfp_status_str(status).decode())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return t.data_ptr()


def exp_bytes(n: int, k: int) -> int:
    return int(lib().bfp_exp_bytes(n, k))


def code_bytes(fmt: int, n: int, k: int) -> int:
    return int(lib().bfp_code_bytes(fmt, n, k))


@dataclass
class BfpMatrix:
    """A BFP matrix in device memory: exponent plane [n][k/16] and code plane (uint8)."""
    fmt: int
    n: int
    k: int
    exp: torch.Tensor
    code: torch.Tensor

    def view(self) -> _Tensor:
        return _Tensor(self.fmt, self.n, self.k, _ptr(self.exp), _ptr(self.code))

    def rows(self, r0: int, r1: int) -> "BfpMatrix":
        """Rows [r0, r1) as a view (no copy)."""
        nb = self.k // 16
        cpr = self.code.numel() // self.n
        return BfpMatrix(self.fmt, r1 - r0, self.k, self.exp.view(-1)[r0 * nb:r1 * nb],
                         self.code.view(-1)[r0 * cpr:r1 * cpr])

    @property
    def nbytes(self) -> int:
        return self.exp.numel() + self.code.numel()


def empty_matrix(fmt: int, n: int, k: int, device="cuda") -> BfpMatrix:
    exp = torch.empty(exp_bytes(n, k), dtype=torch.uint8, device=device)
    code = torch.empty(code_bytes(fmt, n, k), dtype=torch.uint8, device=device)
    return BfpMatrix(fmt, n, k, exp, code)


def bfp_quantize(fmt: int, w: torch.Tensor, out: BfpMatrix | None = None, stream=None) -> BfpMatrix:
    """Encode a device fp32 [n][k] matrix whose rows are contiguous (any row stride; the
    call synchronizes the stream)."""
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a row-major fp32 [n][k] device tensor")
    n, k = w.shape
    if out is None:
        out = empty_matrix(fmt, n, k, w.device)
    _check("bfp_quantize", lib().bfp_quantize(fmt, _ptr(w), n, k, w.stride(0), _ptr(out.exp), _ptr(out.code),
                                              _stream(stream)))
    return out


def bfp_dequantize(w: BfpMatrix, dtype=torch.float32, stream=None) -> torch.Tensor:
    dt = DT_BF16 if dtype == torch.bfloat16 else DT_F32
    out = torch.empty((w.n, w.k), dtype=dtype, device=w.exp.device)
    v = w.view()
    _check("bfp_dequantize", lib().bfp_dequantize(ctypes.byref(v), dt, _ptr(out), _stream(stream)))
    return out


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def bfp_gemm_workspace_bytes(w: BfpMatrix, m: int, w_up: BfpMatrix | None = None) -> int:
    vw = w.view()
    vu = w_up.view() if w_up is not None else None
    return int(lib().bfp_gemm_workspace_bytes(ctypes.byref(vw), ctypes.byref(vu) if vu is not None else None, m))


def bfp_gemm(w: BfpMatrix, x: torch.Tensor, w_up: BfpMatrix | None = None, out_dtype=torch.float32,
             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
             batch_invariant: bool = False) -> torch.Tensor:
    """y = x W^T (or silu(x W^T) * (x Wup^T) when w_up is given); x is [m][k], m <= 32.

    ``workspace`` (uint8 device tensor of at least bfp_gemm_workspace_bytes bytes) is made
    here when not given. ``batch_invariant``: row i is the same bits for every m.
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a row-major [m][k] device tensor")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.n), dtype=out_dtype, device=x.device)
    vw = w.view()
    vu = w_up.view() if w_up is not None else None
    if workspace is None:
        need = bfp_gemm_workspace_bytes(w, m, w_up)
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    st = lib().bfp_gemm(ctypes.byref(vw), ctypes.byref(vu) if vu is not None else None,
                        (EPI_SWIGLU if w_up is not None else EPI_NONE) | (BATCH_INVARIANT if batch_invariant else 0),
                        _ptr(x), _dt(x), m, x.stride(0), _ptr(out), _dt(out), out.stride(0),
                        _ptr(workspace), workspace.numel(), _stream(stream))
    _check("bfp_gemm", st)
    return out


def bfp_gemm_argmax_workspace_bytes(w: BfpMatrix, m: int) -> int:
    return int(lib().bfp_gemm_argmax_workspace_bytes(ctypes.byref(w.view()), m))


def bfp_gemm_argmax(w: BfpMatrix, x: torch.Tensor, idx: torch.Tensor | None = None, val: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None,
                    batch_invariant: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Per row of x ([m][k] bf16, m <= 32): (int32 column, fp32 value) of the largest entry of
    x W^T, the first such column on ties, without materialising x W^T. ``batch_invariant`` as
    in bfp_gemm.

    ``workspace`` (uint8 device tensor of at least bfp_gemm_argmax_workspace_bytes bytes) is
    made here when not given.
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a row-major [m][k] device tensor")
    m = x.shape[0]
    if idx is None:
        idx = torch.empty((m,), dtype=torch.int32, device=x.device)
    if val is None:
        val = torch.empty((m,), dtype=torch.float32, device=x.device)
    if workspace is None:
        need = bfp_gemm_argmax_workspace_bytes(w, m)
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    st = lib().bfp_gemm_argmax(ctypes.byref(w.view()), _ptr(x), _dt(x), m, x.stride(0),
                               BATCH_INVARIANT if batch_invariant else 0, _ptr(idx), _ptr(val),
                               _ptr(workspace), workspace.numel(), _stream(stream))
    _check("bfp_gemm_argmax", st)
    return idx, val


KV_V_BFP8 = 0               # V stored in BFP8 like K
KV_V_BFP4_HADAMARD = 1      # V rotated by the orthonormal Hadamard transform, stored in BFP4


@dataclass
class KvCache:
    """A BFP KV cache in device memory (see bfp_kv_cache in include/libbfp.h)."""
    kv_heads: int
    head_dim: int
    max_tokens: int
    k_exp: torch.Tensor
    k_code: torch.Tensor
    v_exp: torch.Tensor
    v_code: torch.Tensor
    v_format: int = KV_V_BFP8

    @staticmethod
    def empty(kv_heads: int, head_dim: int, max_tokens: int, device="cuda", v_format: int = KV_V_BFP8) -> "KvCache":
        rows = kv_heads * max_tokens
        ne, nc = exp_bytes(rows, head_dim), code_bytes(BFP8, rows, head_dim)
        nv = code_bytes(BFP4 if v_format == KV_V_BFP4_HADAMARD else BFP8, rows, head_dim)
        z = lambda n: torch.zeros((n,), dtype=torch.uint8, device=device)
        return KvCache(kv_heads, head_dim, max_tokens, z(ne), z(nc), z(ne), z(nv), v_format)

    def view(self) -> _KvCache:
        return _KvCache(self.kv_heads, self.head_dim, self.max_tokens, _ptr(self.k_exp), _ptr(self.k_code),
                        _ptr(self.v_exp), _ptr(self.v_code), self.v_format)

    @property
    def nbytes(self) -> int:
        return self.k_exp.numel() + self.k_code.numel() + self.v_exp.numel() + self.v_code.numel()


def bfp_kv_append(cache: KvCache, k: torch.Tensor, v: torch.Tensor, pos: int, stream=None) -> None:
    """Encode k, v ([n][kv_heads][head_dim], fp32 or bf16) into token slots pos .. pos + n - 1."""
    if k.shape != v.shape or k.dtype != v.dtype or not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k and v must be contiguous [n][kv_heads][head_dim] tensors of one dtype")
    st = lib().bfp_kv_append(ctypes.byref(cache.view()), _ptr(k), _ptr(v), _dt(k), pos, k.shape[0], _stream(stream))
    _check("bfp_kv_append", st)


def bfp_attn_decode_workspace_bytes(cache: KvCache, q_heads: int, seq_len: int) -> int:
    return int(lib().bfp_attn_decode_workspace_bytes(ctypes.byref(cache.view()), q_heads, seq_len))


def bfp_attn_decode(cache: KvCache, q: torch.Tensor, seq_len: int, scale: float, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Single-token attention of q ([q_heads][head_dim], fp32 or bf16) over the first seq_len
    cached tokens; returns fp32 [q_heads][head_dim]."""
    if q.dim() != 2 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [q_heads][head_dim] tensor")
    hq = q.shape[0]
    if out is None:
        out = torch.empty((hq, cache.head_dim), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = bfp_attn_decode_workspace_bytes(cache, hq, seq_len)
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    st = lib().bfp_attn_decode(ctypes.byref(cache.view()), _ptr(q), _dt(q), hq, seq_len, float(scale), _ptr(out),
                               _ptr(workspace), workspace.numel(), _stream(stream))
    _check("bfp_attn_decode", st)
    return out


@dataclass
class MoeLayer:
    """Device tensors of one MoE layer (see bfp_moe_layer in include/libbfp.h)."""
    n_experts: int
    top_k: int
    hidden: int
    inter: int
    router_w: torch.Tensor            # bf16 bits as int16/uint16 or bfloat16 [E][hidden]
    router_bias: torch.Tensor | None  # fp32 [E]
    gate: BfpMatrix
    up: BfpMatrix
    down: BfpMatrix
    sh_gate: BfpMatrix | None
    sh_up: BfpMatrix | None
    sh_down: BfpMatrix | None
    sh_gate_w: torch.Tensor | None    # bf16 [hidden]

    def view(self) -> _MoeLayer:
        absent = _Tensor(0, 0, 0, None, None)
        return _MoeLayer(self.n_experts, self.top_k, self.hidden, self.inter,
                         _ptr(self.router_w), _ptr(self.router_bias),
                         self.gate.view(), self.up.view(), self.down.view(),
                         self.sh_gate.view() if self.sh_gate is not None else absent,
                         self.sh_up.view() if self.sh_up is not None else absent,
                         self.sh_down.view() if self.sh_down is not None else absent,
                         _ptr(self.sh_gate_w))


def bfp_moe_route(layer: MoeLayer, x: torch.Tensor, stream=None):
    """Routing step: returns (ids int32 [m][top_k], weights fp32 [m][top_k], g fp32 [m])."""
    m = x.shape[0]
    ids = torch.empty((m, layer.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((m, layer.top_k), dtype=torch.float32, device=x.device)
    g = torch.empty((m,), dtype=torch.float32, device=x.device)
    v = layer.view()
    need = int(lib().bfp_moe_route_workspace_bytes(ctypes.byref(v), m))
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    _check("bfp_moe_route", lib().bfp_moe_route(ctypes.byref(v), _ptr(x), m, _ptr(ids), _ptr(w), _ptr(g),
                                                _ptr(ws), ws.numel(), _stream(stream)))
    return ids, w, g


def bfp_moe_dispatch(ids: torch.Tensor, n_experts: int, stream=None):
    """Counting sort by expert: returns (counts [E], offsets [E+1], perm [m*top_k]) int32."""
    m, top_k = ids.shape
    counts = torch.empty((n_experts,), dtype=torch.int32, device=ids.device)
    offsets = torch.empty((n_experts + 1,), dtype=torch.int32, device=ids.device)
    perm = torch.empty((m * top_k,), dtype=torch.int32, device=ids.device)
    _check("bfp_moe_dispatch", lib().bfp_moe_dispatch(_ptr(ids), m, top_k, n_experts, _ptr(counts),
                                                      _ptr(offsets), _ptr(perm), _stream(stream)))
    return counts, offsets, perm


def bfp_moe_workspace_bytes(layer: MoeLayer, m: int) -> int:
    v = layer.view()
    return int(lib().bfp_moe_workspace_bytes(ctypes.byref(v), m))


def bfp_moe_forward(layer: MoeLayer, x: torch.Tensor, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, topk_ids: torch.Tensor | None = None,
                    topk_w: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = MoE(x) for x bf16 [m][hidden]; returns fp32 [m][hidden]."""
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, layer.hidden), dtype=torch.float32, device=x.device)
    need = bfp_moe_workspace_bytes(layer, m)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    v = layer.view()
    st = lib().bfp_moe_forward(ctypes.byref(v), _ptr(x), m, _ptr(out), _ptr(topk_ids), _ptr(topk_w),
                               _ptr(workspace), workspace.numel(), _stream(stream))
    _check("bfp_moe_forward", st)
    return out


MOE_NOALLOC_SCRATCH_BYTES = 8 << 20


def bfp_moe_forward_noalloc(layer: MoeLayer, x: torch.Tensor, out: torch.Tensor, topk_ids: torch.Tensor | None = None,
                            topk_w: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode MoE (m <= 32) on the library's own device scratch: allocates nothing (the caller
    passes the output). Calls that overlap on one device race."""
    v = layer.view()
    st = lib().bfp_moe_forward_noalloc(ctypes.byref(v), _ptr(x), x.shape[0], _ptr(out), _ptr(topk_ids),
                                       _ptr(topk_w), _stream(stream))
    _check("bfp_moe_forward_noalloc", st)
    return out
