"""SageAttention2 forward pass for MI355X (gfx950): thin Python binding over libsage2.so.

The binding only marshals arguments: every step of the method runs in the library's HIP kernels.
PyTorch provides device memory and streams. The library is loaded on first use; if it is missing
the call fails with an error (there is no fallback implementation).

    import quantized_exact_attention_token_amd as sage2
    o = sage2.attention(q, k, v, causal=True)          # q [B, Nq, Hq, d], k/v [B, Nkv, Hkv, d]

Lower level, mirroring the C ABI of include/sage2.h:
    p = sage2.make_params(q, k, v, o, causal=...)
    ws = torch.empty(sage2.workspace_size(p), dtype=torch.uint8, device=q.device)
    sage2.quantize_smooth(p, q, k, v, ws); sage2.attn_fwd(p, ws, o)
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsage2.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(7)
F16, BF16, F32 = 0, 1, 2
NO_K_SMOOTH, NO_Q_SMOOTH, PER_BLOCK_SCALES, NO_FP32_FOLD = 1, 2, 4, 8  # sage2_flag: ablations

# Symbols the header declares; tests check that the library exports every one.
EXPORTS = ("sage2_workspace_size", "sage2_quantize_smooth", "sage2_attn_fwd", "sage2_status_string",
           "sage2_workspace_layout", "sage2_debug_attn_tiles")


class Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32),
        ("N_q", ctypes.c_int32), ("N_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_kv", ctypes.c_void_p),
        ("cu_seqlens_q_host", ctypes.c_void_p), ("cu_seqlens_kv_host", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("flags", ctypes.c_int32),
    ]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "total_bytes", "q_rows", "kv_rows", "q_blocks", "delta_len", "seq_table", "k_partial",
        "v_partial", "kbar", "sv", "sv_inv", "qbar", "qcode", "sq", "kcode", "sk", "v8",
        "delta")]


class Sage2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib():
    """Loads libsage2.so (built by quantized_exact_attention_token_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python quantized_exact_attention_token_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        PP = ctypes.POINTER(Params)
        L.sage2_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
        L.sage2_quantize_smooth.argtypes = [PP, P, P, P, P, S, P]
        L.sage2_attn_fwd.argtypes = [PP, P, S, P, P]
        L.sage2_status_string.argtypes = [ctypes.c_int]
        L.sage2_status_string.restype = ctypes.c_char_p
        L.sage2_workspace_layout.argtypes = [PP, ctypes.POINTER(WsLayout)]
        L.sage2_debug_attn_tiles.argtypes = [PP, P, S, ctypes.c_int32, ctypes.c_int32, P, P, P, P]
        for f in ("sage2_workspace_size", "sage2_quantize_smooth", "sage2_attn_fwd",
                  "sage2_workspace_layout", "sage2_debug_attn_tiles"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sage2_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise Sage2Error(status, where)


_DT = None


def _dtype_code(dt) -> int:
    import torch
    global _DT
    if _DT is None:
        _DT = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    return _DT[dt]


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_params(q, k, v, o=None, causal: bool = False, sm_scale: float = 0.0,
                cu_seqlens_q=None, cu_seqlens_kv=None, max_seqlen_q=None, max_seqlen_kv=None,
                out_dtype=None, flags: int = 0) -> Params:
    """Params for dense q [B, Nq, Hq, d], k/v [B, Nkv, Hkv, d] (any strides with channel stride 1),
    or for packed q [Tq, Hq, d], k/v [Tkv, Hkv, d] with cu_seqlens (int32, B+1, device).
    `flags` takes NO_K_SMOOTH / NO_Q_SMOOTH / PER_BLOCK_SCALES / NO_FP32_FOLD (ablations; 0 = the
    full method)."""
    p = Params()
    p.flags = int(flags)
    varlen = cu_seqlens_q is not None
    # The library takes raw device pointers and cannot tell what they point to: a host tensor, a
    # tensor on another device or a mismatched dtype would be read as if it were right.
    named = [("q", q), ("k", k), ("v", v)] + ([("o", o)] if o is not None else [])
    if varlen:
        named += [("cu_seqlens_q", cu_seqlens_q)] + (
            [("cu_seqlens_kv", cu_seqlens_kv)] if cu_seqlens_kv is not None else [])
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"q, k and v must share one dtype (got {q.dtype}, {k.dtype}, {v.dtype})")
    if tuple(k.shape) != tuple(v.shape) or k.dim() != q.dim() or k.shape[-1] != q.shape[-1]:
        raise ValueError(f"shapes do not fit: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if q.dim() != (3 if varlen else 4):
        raise ValueError("q must be [B, N, H, d], or [tokens, H, d] with cu_seqlens")
    if o is not None and tuple(o.shape) != tuple(q.shape):
        raise ValueError(f"o must have q's shape {tuple(q.shape)}, not {tuple(o.shape)}")
    for name, t in named:
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be on q's device ({q.device}), not {t.device}")
    if varlen:
        if cu_seqlens_kv is None:
            raise ValueError("cu_seqlens_kv is required with cu_seqlens_q")
        for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
            if c.dtype != torch_int32() or c.dim() != 1 or not c.is_contiguous():
                raise ValueError(f"{name} must be a contiguous 1-D int32 tensor")
        hq, hkv = q.shape[1], k.shape[1]
        cq_host = cu_seqlens_q.to("cpu", torch_int32()).contiguous()
        ck_host = cu_seqlens_kv.to("cpu", torch_int32()).contiguous()
        lq = (cq_host[1:] - cq_host[:-1])
        lk = (ck_host[1:] - ck_host[:-1])
        p.B = cq_host.numel() - 1
        p.N_q = int(max_seqlen_q if max_seqlen_q is not None else max(1, int(lq.max())))
        p.N_kv = int(max_seqlen_kv if max_seqlen_kv is not None else max(1, int(lk.max())))
        p.cu_seqlens_q = cu_seqlens_q.data_ptr()
        p.cu_seqlens_kv = cu_seqlens_kv.data_ptr()
        p.cu_seqlens_q_host = cq_host.data_ptr()
        p.cu_seqlens_kv_host = ck_host.data_ptr()
        p._keep = (cq_host, ck_host)  # host copies must outlive the params
        strides = lambda t: (0, t.stride(0), t.stride(1))
    else:
        p.B, p.N_q, hq = q.shape[0], q.shape[1], q.shape[2]
        p.N_kv, hkv = k.shape[1], k.shape[2]
        strides = lambda t: (t.stride(0), t.stride(1), t.stride(2))
    p.H_q, p.H_kv, p.d = hq, hkv, q.shape[-1]
    p.causal = int(bool(causal))
    p.in_dtype = _dtype_code(q.dtype)
    p.out_dtype = _dtype_code(out_dtype if out_dtype is not None else (o.dtype if o is not None else q.dtype))
    p.sm_scale = float(sm_scale)
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v)):
        if t.stride(-1) != 1:
            raise ValueError("channel stride must be 1")
        getattr(p, name)[:] = strides(t)
    if o is not None:
        getattr(p, "o_stride")[:] = strides(o)
    return p


def torch_int32():
    import torch
    return torch.int32


def workspace_size(p: Params) -> int:
    n = ctypes.c_size_t()
    _check(lib().sage2_workspace_size(ctypes.byref(p), ctypes.byref(n)), "sage2_workspace_size")
    return int(n.value)


def workspace_layout(p: Params) -> WsLayout:
    lay = WsLayout()
    _check(lib().sage2_workspace_layout(ctypes.byref(p), ctypes.byref(lay)), "sage2_workspace_layout")
    return lay


def quantize_smooth(p: Params, q, k, v, ws, stream=None):
    _check(lib().sage2_quantize_smooth(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       ws.data_ptr(), ws.numel() * ws.element_size(),
                                       _stream_ptr(stream)), "sage2_quantize_smooth")


def attn_fwd(p: Params, ws, o, stream=None):
    _check(lib().sage2_attn_fwd(ctypes.byref(p), ws.data_ptr(), ws.numel() * ws.element_size(),
                                o.data_ptr(), _stream_ptr(stream)), "sage2_attn_fwd")


def debug_attn_tiles(p: Params, ws, q_begin: int, q_count: int, s_out=None, p8_out=None, o=None,
                     stream=None):
    """Runs the attention kernel with its tile dump (sage2_debug_attn_tiles): INT32 S into s_out and
    P~ codes into p8_out ([B, H_q, q_count, N_kv] int32 / uint8 device tensors, either may be None),
    the output into o when given."""
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(lib().sage2_debug_attn_tiles(ctypes.byref(p), ws.data_ptr(),
                                        ws.numel() * ws.element_size(), int(q_begin), int(q_count),
                                        ptr(s_out), ptr(p8_out), ptr(o), _stream_ptr(stream)),
           "sage2_debug_attn_tiles")


def attention(q, k, v, causal: bool = False, sm_scale: float = 0.0, out_dtype=None,
              cu_seqlens_q=None, cu_seqlens_kv=None, max_seqlen_q=None, max_seqlen_kv=None,
              stream=None, flags: int = 0):
    """Allocates the output and a workspace with torch, then runs the pre-pass and the kernel."""
    import torch
    odt = out_dtype or q.dtype
    o = torch.empty(q.shape, dtype=odt, device=q.device)
    p = make_params(q, k, v, o, causal, sm_scale, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
                    max_seqlen_kv, flags=flags)
    ws = torch.empty(workspace_size(p), dtype=torch.uint8, device=q.device)
    quantize_smooth(p, q, k, v, ws, stream)
    attn_fwd(p, ws, o, stream)
    if stream is not None:
        # the kernels may still be reading the workspace (and writing o) on `stream` after this
        # returns: keep torch's allocator from handing their memory out on another stream meanwhile
        ws.record_stream(stream)
        o.record_stream(stream)
    return o
