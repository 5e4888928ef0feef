"""CPU oracle for the SageAttention2 forward pass (ctypes wrapper around sage2_oracle.cpp).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the
benchmark use it; the GPU library and its Python binding never import it.

All arrays are numpy, one sequence at a time, head-major:
  q [Hq, Lq, d], k/v [Hkv, Lkv, d] float32 (exact widenings of fp16/bf16 inputs).
Batches and packed variable-length inputs are handled by the caller, one sequence per call
(the method's statistics are all per sequence and per head).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage2_oracle.cpp")
_LIB = os.path.join(_HERE, "libsage2_oracle.so")

NO_K_SMOOTH = 1
NO_Q_SMOOTH = 2
PER_BLOCK = 4
DELTA_F64 = 16         # correction term as one fp64 dot product (alternative reading, evidence only)
ATTN_NO_P8 = 1         # P~ unquantized
ATTN_V_EXACT = 2       # error budget: unquantized V
ATTN_QK_EXACT = 4      # error budget: logits from the unquantized Q, K
ATTN_NARROW_ACC = 8    # ablation: P~V sums in a float of `acc_bits` mantissa bits
ATTN_SINGLE_LEVEL = 16  # ablation: no FP32 fold

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (plain C++17, no contraction of floating-point operations)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                        "-pthread", "-Wall", _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        F = ctypes.c_float
        L.orc_quantize.argtypes = [I, I, I, I, I, F, I, P, P, P, P, P, P, P, P, P, P, P, P, I]
        L.orc_qk_i32.argtypes = [I, I, I, I, I, P, P, I, I, P, I]
        L.orc_logits.argtypes = [I, I, I, I, I, F, I, P, P, P, P, P, P, I, P, I]
        L.orc_attn_quant.argtypes = [I, I, I, I, I, F, I, I, I, P, P, P, P, P, P, P, P, I, P, P,
                                     P, P, P, P, P, I, P, I, I]
        L.orc_attn_fp64.argtypes = [I, I, I, I, I, F, I, P, P, P, P, I, P, I]
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_kgroup.argtypes = [I]
        for fn in (L.orc_quantize, L.orc_qk_i32, L.orc_logits, L.orc_attn_quant, L.orc_attn_fp64,
                   L.orc_kgroup):
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


def kgroup(j: int) -> int:
    return int(lib().orc_kgroup(int(j)))


class Quantized:
    """Outputs of the smoothing + quantization steps for one sequence."""

    def __init__(self, Hq, Hkv, Lq, Lkv, d, sm_scale):
        self.Hq, self.Hkv, self.Lq, self.Lkv, self.d, self.sm_scale = Hq, Hkv, Lq, Lkv, d, sm_scale
        nqb = (Lq + 127) // 128
        ngk = 2 * ((Lkv + 31) // 32)
        self.kbar = np.zeros((Hkv, d), np.float32)
        self.qbar = np.zeros((Hq, nqb, d), np.float32)
        self.qcode = np.zeros((Hq, Lq, d), np.int8)
        self.sq = np.zeros((Hq, Lq), np.float32)
        self.kcode = np.zeros((Hkv, Lkv, d), np.int8)
        self.sk = np.zeros((Hkv, ngk), np.float32)
        self.v8 = np.zeros((Hkv, Lkv, d), np.uint8)
        self.sv = np.zeros((Hkv, d), np.float32)
        self.delta = None


def quantize(q, k, v, sm_scale: float = 0.0, flags: int = 0, with_delta: bool = True,
             nthreads: int = 0) -> Quantized:
    q, k, v = _f32(q), _f32(k), _f32(v)
    Hq, Lq, d = q.shape
    Hkv, Lkv, _ = k.shape
    z = Quantized(Hq, Hkv, Lq, Lkv, d, sm_scale)
    if with_delta:
        z.delta = np.zeros((Hq, z.qbar.shape[1], Lkv), np.float32)
    rc = lib().orc_quantize(Hq, Hkv, Lq, Lkv, d, sm_scale, flags, _p(q), _p(k), _p(v),
                            _p(z.kbar), _p(z.qbar), _p(z.qcode), _p(z.sq), _p(z.kcode), _p(z.sk),
                            _p(z.v8), _p(z.sv), _p(z.delta), nthreads)
    if rc != 0:
        raise ValueError("orc_quantize rejected its arguments")
    return z


def qk_i32(z: Quantized, row0: int = 0, nrows: int | None = None, nthreads: int = 0):
    nrows = z.Lq - row0 if nrows is None else nrows
    s = np.zeros((z.Hq, nrows, z.Lkv), np.int32)
    rc = lib().orc_qk_i32(z.Hq, z.Hkv, z.Lq, z.Lkv, z.d, _p(z.qcode), _p(z.kcode), row0, nrows,
                          _p(s), nthreads)
    if rc != 0:
        raise ValueError("orc_qk_i32 rejected its arguments")
    return s


def _rows(rows, L):
    if rows is None:
        return None, L
    r = np.ascontiguousarray(rows, dtype=np.int32)
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < L))
    return r, int(r.size)


def logits(z: Quantized, causal: bool, rows=None, nthreads: int = 0):
    r, n = _rows(rows, z.Lq)
    x = np.zeros((z.Hq, n, z.Lkv), np.float32)
    rc = lib().orc_logits(z.Hq, z.Hkv, z.Lq, z.Lkv, z.d, z.sm_scale, int(causal), _p(z.qcode),
                          _p(z.sq), _p(z.kcode), _p(z.sk), _p(z.delta), _p(r), n, _p(x), nthreads)
    if rc != 0:
        raise ValueError("orc_logits rejected its arguments")
    return x


def attn_quant(z: Quantized, causal: bool, rows=None, bn: int = 128, flags: int = 0,
               nthreads: int = 0, exact=None, codes: bool = False, acc_bits: int = 0,
               band_log2: int = 0):
    """Returns (out, allow): [Hq, nrows, d] float64 each. `allow` bounds the effect of FP8
    roundings of P~ that sit within the kernel's arithmetic error of a rounding boundary.

    exact = (q, k, v) float32 head-major unquantized inputs, for ATTN_QK_EXACT / ATTN_V_EXACT.
    codes=True adds (p8, amb) [Hq, nrows, Lkv] uint8: each P~ code and whether it is ambiguous.
    band_log2 > 0 adds the single-level accumulation error band [Hq, nrows, d] (relative error
    2^-band_log2 per 64-key step). Extra outputs follow (out, allow) in that order."""
    r, n = _rows(rows, z.Lq)
    out = np.zeros((z.Hq, n, z.d), np.float64)
    allow = np.zeros((z.Hq, n, z.d), np.float64)
    qe = ke = ve = None
    if exact is not None:
        qe, ke, ve = (_f32(a) for a in exact)
    p8 = amb = band = None
    if codes:
        p8 = np.zeros((z.Hq, n, z.Lkv), np.uint8)
        amb = np.zeros((z.Hq, n, z.Lkv), np.uint8)
    if band_log2:
        band = np.zeros((z.Hq, n, z.d), np.float64)
    rc = lib().orc_attn_quant(z.Hq, z.Hkv, z.Lq, z.Lkv, z.d, z.sm_scale, int(causal), bn, flags,
                              _p(z.qcode), _p(z.sq), _p(z.kcode), _p(z.sk), _p(z.v8), _p(z.sv),
                              _p(z.delta), _p(r), n, _p(out), _p(allow), _p(qe), _p(ke), _p(ve),
                              _p(p8), _p(amb), int(acc_bits), _p(band), int(band_log2), nthreads)
    if rc != 0:
        raise ValueError("orc_attn_quant rejected its arguments")
    res = (out, allow)
    if codes:
        res += (p8, amb)
    if band_log2:
        res += (band,)
    return res


def attn_fp64(q, k, v, causal: bool, sm_scale: float = 0.0, rows=None, nthreads: int = 0):
    q, k, v = _f32(q), _f32(k), _f32(v)
    Hq, Lq, d = q.shape
    Hkv, Lkv, _ = k.shape
    r, n = _rows(rows, Lq)
    out = np.zeros((Hq, n, d), np.float64)
    rc = lib().orc_attn_fp64(Hq, Hkv, Lq, Lkv, d, sm_scale, int(causal), _p(q), _p(k), _p(v),
                             _p(r), n, _p(out), nthreads)
    if rc != 0:
        raise ValueError("orc_attn_fp64 rejected its arguments")
    return out
