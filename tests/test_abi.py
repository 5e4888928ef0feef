"""C ABI checks that need no GPU: the library loads, exports every declared symbol, and rejects
bad arguments on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

import quantized_exact_attention_token_amd as sage2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sage2.LIB_PATH):
        from quantized_exact_attention_token_amd import build
        build.build()
    return sage2.lib()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "sage2.h")).read()
    declared = set(re.findall(r"\b(sage2_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(sage2.EXPORTS), declared ^ set(sage2.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def _params(**kw):
    p = sage2.Params()
    p.B, p.H_q, p.H_kv, p.N_q, p.N_kv, p.d = 2, 8, 2, 300, 500, 128
    p.causal, p.in_dtype, p.out_dtype, p.sm_scale = 1, sage2.BF16, sage2.BF16, 0.0
    for name in ("q_stride", "o_stride"):
        getattr(p, name)[:] = (300 * 8 * 128, 8 * 128, 128)
    for name in ("k_stride", "v_stride"):
        getattr(p, name)[:] = (500 * 2 * 128, 2 * 128, 128)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _ws_status(lib, p):
    n = ctypes.c_size_t()
    return lib.sage2_workspace_size(ctypes.byref(p), ctypes.byref(n)), n.value


def test_workspace_size_closed_form(lib):
    st, n = _ws_status(lib, _params())
    assert st == sage2.OK
    lay = sage2.workspace_layout(_params())
    assert lay.total_bytes == n
    # per sequence: Q rows padded to 384 (3 blocks), K/V rows to 512; causal correction rows of
    # 384 (block 0 sees keys up to 127 + 200), 512, 512 keys
    assert (lay.q_rows, lay.kv_rows, lay.q_blocks, lay.delta_len) == (768, 1024, 6, 2 * (384 + 512 + 512))
    assert n >= 8 * 768 * 64 + 2 * 1024 * 64 + 2 * 1024 * 128 + 8 * 2816 * 4
    full = sage2.workspace_layout(_params(causal=0))
    assert full.delta_len == 2 * 3 * 512
    offs = [lay.seq_table, lay.k_partial, lay.v_partial, lay.kbar, lay.sv, lay.sv_inv, lay.qbar,
            lay.qcode, lay.sq, lay.kcode, lay.sk, lay.v8, lay.delta]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.delta + 8 * lay.delta_len * 4 <= n


@pytest.mark.parametrize("field,value,status", [
    ("d", 100, sage2.ERR_UNSUPPORTED),   # not a multiple of 8
    ("d", 136, sage2.ERR_UNSUPPORTED),
    ("d", 256, sage2.ERR_UNSUPPORTED),
    ("d", 0, sage2.ERR_UNSUPPORTED),
    ("flags", 16, sage2.ERR_UNSUPPORTED),
    ("flags", -1, sage2.ERR_UNSUPPORTED),
    ("in_dtype", sage2.F32, sage2.ERR_UNSUPPORTED),
    ("out_dtype", 7, sage2.ERR_UNSUPPORTED),
    ("causal", 2, sage2.ERR_UNSUPPORTED),
    ("sm_scale", float("nan"), sage2.ERR_UNSUPPORTED),
    ("sm_scale", float("inf"), sage2.ERR_UNSUPPORTED),
    ("B", 0, sage2.ERR_SHAPE),
    ("H_q", -1, sage2.ERR_SHAPE),
    ("H_kv", 3, sage2.ERR_SHAPE),       # 8 % 3 != 0
    ("N_q", 0, sage2.ERR_SHAPE),
    ("N_kv", 0, sage2.ERR_SHAPE),
])
def test_rejects_bad_sizes(lib, field, value, status):
    assert _ws_status(lib, _params(**{field: value}))[0] == status


@pytest.mark.parametrize("d,padded", [(8, 64), (48, 64), (64, 64), (72, 128), (96, 128), (128, 128)])
def test_head_dim_padding_layout(lib, d, padded):
    """Any multiple of 8 up to 128 is accepted; the workspace is that of the padded head dim."""
    def mk(dd):
        p = _params(d=dd)
        for name in ("q_stride", "o_stride"):
            getattr(p, name)[:] = (300 * 8 * dd, 8 * dd, dd)
        for name in ("k_stride", "v_stride"):
            getattr(p, name)[:] = (500 * 2 * dd, 2 * dd, dd)
        return p
    st, n = _ws_status(lib, mk(d))
    assert st == sage2.OK
    assert n == _ws_status(lib, mk(padded))[1]


def test_ablation_flags_accepted(lib):
    for f in (0, sage2.NO_K_SMOOTH, sage2.NO_Q_SMOOTH, sage2.PER_BLOCK_SCALES, sage2.NO_FP32_FOLD, 15):
        assert _ws_status(lib, _params(flags=f))[0] == sage2.OK


def test_rejects_misaligned_strides(lib):
    p = _params()
    p.q_stride[1] = 8 * 128 + 4   # 8 bytes: not a multiple of 16
    assert _ws_status(lib, p)[0] == sage2.ERR_ALIGN
    p = _params()
    p.o_stride[2] = 130
    assert _ws_status(lib, p)[0] == sage2.ERR_ALIGN


def test_null_pointers(lib):
    n = ctypes.c_size_t()
    assert lib.sage2_workspace_size(None, ctypes.byref(n)) == sage2.ERR_NULL
    p = _params()
    assert lib.sage2_workspace_size(ctypes.byref(p), None) == sage2.ERR_NULL
    assert lib.sage2_quantize_smooth(ctypes.byref(p), None, 256, 256, 256, 1 << 30, None) == sage2.ERR_NULL
    assert lib.sage2_attn_fwd(ctypes.byref(p), 256, 1 << 30, None, None) == sage2.ERR_NULL
    assert lib.sage2_attn_fwd(ctypes.byref(p), None, 1 << 30, 256, None) == sage2.ERR_NULL
    assert lib.sage2_debug_attn_tiles(ctypes.byref(p), 256, 1 << 30, 0, 1, None, None, None, None) == sage2.ERR_NULL


def test_alignment_and_workspace_checks(lib):
    p = _params()
    _, need = _ws_status(lib, p)
    # misaligned data pointers and workspace (never dereferenced: checks run first)
    assert lib.sage2_quantize_smooth(ctypes.byref(p), 0x1008, 0x2000, 0x3000, 0x10000, need, None) == sage2.ERR_ALIGN
    assert lib.sage2_quantize_smooth(ctypes.byref(p), 0x1000, 0x2000, 0x3000, 0x10080, need, None) == sage2.ERR_ALIGN
    assert lib.sage2_quantize_smooth(ctypes.byref(p), 0x1000, 0x2000, 0x3000, 0x10000, need - 1, None) == sage2.ERR_WORKSPACE
    assert lib.sage2_attn_fwd(ctypes.byref(p), 0x10000, need - 256, 0x1000, None) == sage2.ERR_WORKSPACE
    assert lib.sage2_attn_fwd(ctypes.byref(p), 0x10000, need, 0x1004, None) == sage2.ERR_ALIGN
    dbg = lib.sage2_debug_attn_tiles
    assert dbg(ctypes.byref(p), 0x10000, need, 250, 100, 0x1000, None, None, None) == sage2.ERR_SHAPE
    assert dbg(ctypes.byref(p), 0x10000, need, -1, 10, None, 0x1000, None, None) == sage2.ERR_SHAPE
    assert dbg(ctypes.byref(p), 0x10000, need, 0, 10, 0x1000, None, 0x1008, None) == sage2.ERR_ALIGN
    pf = _params(flags=sage2.NO_FP32_FOLD)
    assert dbg(ctypes.byref(pf), 0x10000, need, 0, 10, 0x1000, None, None, None) == sage2.ERR_UNSUPPORTED


def _varlen(lib, cu_q, cu_kv, Nq=None, Nkv=None, drop=None):
    p = _params()
    aq = (ctypes.c_int32 * len(cu_q))(*cu_q)
    ak = (ctypes.c_int32 * len(cu_kv))(*cu_kv)
    p.B = len(cu_q) - 1
    p.N_q = Nq if Nq is not None else max(1, max(b - a for a, b in zip(cu_q, cu_q[1:])))
    p.N_kv = Nkv if Nkv is not None else max(1, max(b - a for a, b in zip(cu_kv, cu_kv[1:])))
    p.cu_seqlens_q, p.cu_seqlens_kv = 0x100, 0x200   # device copies: never read by the host
    p.cu_seqlens_q_host = ctypes.cast(aq, ctypes.c_void_p).value
    p.cu_seqlens_kv_host = ctypes.cast(ak, ctypes.c_void_p).value
    if drop:
        setattr(p, drop, None)
    st, n = _ws_status(lib, p)
    return st, p, (aq, ak)


def test_varlen_validation(lib):
    assert _varlen(lib, [0, 100, 300], [0, 100, 300])[0] == sage2.OK
    assert _varlen(lib, [0, 100, 100, 300], [0, 50, 50, 120])[0] == sage2.OK   # empty sequence
    assert _varlen(lib, [1, 100, 300], [0, 100, 300])[0] == sage2.ERR_SHAPE    # does not start at 0
    assert _varlen(lib, [0, 300, 100], [0, 100, 300])[0] == sage2.ERR_SHAPE    # decreasing
    assert _varlen(lib, [0, 100, 300], [0, 100, 300], Nq=150)[0] == sage2.ERR_SHAPE  # longer than N_q
    for f in ("cu_seqlens_q", "cu_seqlens_kv", "cu_seqlens_q_host", "cu_seqlens_kv_host"):
        assert _varlen(lib, [0, 100, 300], [0, 100, 300], drop=f)[0] == sage2.ERR_NULL, f


def test_varlen_layout_pads_each_sequence(lib):
    st, p, keep = _varlen(lib, [0, 100, 100, 300], [0, 50, 50, 420])
    assert st == sage2.OK
    lay = sage2.workspace_layout(p)
    assert lay.q_rows == 128 + 0 + 256
    assert lay.kv_rows == 128 + 0 + 384      # kv lengths 50, 0, 370
    assert lay.q_blocks == 1 + 0 + 2
    assert lay.delta_len == 1 * 128 + 2 * 384


def test_status_strings(lib):
    for s in range(7):
        assert len(sage2.status_string(s)) > 0
    assert sage2.status_string(99) == "unknown status"


def test_rejects_layouts_past_int32(lib):
    """Per-head workspace extents are carried as int32 on the device: a dense shape whose correction
    table would pass 2^31 - 1 entries per head is refused before any sizing overflow."""
    p = _params(N_q=200_000, N_kv=200_000, B=8, causal=0)   # 8 * 1563 Q blocks * 200064 keys > 2^31
    for name in ("q_stride", "o_stride"):
        getattr(p, name)[:] = (200_000 * 8 * 128, 8 * 128, 128)
    for name in ("k_stride", "v_stride"):
        getattr(p, name)[:] = (200_000 * 2 * 128, 2 * 128, 128)
    assert _ws_status(lib, p)[0] == sage2.ERR_SHAPE
    p.B = 1   # 1563 * 200064 = 3.1e8 entries per head: fine
    assert _ws_status(lib, p)[0] == sage2.OK
    p.B, p.causal = 8, 1   # causal: about half the table, 1.25e9 entries: fine
    assert _ws_status(lib, p)[0] == sage2.OK
    p.B = 16               # 2.5e9: refused
    assert _ws_status(lib, p)[0] == sage2.ERR_SHAPE


def test_causal_correction_rows_match_a_plain_loop(lib):
    """The compact causal correction-table length (a closed form in the library) equals the plain
    per-block sum of the keys each Q block can see, rounded up to 128, on random dense and packed
    shapes, including N_q != N_kv and empty sequences."""
    import numpy as np
    import gpu_harness as H
    rng = np.random.default_rng(5)
    for _ in range(300):
        causal = int(rng.integers(2))
        nseq = int(rng.integers(1, 5))
        lq = [int(x) for x in rng.integers(0, 1200, nseq)]
        lk = [int(x) for x in rng.integers(0, 1200, nseq)]
        if rng.integers(2):  # dense
            lq, lk = [max(1, lq[0])] * nseq, [max(1, lk[0])] * nseq
            p = _params(B=nseq, N_q=lq[0], N_kv=lk[0], causal=causal)
            keep = None
        else:
            cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
            ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
            keep = (cq, ck)
            p = _params(B=nseq, N_q=max(1, max(lq)), N_kv=max(1, max(lk)), causal=causal)
            p.cu_seqlens_q = p.cu_seqlens_kv = 0x1000  # device pointers: never dereferenced here
            p.cu_seqlens_q_host = cq.ctypes.data
            p.cu_seqlens_kv_host = ck.ctypes.data
        lay = sage2.workspace_layout(p)
        want = sum(sum(H.delta_row_keys(bool(causal), a, b)) for a, b in zip(lq, lk))
        assert lay.delta_len == want, (causal, lq, lk, lay.delta_len, want)



def test_binding_rejects_what_the_library_cannot_check():
    """The C ABI takes raw device pointers; the binding refuses host tensors, mixed dtypes and
    mismatched shapes before any pointer reaches the library (no GPU needed to check this)."""
    import torch
    q = torch.zeros(1, 16, 4, 64, dtype=torch.float16)
    k = torch.zeros(1, 16, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="dtype"):
        sage2.make_params(q, k.to(torch.bfloat16), k, causal=True)
    with pytest.raises(ValueError, match="shapes"):
        sage2.make_params(q, k, k[:, :8], causal=True)
    with pytest.raises(ValueError, match="o must have"):
        sage2.make_params(q, k, k, o=q[:, :8], causal=True)
    with pytest.raises(ValueError, match="device"):
        sage2.make_params(q, k, k, causal=True)       # host tensors
    with pytest.raises(ValueError, match="device"):
        sage2.make_params(q[0], k[0], k[0], causal=False,
                          cu_seqlens_q=torch.tensor([0, 16], dtype=torch.int32),
                          cu_seqlens_kv=torch.tensor([0, 16], dtype=torch.int32))
