"""Parity checks of one sequence of a GPU run against the oracle (used by the GPU tests, the smoke
check and the benchmark's sampled verification)."""
from __future__ import annotations

import numpy as np

import oracle as O
import gpu_harness as H


def _eq(name, gpu, ref):
    assert gpu.shape == ref.shape, f"{name}: shape {gpu.shape} vs {ref.shape}"
    if not np.array_equal(gpu, ref):
        diff = np.argwhere(gpu != ref)
        raise AssertionError(f"{name}: {len(diff)} mismatches, first at {tuple(diff[0])}: "
                             f"gpu {gpu[tuple(diff[0])]} oracle {ref[tuple(diff[0])]}")


def check_sequence(run: H.GpuRun, b: int, heads=None, rows=None, ws=None, check_s=True,
                   nthreads=0):
    """Bit-exact pre-pass outputs and INT32 QK^T, tolerance-checked attention output, for sequence
    b and the kv-head range `heads` = (first, count) (all heads when None), on query rows `rows`
    (all when None). Returns measured figures."""
    w = run.w
    grp = w.Hq // w.Hkv
    g0, ng = heads if heads is not None else (0, w.Hkv)
    h0, nh = g0 * grp, ng * grp
    q, k, v = run.seq_inputs(b, (g0, ng))
    lq, lk = q.shape[1], k.shape[1]
    if ws is None:
        ws = run.ws_host()
    dec = run.decode(ws, b)
    info = {"lq": lq, "lkv": lk}
    if lq == 0:
        return info
    if lk == 0:
        # no keys: every row is fully masked and outputs zeros
        assert np.all(run.out_seq(b)[h0:h0 + nh] == 0)
        return info
    z = O.quantize(q, k, v, sm_scale=run.sm_scale, flags=run.flags, nthreads=nthreads)
    qs, kvs = slice(h0, h0 + nh), slice(g0, g0 + ng)
    _eq("kbar", dec["kbar"][kvs], z.kbar)
    _eq("sv", dec["sv"][kvs], z.sv)
    _eq("qbar", dec["qbar"][qs], z.qbar)
    _eq("qcode", dec["qcode"][qs], z.qcode)
    assert not dec["qcode_pad"].any(), "padding rows of the Q codes are not zero"
    _eq("sq", dec["sq"][qs], z.sq)
    _eq("kcode", dec["kcode"][kvs], z.kcode)
    _eq("sk", dec["sk"][kvs], z.sk)
    _eq("v8", dec["v8"][kvs], z.v8)
    gd = dec["delta"][qs]
    if w.causal:
        nqb = gd.shape[1]
        vis = np.zeros(gd.shape[1:], bool)
        for qb in range(nqb):
            jmax = min(lq, 128 * (qb + 1)) - 1 + (lk - lq)
            vis[qb, :max(0, jmax + 1)] = True
        _eq("delta(visible)", gd[:, vis], z.delta[:, vis])  # hidden entries are unspecified
    else:
        _eq("delta", gd, z.delta)

    if rows is None:
        rows = np.arange(lq, dtype=np.int32)
    rows = np.asarray(rows, dtype=np.int32)
    if check_s:
        # INT32 QK^T from the kernel's MFMA path for one contiguous row range
        r0 = int(rows[0])
        rn = int(min(lq - r0, 64))
        s_gpu = run.debug_qk(r0, rn)[b][qs][:, :, :lk]
        s_ref = O.qk_i32(z, r0, rn, nthreads=nthreads)
        _eq("S int32", s_gpu, s_ref)
    ref, allow = O.attn_quant(z, w.causal, rows=rows, nthreads=nthreads)
    gpu = run.out_seq(b)[qs][:, rows]
    info.update(H.check_output(gpu, ref, allow, run.o.dtype, f"{w.name} seq {b}"))
    exact = O.attn_fp64(q, k, v, w.causal, sm_scale=run.sm_scale, rows=rows, nthreads=nthreads)
    info["cos_fp64_gpu"] = H.cos(gpu, exact)
    info["cos_fp64_oracle"] = H.cos(ref, exact)
    return info
