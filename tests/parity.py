"""Parity checks of one sequence of a GPU run against the oracle (used by the GPU tests, the smoke
check and the benchmark's sampled verification)."""
from __future__ import annotations

import numpy as np

import oracle as O
import gpu_harness as H

SAGE2_NO_FP32_FOLD = 8       # sage2_flag: single-level P~V accumulation (ablation)
SINGLE_LEVEL_BAND_LOG2 = 10  # per-64-key-step relative error bound of that ablation's model


def _eq(name, gpu, ref):
    assert gpu.shape == ref.shape, f"{name}: shape {gpu.shape} vs {ref.shape}"
    if not np.array_equal(gpu, ref):
        diff = np.argwhere(gpu != ref)
        raise AssertionError(f"{name}: {len(diff)} mismatches, first at {tuple(diff[0])}: "
                             f"gpu {gpu[tuple(diff[0])]} oracle {ref[tuple(diff[0])]}")


def check_sequence(run: H.DeviceRun, b: int, heads=None, rows=None, ws=None, check_s=True,
                   nthreads=0, extra_outputs=None):
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
    # the library's flags: the smoothing / scale ablations map onto the oracle's quantizer flags;
    # the single-level ablation (no FP32 fold) onto its attention model
    qflags = run.flags & (O.NO_K_SMOOTH | O.NO_Q_SMOOTH | O.PER_BLOCK)
    single = bool(run.flags & SAGE2_NO_FP32_FOLD)
    z = O.quantize(q, k, v, sm_scale=run.sm_scale, flags=qflags, nthreads=nthreads)
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
    if check_s and not single:
        # INT32 QK^T and the P~ codes from the attention kernel's own tiles, one contiguous range
        info.update(check_tiles(run, b, z, qs, int(rows[0]), int(min(lq - int(rows[0]), 64)),
                                nthreads=nthreads))
    if single:
        # its own model: the running output accumulates inside the FP8 MFMA across tiles, each
        # 64-key MFMA adding its C input and products with a relative error of at most 2^-10 of
        # their magnitudes (twice the per-instruction error measured on gfx950); the model's band
        # is added to the allowance
        ref, allow, band = O.attn_quant(z, w.causal, rows=rows, flags=O.ATTN_SINGLE_LEVEL,
                                        band_log2=SINGLE_LEVEL_BAND_LOG2, nthreads=nthreads)
        info["single_level_band_max"] = float(band.max())
        allow = allow + band
    else:
        ref, allow = O.attn_quant(z, w.causal, rows=rows, nthreads=nthreads)
    gpu = run.out_seq(b)[qs][:, rows]
    info.update(H.check_output(gpu, ref, allow, run.o.dtype, f"{w.name} seq {b}"))
    # the same workspace through other output dtypes (f32: the bare 1e-2 bound plus the allowance)
    for name, o in (extra_outputs or {}).items():
        g2 = run.out_seq(b, o)[qs][:, rows]
        sub = H.check_output(g2, ref, allow, o.dtype, f"{w.name} seq {b} ({name} output)")
        info.update({f"{k}_{name}": v for k, v in sub.items()})
    exact = O.attn_fp64(q, k, v, w.causal, sm_scale=run.sm_scale, rows=rows, nthreads=nthreads)
    info["cos_fp64_gpu"] = H.cos(gpu, exact)
    info["cos_fp64_oracle"] = H.cos(ref, exact)
    info["maxerr_fp64_gpu"] = float(np.abs(gpu - exact).max())
    return info


def visited_keys(lq, lk, causal, rows):
    """[len(rows), lk] bool: the keys of the 128-key tiles that a row's 32-row wave computes (all
    tiles, or under a causal mask the tiles up to the wave's last visible key)."""
    rows = np.asarray(rows)
    if not causal:
        return np.ones((len(rows), lk), bool)
    w0 = rows // 32 * 32
    kmax = np.minimum(lq, w0 + 32) - 1 + (lk - lq)
    nt = np.where(kmax < 0, 0, kmax // 128 + 1)
    return np.arange(lk)[None, :] < 128 * nt[:, None]


def check_tiles(run, b, z, qs, r0, rn, nthreads=0):
    """Bit-exact INT32 S and P~ codes of rows [r0, r0 + rn) of sequence b (q heads `qs`) against
    the oracle: S on every key the kernel's wave visits, which include every visible key; P~ codes
    on every visible key except those the oracle marks ambiguous (both codes correct there). Returns
    the counts."""
    w = run.w
    lq, lk = z.Lq, z.Lkv
    s_gpu, p8_gpu = run.debug_tiles(r0, rn)
    s_gpu, p8_gpu = s_gpu[b][qs][:, :, :lk], p8_gpu[b][qs][:, :, :lk]
    rows = np.arange(r0, r0 + rn, dtype=np.int32)
    vis_tile = visited_keys(lq, lk, w.causal, rows)
    visible = np.ones((rn, lk), bool)
    if w.causal:
        visible = np.arange(lk)[None, :] <= rows[:, None] + (lk - lq)
    assert np.all(vis_tile[visible]), "a visible key lies in a tile the kernel skips"
    # entries outside the visited tiles must be untouched
    assert np.all(s_gpu[:, ~vis_tile] == -(2 ** 31)), "S written outside the visited tiles"
    assert np.all(p8_gpu[:, ~vis_tile] == 0xFF), "P~ written outside the visited tiles"
    s_ref = O.qk_i32(z, r0, rn, nthreads=nthreads)
    _eq("S int32 (attention kernel tiles)", s_gpu[:, vis_tile], s_ref[:, vis_tile])
    _, _, p8_ref, amb = O.attn_quant(z, w.causal, rows=rows, codes=True, nthreads=nthreads)
    sel = np.broadcast_to(vis_tile, p8_ref.shape)
    ok = sel & (amb == 0)
    _eq("P~ codes (unambiguous)", p8_gpu[ok], p8_ref[ok])
    flips = int(((p8_gpu != p8_ref) & sel & (amb != 0)).sum())
    return {"s_checked": int(sel.sum()), "p8_checked": int(ok.sum()), "p8_ambiguous": int((amb[sel] != 0).sum()),
            "p8_flips": flips}

