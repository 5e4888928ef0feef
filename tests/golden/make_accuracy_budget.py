"""Writes tests/golden/accuracy_budget.json: the method's accuracy against FP64 attention on each
workload's recipe, split by quantizer, from the CPU oracle alone.

For every workload the sample is the one the full-size GPU parity tests check: the last kv head
with its q heads, of the last batch element (dense) or of every sequence (packed), on the query
rows `sample_rows(L)` (the first 8, the last 8 and 40 evenly spaced). On those rows it records the
cosine similarity and the max-abs error against FP64 attention (oracle part (ii)) of:
  full           the whole method (oracle part (i));
  int4_qk_only   INT4 Q/K with smoothing, P~ and V unquantized;
  fp8_v_only     exact logits, V in FP8, P~ unquantized;
  fp8_p_only     exact logits and V, P~ in FP8;
  and the ablations the pages argue from (no K smoothing, no Q smoothing, neither, per-block
  scales; a narrow 13- or 10-bit P~V accumulator with and without the FP32 fold).
Each setting also records its max-abs difference from the full method ("maxerr_vs_full"), which
isolates what that one change costs.
`floor_cos_fp64` = the full method's lowest cosine over the sample minus 1e-3: the GPU path, whose
output matches the oracle's to 1e-2, must reach it.

Run from the repository root: python tests/golden/make_accuracy_budget.py [workload ...]
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from quantized_exact_attention_token_amd import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "accuracy_budget.json")
NARROW_BITS = (13, 10)


def sample_rows(L: int, n: int = 40) -> np.ndarray:
    r = np.unique(np.concatenate([np.arange(min(8, L)), np.arange(max(0, L - 8), L),
                                  np.linspace(0, L - 1, n).astype(np.int64)]))
    return r.astype(np.int32)


def _cos(a, b):
    a, b = np.ravel(a).astype(np.float64), np.ravel(b).astype(np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def sequences(w: W.Workload):
    """(b, q, k, v) of the sample: head-major float32 arrays of the last kv-head group."""
    q, k, v, cu = W.generate(w)
    grp = w.Hq // w.Hkv
    g0 = w.Hkv - 1
    f = lambda t: t.float().permute(1, 0, 2).contiguous().numpy()
    if cu is None:
        b = w.B - 1
        yield b, f(q[b][:, g0 * grp:]), f(k[b][:, g0:]), f(v[b][:, g0:])
        return
    cq = cu.numpy()
    ck = W.cu_seqlens(w.kv_lens).numpy()
    for b in range(len(cq) - 1):
        sl, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        if cq[b + 1] == cq[b] or ck[b + 1] == ck[b]:
            continue
        yield b, f(q[sl][:, g0 * grp:]), f(k[sk][:, g0:]), f(v[sk][:, g0:])


def budget(w: W.Workload, threads: int = 0):
    seqs = []
    for b, q, k, v in sequences(w):
        rows = sample_rows(q.shape[1])
        exact = O.attn_fp64(q, k, v, w.causal, rows=rows, nthreads=threads)
        z = O.quantize(q, k, v, nthreads=threads)
        res = {}
        full = O.attn_quant(z, w.causal, rows=rows, nthreads=threads)[0]

        def rec(name, out):
            res[name] = {"cos": _cos(out, exact), "maxerr": float(np.abs(out - exact).max()),
                         "maxerr_vs_full": float(np.abs(out - full).max())}

        ex = (q, k, v)
        rec("full", full)
        rec("int4_qk_only", O.attn_quant(z, w.causal, rows=rows, nthreads=threads, exact=ex,
                                         flags=O.ATTN_NO_P8 | O.ATTN_V_EXACT)[0])
        rec("fp8_v_only", O.attn_quant(z, w.causal, rows=rows, nthreads=threads, exact=ex,
                                       flags=O.ATTN_QK_EXACT | O.ATTN_NO_P8)[0])
        rec("fp8_p_only", O.attn_quant(z, w.causal, rows=rows, nthreads=threads, exact=ex,
                                       flags=O.ATTN_QK_EXACT | O.ATTN_V_EXACT)[0])
        for bits in NARROW_BITS:
            rec(f"narrow{bits}_two_level", O.attn_quant(z, w.causal, rows=rows, nthreads=threads,
                                                        flags=O.ATTN_NARROW_ACC, acc_bits=bits)[0])
            rec(f"narrow{bits}_single_level", O.attn_quant(
                z, w.causal, rows=rows, nthreads=threads,
                flags=O.ATTN_NARROW_ACC | O.ATTN_SINGLE_LEVEL, acc_bits=bits)[0])
        for name, fl in (("no_k_smooth", O.NO_K_SMOOTH), ("no_q_smooth", O.NO_Q_SMOOTH),
                         ("no_smoothing", O.NO_K_SMOOTH | O.NO_Q_SMOOTH),
                         ("per_block_scales", O.PER_BLOCK)):
            za = O.quantize(q, k, v, flags=fl, nthreads=threads)
            rec(name, O.attn_quant(za, w.causal, rows=rows, nthreads=threads)[0])
        seqs.append({"b": int(b), "L_q": int(q.shape[1]), "L_kv": int(k.shape[1]),
                     "q_heads": [int(w.Hq - q.shape[0]), int(w.Hq)], "rows": rows.tolist(),
                     "settings": res})
    floor = min(s["settings"]["full"]["cos"] for s in seqs) - 1e-3
    return {"recipe": f"B{w.B} Hq{w.Hq} Hkv{w.Hkv} N{w.Nq} d{w.d} {str(w.dtype).split('.')[-1]} "
                      f"causal={w.causal}", "sequences": seqs, "floor_cos_fp64": floor}


def main(names):
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as fh:
            data = json.load(fh)
    for name in names:
        t0 = time.time()
        data[name] = budget(W.WORKLOADS[name])
        full = [s["settings"]["full"]["cos"] for s in data[name]["sequences"]]
        print(f"{name}: full-method cos vs FP64 {min(full):.4f} ({time.time() - t0:.0f} s)",
              flush=True)
    data["_about"] = ("cos / max-abs error against FP64 attention on the sampled rows; written by "
                      "tests/golden/make_accuracy_budget.py from the CPU oracle only")
    with open(OUT, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny", "mha4k", "prefill8k", "gqa16k", "diffusion32k", "diffusion_varlen"])
