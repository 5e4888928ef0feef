"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

For each workload the whole HIP path runs at its real size; the oracle then checks, for a subset
of kv heads (and their q heads): bit-exact means, codes, scales and correction table, the exact
INT32 QK^T and the P~ codes of a 64-row range taken from the attention kernel's own tiles, and the
attention output on sampled rows (first, last and evenly spaced rows), to the same bar as the small
cases, in the workload's output dtype and again in f32 (the bare 1e-2 bound plus the P~ allowance).
Accuracy against FP64 attention must reach the floor recorded for the workload by the oracle's
error budget (tests/golden/accuracy_budget.json, same heads and rows).
"""
import json
import os

import numpy as np
import pytest
import torch

import gpu_harness as H
import parity as P
from quantized_exact_attention_token_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

with open(os.path.join(os.path.dirname(__file__), "golden", "accuracy_budget.json")) as _fh:
    BUDGET = json.load(_fh)


@pytest.mark.parametrize("name", ["mha4k", "prefill8k", "gqa16k", "diffusion32k", "diffusion_varlen"])
def test_full_size(name):
    w = W.WORKLOADS[name]
    print(f"[parity-full] {name}: start", flush=True)
    run = H.DeviceRun(w)
    run.run()
    o32 = run.attn_as(torch.float32)
    ws = run.ws_host()
    heads = (w.Hkv - 1, 1)  # the last kv head and its q heads
    budget = {s["b"]: s for s in BUDGET[name]["sequences"]}
    for b in sorted(budget):
        rows = np.asarray(budget[b]["rows"], np.int32)
        info = P.check_sequence(run, b, heads=heads, rows=rows, ws=ws, nthreads=16,
                                extra_outputs={"f32": o32})
        assert abs(info["cos_fp64_gpu"] - info["cos_fp64_oracle"]) < 1e-3
        assert info["cos_fp64_gpu"] >= BUDGET[name]["floor_cos_fp64"], info["cos_fp64_gpu"]
        print(f"[parity-full] {name} seq {b}: " + ", ".join(
            f"{k}={v:.6g}" if isinstance(v, float) else f"{k}={v}" for k, v in info.items()), flush=True)


def test_full_size_deterministic():
    """The whole path at the benchmark's workload (gqa16k) twice: bit-identical outputs."""
    w = W.WORKLOADS["gqa16k"]
    run = H.DeviceRun(w)
    a = run.run().clone()
    run.o.fill_(0)
    run.ws.fill_(0xA5)
    b = run.run()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


ABLATIONS = {"no_k_smooth": 1, "no_q_smooth": 2, "no_smoothing": 3, "per_block_scales": 4}


@pytest.mark.parametrize("name", ["mha4k", "prefill8k", "gqa16k", "diffusion32k", "diffusion_varlen"])
@pytest.mark.parametrize("ablation", list(ABLATIONS))
def test_full_size_ablation(name, ablation):
    """Each smoothing / scale-granularity ablation at full size through the GPU path: codes, scales
    and correction table bit-exact against the oracle's ablation, output to the usual bar, and the
    accuracy against FP64 equal (to 1e-3) to the oracle's figure recorded for that ablation on the
    same heads and rows (tests/golden/accuracy_budget.json)."""
    w = W.WORKLOADS[name]
    print(f"[ablation-full] {name} {ablation}: start", flush=True)
    run = H.DeviceRun(w, flags=ABLATIONS[ablation])
    run.run()
    ws = run.ws_host()
    budget = {s["b"]: s for s in BUDGET[name]["sequences"]}
    for b in sorted(budget):
        rows = np.asarray(budget[b]["rows"], np.int32)
        info = P.check_sequence(run, b, heads=(w.Hkv - 1, 1), rows=rows, ws=ws, check_s=False,
                                nthreads=16)
        want = budget[b]["settings"][ablation]["cos"]
        print(f"[ablation-full] {name} {ablation} seq {b}: cos_fp64 gpu={info['cos_fp64_gpu']:.4f} "
              f"oracle={want:.4f} maxerr_fp64 gpu={info['maxerr_fp64_gpu']:.4f} "
              f"max_abs_vs_oracle={info['max_abs']:.3g}", flush=True)
        assert abs(info["cos_fp64_gpu"] - want) < 1e-3, (info["cos_fp64_gpu"], want)


def test_full_size_single_level_ablation():
    """The single-level accumulation ablation (no FP32 fold) at the benchmark's workload, held to
    its own model (the oracle's single-level form plus its per-step error band)."""
    w = W.WORKLOADS["gqa16k"]
    run = H.DeviceRun(w, flags=8, out_dtype=torch.float32)
    run.run()
    rows = np.asarray(BUDGET["gqa16k"]["sequences"][0]["rows"], np.int32)
    info = P.check_sequence(run, 0, heads=(w.Hkv - 1, 1), rows=rows, check_s=False, nthreads=16)
    two = H.DeviceRun(w, out_dtype=torch.float32)
    two.run()
    d = (run.o - two.o).abs().max().item()
    print(f"[ablation-full] gqa16k no_fp32_fold: band_max={info['single_level_band_max']:.3g} "
          f"max_abs_vs_model={info['max_abs']:.3g} max|single - two-level| (GPU, all rows)={d:.3g}",
          flush=True)


def test_long_sequence():
    """A sequence four times the benchmark's length: causal GQA, 65536 tokens, 4 q heads on one kv
    head, d = 128, the gqa16k recipe. The Q blocks at the end visit 512 key tiles; the pre-pass
    outputs (the correction table's 4 x 512 rows included), the INT32 S and P~ codes of a 64-row
    range from the attention kernel's own tiles and the output on sampled rows meet the usual bar."""
    w = W.Workload("long64k", 1, 4, 1, 65536, 65536, 128, torch.bfloat16, True, 1200,
                   k_offset_std=4.0, q_offset_std=4.0, n_outliers=4, outlier_scale=20.0)
    print("[parity-full] long64k: start", flush=True)
    run = H.DeviceRun(w)
    run.run()
    o32 = run.attn_as(torch.float32)
    n = w.Nq
    rows = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n),
                                     np.linspace(0, n - 1, 40).astype(np.int64)])).astype(np.int32)
    info = P.check_sequence(run, 0, heads=(0, 1), rows=rows, nthreads=16, extra_outputs={"f32": o32})
    assert abs(info["cos_fp64_gpu"] - info["cos_fp64_oracle"]) < 1e-3
    print("[parity-full] long64k: " + ", ".join(
        f"{k}={v:.6g}" if isinstance(v, float) else f"{k}={v}" for k, v in info.items()), flush=True)
