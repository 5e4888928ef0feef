"""The two hot-path calls captured in a HIP graph (the header states that the calls enqueue kernels
only: no host callback, no allocation, no synchronization, so they may be captured).

sage2_quantize_smooth + sage2_attn_fwd are captured once into one graph on torch's capture stream and
the graph is replayed several times. Before each replay the input buffers get new contents (eager
copies, with synchronizations between the replays); every replay's output must equal, bit for bit,
an eager run of the same two calls on those inputs with a workspace and output of its own. The
kernels' results do not depend on a workspace's earlier contents, and the workspace path is checked
against the oracle elsewhere, so equality with the eager run is the whole check.
"""
import pytest
import torch

import gpu_harness as H
import quantized_exact_attention_token_amd as sage2
from quantized_exact_attention_token_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = {
    "causal_gqa_d128": W.custom(1, 8, 2, 1000, 1000, 128, torch.bfloat16, True, seed=81,
                                n_outliers=2, outlier_scale=20.0, k_offset_std=4.0),
    "varlen_d64": W.custom(3, 4, 2, 300, 300, 64, torch.float16, False, seed=82,
                           seqlens=[300, 17, 129]),
}


def _eager(run, q, k, v):
    ws = torch.empty_like(run.ws)
    ws.fill_(0x5A)
    o = torch.full_like(run.o, float("nan"))
    sage2.quantize_smooth(run.p, q, k, v, ws)
    sage2.attn_fwd(run.p, ws, o)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager_runs(name):
    w = CASES[name]
    print(f"[graph] {name}: start", flush=True)
    run = H.DeviceRun(w)
    # warm-up on a side stream before capture (library and torch state settled)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.prepass()
        run.attn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.prepass()
        run.attn()
    torch.cuda.synchronize()

    for rep in range(4):
        if rep:
            gen = torch.Generator().manual_seed(1000 + rep)
            for t, scale in ((run.q, 1.0 + rep), (run.k, 2.0), (run.v, 0.5 * rep)):
                t.copy_((torch.randn(t.shape, generator=gen) * scale).to(t.dtype))
        run.o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = run.o.clone()
        ref = _eager(run, run.q, run.k, run.v)
        assert not torch.isnan(ref).any()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (name, rep)
        print(f"[graph] {name} replay {rep}: equal to the eager run", flush=True)
