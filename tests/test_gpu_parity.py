"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on seeded inputs.

Bar: bit-exact K/Q means, INT4 codes and scales, FP8 V codes and scales, correction table and
INT32 QK^T; output within 1e-2 max-abs (plus the allowance for P~ roundings that sit within the
kernel's arithmetic error of an FP8 boundary, plus half an ulp of the output format) and cosine
>= 0.9999 against the oracle's quantized pipeline. Accuracy against FP64 attention is recorded
and must match the oracle's own to within 1e-3 (the GPU path is as accurate as the method).
"""
import os

import numpy as np
import pytest
import torch

import gpu_harness as H
import parity as P
from quantized_exact_attention_token_amd import workloads as W

pytestmark = pytest.mark.gpu


def _report(name, info):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.6g}" if isinstance(v, float) else f"{k}={v}"
                                         for k, v in info.items()), flush=True)


def _full_check(w, out_dtype=None, layout="bnhd", flags=0, sm_scale=0.0, modify=None):
    run = H.DeviceRun(w, out_dtype=out_dtype, layout=layout, flags=flags, sm_scale=sm_scale,
                   modify=modify)
    run.run()
    ws = run.ws_host()
    for b, _ in enumerate(run.sequences()):
        info = P.check_sequence(run, b, ws=ws)
        if "cos_fp64_gpu" in info:
            assert abs(info["cos_fp64_gpu"] - info["cos_fp64_oracle"]) < 1e-3
        _report(f"{w.name} b{b}", info)
    return run


@pytest.mark.parametrize("out", ["f16", "bf16", "f32"])
def test_tiny_all_outputs(out):
    _full_check(W.WORKLOADS["tiny"], out_dtype=H.OUT_DTYPES[out])


def test_tiny_deterministic():
    run = H.DeviceRun(W.WORKLOADS["tiny"])
    a = run.run().clone()
    run.o.fill_(0)
    b = run.run()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


EDGE = [
    # (B, Hq, Hkv, Nq, Nkv, d, dtype, causal)
    (1, 2, 2, 1, 1, 64, torch.float16, False),
    (1, 2, 1, 31, 31, 128, torch.bfloat16, True),
    (2, 4, 2, 63, 63, 64, torch.float16, True),
    (1, 2, 2, 65, 65, 128, torch.bfloat16, False),
    (1, 8, 1, 127, 127, 64, torch.bfloat16, True),
    (1, 4, 4, 129, 129, 128, torch.float16, True),
    (1, 8, 2, 1000, 1000, 128, torch.bfloat16, True),
    (2, 4, 2, 200, 333, 64, torch.float16, True),    # Nq < Nkv, bottom-right causal
    (1, 4, 2, 333, 200, 128, torch.bfloat16, True),  # Nq > Nkv: leading rows see no key
    (1, 2, 2, 300, 77, 64, torch.float16, False),
    (1, 6, 2, 300, 300, 128, torch.bfloat16, True),  # 3 q heads per kv head (not a power of two)
    (1, 6, 1, 257, 257, 64, torch.float16, True),    # 6 q heads per kv head
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B%d_Hq%d_Hkv%d_Nq%d_Nkv%d_d%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], str(c[6]).split(".")[-1], "causal" if c[7] else "full"))
def test_edge_shapes(case):
    B, Hq, Hkv, Nq, Nkv, d, dt, causal = case
    _full_check(W.custom(B, Hq, Hkv, Nq, Nkv, d, dt, causal, seed=Nq * 7 + Nkv))


@pytest.mark.parametrize("case", [(0.05, 128, torch.bfloat16, True), (0.3, 64, torch.float16, False),
                                  (0.125, 96, torch.bfloat16, True)],
                         ids=["tau0.05_d128_causal", "tau0.3_d64_full", "tau0.125_d96_causal"])
def test_custom_softmax_scale(case):
    """A caller-given softmax scale (not 1/sqrt(d)) reaches the correction table and the logits."""
    tau, d, dt, causal = case
    _full_check(W.custom(1, 4, 2, 300, 300, d, dt, causal, seed=int(tau * 1000) + d), sm_scale=tau)


def test_bhnd_strides():
    _full_check(W.custom(2, 4, 2, 150, 150, 128, torch.bfloat16, True, seed=5), layout="bhnd")


def test_varlen_with_empty_sequences():
    w = W.custom(5, 4, 2, 300, 300, 64, torch.float16, False, seed=8,
                 seqlens=[130, 0, 300, 1, 64])
    _full_check(w)


@pytest.mark.parametrize("case", [
    # (d, dtype, causal, query lengths, key/value lengths)
    (64, torch.float16, True, [100, 0, 257, 33], [300, 64, 128, 0]),
    (128, torch.bfloat16, False, [200, 129, 5], [77, 300, 130]),
], ids=["d64_causal", "d128_full"])
def test_varlen_different_kv_lengths(case):
    """Packed batches whose query and key/value lengths differ per sequence: fewer queries than keys
    (bottom-right causal alignment), more queries than keys (leading rows see no key), empty query
    or key sets."""
    d, dt, causal, lq, lk = case
    w = W.custom(len(lq), 4, 2, max(lq), max(lk), d, dt, causal, seed=sum(lq) + 3 * sum(lk),
                 seqlens=lq, kv_seqlens=lk)
    _full_check(w)


def test_varlen_equals_separate_calls():
    """E1: a packed variable-length batch gives bit-identical outputs to one call per sequence."""
    lens = [100, 257, 64]
    w = W.custom(3, 4, 4, 257, 257, 64, torch.float16, True, seed=9, seqlens=lens)
    run = H.DeviceRun(w)
    packed = run.run().clone()
    cu = run.cu_cpu
    for i, L in enumerate(lens):
        s, e = int(cu[i]), int(cu[i + 1])
        q, k, v = (t[s:e][None].cuda() for t in (run.q_cpu, run.k_cpu, run.v_cpu))
        import quantized_exact_attention_token_amd as sage2
        o = sage2.attention(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[0].view(torch.int16), packed[s:e].view(torch.int16)), i


@pytest.mark.parametrize("case", [(64, torch.float16, False), (128, torch.bfloat16, True)],
                         ids=["d64_full", "d128_causal"])
def test_rising_row_max_renormalizes(case):
    """Logits that climb by hundreds (base 2) along the keys: the running max keeps rising, so the
    kernel's FP32 output buffer is renormalized several times on the way (its fold factor would
    otherwise pass 2^64). The result must still match the oracle."""
    import oracle as O
    d, dt, causal = case
    w = W.custom(1, 2, 1, 512, 512, d, dt, causal, seed=11 + d, key_ramp=8.0, q_shift=4.0)
    run = _full_check(w)
    q, k, v = run.seq_inputs(0)
    z = O.quantize(q, k, v)
    x = O.logits(z, causal, rows=np.array([511], np.int32))[:, 0]
    span = float((x.max(axis=-1) - x.min(axis=-1)).min())
    assert span > 3 * 64, f"logit span {span} too small to reach the renormalization"


HEAD_DIMS = [
    # (d, dtype, causal, Hq, Hkv): padded to 64 or 128 inside the workspace
    (8, torch.float16, False, 2, 2),
    (48, torch.float16, False, 4, 2),
    (80, torch.bfloat16, False, 4, 1),
    (96, torch.bfloat16, True, 4, 2),
    (120, torch.float16, True, 2, 2),
]


@pytest.mark.parametrize("case", HEAD_DIMS, ids=lambda c: "d%d_%s_%s" % (
    c[0], str(c[1]).split(".")[-1], "causal" if c[2] else "full"))
def test_head_dim_padding(case):
    """Head dims below 64/128: zero channels inside the workspace (checked by the decoder), the same
    codes, scales, correction and output as the oracle run on the true head dim, and the default
    softmax scale taken from the true d."""
    d, dt, causal, hq, hkv = case
    _full_check(W.custom(1, hq, hkv, 200, 200, d, dt, causal, seed=300 + d))


@pytest.mark.parametrize("flags", [1, 2, 3, 4, 7, 8], ids=["no_k_smooth", "no_q_smooth", "no_smoothing",
                                                          "per_block_scales", "naive_per_block",
                                                          "no_fp32_fold"])
def test_smoothing_ablations(flags):
    """The ablation flags reproduce the oracle's ablations bit for bit (codes, scales, correction)
    and to the usual bar on the output; accuracy against FP64 is reported by the parity check.
    NO_FP32_FOLD (8) is held to its own model, the oracle's single-level form, whose allowance
    adds the error band of an accumulator that adds each 64-key step with a relative error of up
    to 2^-10; the difference from the two-level GPU output is reported."""
    w = W.custom(1, 4, 2, 300, 300, 128, torch.bfloat16, True, seed=77, k_offset_std=4.0,
                 q_offset_std=4.0)
    run = _full_check(w, flags=flags, out_dtype=torch.float32)
    if flags & 8:
        two = _full_check(w, flags=flags & ~8, out_dtype=torch.float32)
        d = (run.o - two.o).abs().max().item()
        print(f"[parity] no_fp32_fold vs two-level (GPU, f32 output): max |diff| = {d:.3e}", flush=True)



def _random_case(seed):
    """A seeded mixed configuration: batch or packed variable-length sequences (empty ones
    included), GQA groups of 1, 2 or 4, any head dim that is a multiple of 8, either input dtype,
    causal or not, different Q and KV lengths when dense."""
    rng = np.random.default_rng(1000 + seed)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = 8 * int(rng.integers(1, 17))
    dt = torch.float16 if rng.integers(2) else torch.bfloat16
    causal = bool(rng.integers(2))
    if rng.integers(2):
        lens = [int(x) for x in rng.integers(1, 420, size=int(rng.integers(2, 5)))]
        if len(lens) > 2 and rng.integers(2):
            lens[int(rng.integers(len(lens)))] = 0
        n = max(lens)
        return W.custom(len(lens), hq, hkv, n, n, d, dt, causal, seed=seed, seqlens=lens)
    b = int(rng.integers(1, 3))
    nq, nkv = int(rng.integers(1, 420)), int(rng.integers(1, 420))
    return W.custom(b, hq, hkv, nq, nkv, d, dt, causal, seed=seed)


@pytest.mark.parametrize("seed", range(8))
def test_random_configurations(seed):
    """Eight seeded mixed configurations through the whole path (the pre-pass's two fused launches
    split their grids by role, so shapes that leave some roles empty are included)."""
    w = _random_case(seed)
    print(f"[parity] random {seed}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} Nq{w.Nq} Nkv{w.Nkv} d{w.d} "
          f"{str(w.dtype).split('.')[-1]} causal={w.causal} seqlens={w.seqlens}", flush=True)
    _full_check(w)


# Wider mixed configurations: GQA groups of 1 to 8 q heads per kv head (3 and 6 included), up to
# 1500 tokens (many key tiles, ragged tails), outlier and offset strengths varied. A handful run by
# default; SAGE2_WIDE_CASES=N runs N of them.
_WIDE_CASES = int(os.environ.get("SAGE2_WIDE_CASES", "16"))


def _wide_case(seed):
    rng = np.random.default_rng(50000 + seed)
    hkv = int(rng.choice([1, 2, 3]))
    hq = hkv * int(rng.choice([1, 2, 3, 4, 6, 8]))
    d = 8 * int(rng.integers(1, 17))
    dt = torch.float16 if rng.integers(2) else torch.bfloat16
    causal = bool(rng.integers(2))
    kw = dict(n_outliers=int(rng.integers(0, 3)), outlier_scale=float(rng.choice([5.0, 20.0])),
              k_offset_std=float(rng.choice([0.0, 4.0])))
    if rng.integers(2):
        lens = [int(x) for x in rng.integers(0, 1500, size=int(rng.integers(1, 4)))]
        if max(lens) == 0:
            lens[0] = 1
        n = max(lens)
        return W.custom(len(lens), hq, hkv, n, n, d, dt, causal, seed=seed, seqlens=lens, **kw)
    b = int(rng.integers(1, 3))
    nq, nkv = int(rng.integers(1, 1500)), int(rng.integers(1, 1500))
    return W.custom(b, hq, hkv, nq, nkv, d, dt, causal, seed=seed, **kw)


@pytest.mark.parametrize("seed", range(_WIDE_CASES))
def test_wide_random_configurations(seed):
    w = _wide_case(seed)
    print(f"[parity] wide {seed}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} Nq{w.Nq} Nkv{w.Nkv} d{w.d} "
          f"{str(w.dtype).split('.')[-1]} causal={w.causal} seqlens={w.seqlens}", flush=True)
    _full_check(w)


def _zero_groups(q, k, v):
    """Inputs whose smoothed values vanish on whole scale groups, in all three quantizers:
    - K: keys 64..95 (one 32-key subtile: both of its 16-key groups) equal the channel mean
      exactly (every other key pair is mu +- delta on a grid, so the fp64 mean is exactly mu);
    - Q: every row of the second 128-row block equals the same row (its block mean), so those rows
      smooth to zero (per-token scale 0, all codes 0, logits = correction term only);
    - V: channel 7 is zero (scale 0, codes 0, output channel 0)."""
    g = torch.Generator().manual_seed(4242)
    N, Hkv, d = k.shape[1], k.shape[2], k.shape[3]
    mu = torch.randint(-32, 33, (Hkv, d), generator=g).float() / 8
    delta = torch.randint(-16, 17, (N // 2, Hkv, d), generator=g).float() / 8
    e = torch.stack([delta, -delta], dim=1).reshape(N, Hkv, d)
    e[64:96] = 0
    k[0] = (mu[None] + e).to(k.dtype)
    q[0, 128:256] = q[0, 128][None]
    v[0, :, :, 7] = 0


@pytest.mark.parametrize("case", [(128, torch.bfloat16, True), (64, torch.float16, False)],
                         ids=["d128_causal", "d64_full"])
def test_zero_scale_groups(case):
    """Groups whose amax is 0 get scale 0 and codes 0 in the Q, K and V quantizers (bit-exact
    against the oracle), and the attention output still matches."""
    d, dt, causal = case
    w = W.custom(1, 4, 2, 384, 384, d, dt, causal, seed=61, n_outliers=0, k_offset_std=0.0)
    run = _full_check(w, modify=_zero_groups)
    dec = run.decode(run.ws_host(), 0)
    assert np.all(dec["sk"][:, 4:6] == 0) and not dec["kcode"][:, 64:96].any()
    assert np.all(dec["sq"][:, 128:256] == 0) and not dec["qcode"][:, 128:256].any()
    assert np.all(dec["sv"][:, 7] == 0) and not dec["v8"][:, :, 7].any()
    assert not run.o[..., 7].float().abs().sum().item()


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query(causal):
    """Z1 on the GPU: Q = 0 makes every logit 0 and every P~ code 448, so the output is the mean of
    the decoded values (the prefix mean under a causal mask), within the output format's rounding."""
    w = W.custom(1, 2, 1, 300, 300, 128, torch.bfloat16, causal, seed=62)
    run = _full_check(w, out_dtype=torch.float32, modify=lambda q, k, v: q.zero_())
    dec = run.decode(run.ws_host(), 0)
    table = np.array([_e4m3(c) for c in range(256)])
    V = table[dec["v8"][0]] * dec["sv"][0][None, :]
    ref = (np.cumsum(V, axis=0) / np.arange(1, 301)[:, None]) if causal else \
        np.broadcast_to(V.mean(axis=0), V.shape)
    out = run.out_seq(0)
    assert np.max(np.abs(out - ref[None])) < 1e-5 * np.abs(V).max()


def _e4m3(c):
    """OCP e4m3 decode (format definition; used to read the workspace's V codes)."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return float("nan")
    return s * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))



def test_nonfinite_inputs_complete():
    """NaN and Inf inputs give unspecified outputs but must not crash: no address in any kernel
    depends on data values. Every statistic is per (sequence, kv head), so the heads that received
    no non-finite value produce bit-identical outputs to a clean run."""
    w = W.custom(2, 4, 2, 300, 300, 128, torch.bfloat16, True, seed=81)

    def poison(q, k, v):
        q[0, 5, 1, 3] = float("nan")       # batch 0, q head 1 (kv head 0)
        k[0, 200, 0, 7] = float("inf")     # batch 0, kv head 0
        v[1, 17, 1, 0] = float("-inf")     # batch 1, kv head 1
        q[1, 250, 2, :] = float("inf")     # batch 1, q head 2 (kv head 1)

    bad = H.DeviceRun(w, modify=poison)
    bad.run()
    clean = H.DeviceRun(w)
    clean.run()
    as_bits = lambda t: t.view(torch.int16)
    assert torch.equal(as_bits(bad.o[0, :, 2:4]), as_bits(clean.o[0, :, 2:4]))  # batch 0, kv head 1
    assert torch.equal(as_bits(bad.o[1, :, 0:2]), as_bits(clean.o[1, :, 0:2]))  # batch 1, kv head 0


def test_device_seqlens_disagreeing_with_host_copies():
    """Device cu_seqlens that disagree with the host copies the workspace was sized from (here a
    second sequence longer than the stated maximum): the plan kernel treats that sequence as empty,
    so no kernel reads or writes past the workspace or the inputs; its output rows stay untouched
    and the other sequence is still correct."""
    import quantized_exact_attention_token_amd as sage2
    lens = [100, 100]
    w = W.custom(2, 4, 2, 100, 100, 64, torch.float16, False, seed=82, seqlens=lens)
    run = H.DeviceRun(w)
    ref = run.run().clone()
    bad_cu = torch.tensor([0, 100, 5000], dtype=torch.int32, device="cuda")
    p = sage2.make_params(run.q, run.k, run.v, run.o, False, cu_seqlens_q=run.cu,
                          cu_seqlens_kv=run.cu_kv, max_seqlen_q=100, max_seqlen_kv=100)
    p.cu_seqlens_q = bad_cu.data_ptr()      # device copy only; host copies stay [0, 100, 200]
    p.cu_seqlens_kv = bad_cu.data_ptr()
    run.o.fill_(float("nan"))
    sage2.quantize_smooth(p, run.q, run.k, run.v, run.ws)
    sage2.attn_fwd(p, run.ws, run.o)
    torch.cuda.synchronize()
    assert torch.equal(run.o[:100].view(torch.int16), ref[:100].view(torch.int16))
    assert torch.isnan(run.o[100:].float()).all()


def test_attention_on_a_side_stream():
    """The convenience call on a stream other than torch's current one: its workspace is freed on
    return while the kernels may still run, so it must stay reserved for that stream. Allocations
    and writes on the current stream right after the call must not disturb the result."""
    import quantized_exact_attention_token_amd as sage2
    w = W.custom(1, 8, 2, 1000, 1000, 128, torch.bfloat16, True, seed=91, n_outliers=2,
                 outlier_scale=20.0, k_offset_std=4.0)
    run = H.DeviceRun(w)
    ref = run.run().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o = sage2.attention(run.q, run.k, run.v, causal=True, stream=side)
    junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device="cuda") for _ in range(16)]
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    del junk
