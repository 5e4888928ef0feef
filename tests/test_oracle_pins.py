"""Pins for the CPU oracle: each test checks it against something other than itself (closed forms,
invariants, special cases that reduce to a library routine, brute force on tiny inputs).

Which mistake each pin is meant to catch is stated in its docstring.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from quantized_exact_attention_token_amd import workloads as W

LOG2E = np.float32(1.44269504088896340736)


def _L(d, sm_scale=0.0):
    s = np.float32(sm_scale) if sm_scale else np.float32(1.0) / np.sqrt(np.float32(d))
    return np.float32(s * LOG2E)


def _dec_table():
    return np.array([O.e4m3_decode(c) for c in range(256)])


# ------------------------------------------------------------------------------------------------
# L1: FP8 e4m3 codec


def test_e4m3_roundtrip_every_code():
    """decode->encode is the identity on all 254 finite codes (both zeros included): catches a wrong
    bias, a wrong subnormal rule or a wrong mantissa width."""
    for c in range(256):
        if c & 0x7F == 0x7F:
            assert math.isnan(O.e4m3_decode(c))
            continue
        assert O.e4m3_encode(O.e4m3_decode(c)) == c, hex(c)
    # closed forms from the format: largest finite, smallest normal, smallest subnormal
    assert O.e4m3_decode(0x7E) == 448.0
    assert O.e4m3_decode(0x08) == 2.0 ** -6
    assert O.e4m3_decode(0x01) == 2.0 ** -9
    assert O.e4m3_decode(0x38) == 1.0


def test_e4m3_ties_to_even_and_saturation():
    """Midpoints between neighbouring codes go to the even mantissa; anything past 448 saturates;
    values just off a midpoint go to the nearer code."""
    for c in range(0, 0x7E):
        lo, hi = O.e4m3_decode(c), O.e4m3_decode(c + 1)
        mid = (lo + hi) / 2
        even = c if (c & 1) == 0 else c + 1
        assert O.e4m3_encode(mid) == even, hex(c)
        assert O.e4m3_encode(-mid) == 0x80 | even
        assert O.e4m3_encode(np.nextafter(mid, 0.0)) == c
        assert O.e4m3_encode(np.nextafter(mid, 1e9)) == c + 1
    for x in (448.0, 455.9, 464.0, 500.0, 1e30, math.inf):
        assert O.e4m3_encode(x) == 0x7E
        assert O.e4m3_encode(-x) == 0xFE
    assert O.e4m3_encode(-0.0) == 0x80
    assert O.e4m3_encode(2.0 ** -11) == 0x00      # below half the smallest subnormal
    assert O.e4m3_encode(2.0 ** -10) == 0x00      # exactly half: tie to even (0)
    assert O.e4m3_encode(3 * 2.0 ** -10) == 0x02  # 1.5 subnormal steps: tie to even (2)


def test_e4m3_matches_torch_cast_in_range():
    """Cross-check against torch's float32 -> float8_e4m3fn cast (a library routine) on in-range
    values, including exact midpoints."""
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000),
        [(O.e4m3_decode(c) + O.e4m3_decode(c + 1)) / 2 for c in range(0x7E)],
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([O.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------------------------------------
# helpers


def _seq(w, b=0):
    """One sequence of a workload as head-major float32 arrays (exact widening)."""
    q, k, v, cu = W.generate(w)
    if cu is not None:
        s, e = int(cu[b]), int(cu[b + 1])
        q, k, v = q[s:e], k[s:e], v[s:e]
    else:
        q, k, v = q[b], k[b], v[b]
    f = lambda t: t.float().permute(1, 0, 2).contiguous().numpy()
    return f(q), f(k), f(v)


def _cos(a, b):
    a, b = a.ravel().astype(np.float64), b.ravel().astype(np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _budget():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "accuracy_budget.json")) as fh:
        return json.load(fh)


# ------------------------------------------------------------------------------------------------
# smoothing statistics


def test_means_match_exact_sums():
    """k̄ and q̄ equal the exactly-summed means (fp16 inputs of moderate size sum exactly in fp64,
    so numpy's fp64 mean is the same closed form): catches a wrong axis, a wrong count for a ragged
    last Q block, or a mean over the wrong tokens."""
    w = W.custom(1, 4, 2, 300, 333, 64, torch.float16, seed=3, q_offset_std=2.0)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    kbar = (k.astype(np.float64).sum(axis=1) / k.shape[1]).astype(np.float32)
    assert np.array_equal(z.kbar, kbar)
    for b in range(z.qbar.shape[1]):
        rows = q[:, 128 * b:min(q.shape[1], 128 * b + 128)].astype(np.float64)
        qb = (rows.sum(axis=1) / rows.shape[1]).astype(np.float32)
        assert np.array_equal(z.qbar[:, b], qb), b


def test_k_shift_invariance_quantized():
    """I1: adding a constant vector c to every key changes k̄ by exactly c and nothing else in the
    quantized pipeline (inputs on a grid where every sum is exact): catches a dropped or misplaced
    K mean subtraction."""
    rng = np.random.default_rng(11)
    Hq, Hkv, L, d = 2, 1, 64, 64
    q = (rng.integers(-64, 64, (Hq, L, d)) / 16).astype(np.float32)
    k = (rng.integers(-64, 64, (Hkv, L, d)) / 16).astype(np.float32)
    v = rng.standard_normal((Hkv, L, d)).astype(np.float32)
    c = rng.integers(-50, 50, (1, 1, d)).astype(np.float32)
    z0, z1 = O.quantize(q, k, v), O.quantize(q, k + c, v)
    assert np.array_equal(z1.kbar, z0.kbar + c[0])
    for name in ("kcode", "sk", "qcode", "sq", "delta"):
        assert np.array_equal(getattr(z0, name), getattr(z1, name)), name
    o0, _ = O.attn_quant(z0, False)
    o1, _ = O.attn_quant(z1, False)
    assert np.array_equal(o0, o1)
    # without the K mean subtraction the codes do change
    zn = O.quantize(q, k + c, v, flags=O.NO_K_SMOOTH)
    assert not np.array_equal(zn.kcode, z0.kcode)


def test_k_shift_invariance_fp64():
    """I1 for the exact reference: softmax ignores a per-row constant, so shifting every key by c
    leaves FP64 attention unchanged (to rounding)."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 40, 64)).astype(np.float32)
    k = (np.round(rng.standard_normal((2, 50, 64)) * 1024) / 1024).astype(np.float32)  # k + c exact
    v = rng.standard_normal((2, 50, 64)).astype(np.float32)
    c = (rng.integers(-8, 8, (1, 1, 64))).astype(np.float32)
    a = O.attn_fp64(q, k, v, False)
    b = O.attn_fp64(q, k + c, v, False)
    assert np.max(np.abs(a - b)) < 1e-12 * 50


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lkv", [(37, 37), (20, 45), (45, 20)])
def test_fp64_matches_torch_sdpa(causal, Lq, Lkv):
    """The exact reference equals torch's scaled-dot-product attention in float64 (a library
    routine), with a bottom-right aligned causal mask; GQA by repeating K/V heads."""
    rng = np.random.default_rng(13)
    Hq, Hkv, d = 4, 2, 64
    q = rng.standard_normal((Hq, Lq, d)).astype(np.float32)
    k = rng.standard_normal((Hkv, Lkv, d)).astype(np.float32)
    v = rng.standard_normal((Hkv, Lkv, d)).astype(np.float32)
    ours = O.attn_fp64(q, k, v, causal)
    tq = torch.from_numpy(q).double()
    tk = torch.from_numpy(k).double().repeat_interleave(Hq // Hkv, 0)
    tv = torch.from_numpy(v).double().repeat_interleave(Hq // Hkv, 0)
    mask = None
    if causal:
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lkv)[None, :]
        mask = j <= i + (Lkv - Lq)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref.numpy()
    if causal and Lq > Lkv:  # rows with no visible key: the method outputs 0
        dead = np.arange(Lq) + (Lkv - Lq) < 0
        ref[:, dead] = 0.0
    assert np.max(np.abs(ours - ref)) < 1e-12


# ------------------------------------------------------------------------------------------------
# INT4 quantizer


def test_int4_round_trip_bound():
    """I3: every smoothed value is within half a step of its reconstruction, every code is in
    [-7, 7] and each nonzero group reaches +-7 at its largest element: catches a wrong scale, a
    wrong rounding, or a code computed against another group's scale."""
    w = W.custom(1, 4, 2, 200, 230, 128, torch.bfloat16, seed=5, n_outliers=3, outlier_scale=20.0,
                 k_offset_std=4.0)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    qt = q - np.repeat(z.qbar, 128, axis=1)[:, :q.shape[1]]
    rec = z.sq[..., None] * z.qcode
    assert np.all(np.abs(qt - rec) <= z.sq[..., None] / 2 * (1 + 2 ** -20))
    assert np.all(np.abs(z.qcode) <= 7)
    assert np.all(np.abs(z.qcode).max(axis=2)[z.sq > 0] == 7)
    kt = k - z.kbar[:, None, :]
    grp = np.array([O.kgroup(j) for j in range(k.shape[1])])
    skj = z.sk[:, grp]
    assert np.all(np.abs(kt - skj[..., None] * z.kcode) <= skj[..., None] / 2 * (1 + 2 ** -20))
    for g in range(z.sk.shape[1]):
        members = grp == g
        if members.any():
            assert np.abs(z.kcode[:, members]).max() == 7


def test_k_groups_follow_lane_halves():
    """The K scale groups are the two 16-key halves of each 32-key tile split on bit 2 of the key
    index (the keys one gfx950 MFMA lane half owns). Scaling exactly those keys by 1000 scales
    exactly the odd groups' scales: a contiguous or strided grouping fails."""
    rng = np.random.default_rng(21)
    L, d = 96, 64
    k = rng.standard_normal((1, L, d)).astype(np.float32)
    sel = ((np.arange(L) >> 2) & 1) == 1
    k2 = k.copy()
    k2[:, sel] *= 1000
    q = rng.standard_normal((1, 8, d)).astype(np.float32)
    # the K mean is switched off here: it is not under test and the scaled keys would dominate it
    z = O.quantize(q, k2, k2, flags=O.NO_K_SMOOTH)
    ratio = z.sk[0, 1::2] / z.sk[0, 0::2]
    assert np.all(ratio > 300), ratio
    assert [O.kgroup(j) for j in range(32)] == [((j >> 2) & 1) for j in range(32)]


# ------------------------------------------------------------------------------------------------
# correction term and logits


def _grid_inputs(rng, Hq, Lq, Lkv, d, qbar_val):
    """Q rows in +-pairs around a chosen block mean, K rows in +-pairs around a per-channel offset:
    every mean is exact, every smoothed value an integer in [-7, 7] with a 7 in each row/group."""
    assert Lq % 2 == 0 and Lkv % 32 == 0
    qt = rng.integers(-7, 8, (Hq, Lq // 2, d)).astype(np.float32)
    qt[:, :, 0] = 7
    qt = np.stack([qt, -qt], axis=2).reshape(Hq, Lq, d)
    kt = rng.integers(-7, 8, (1, Lkv // 2, d)).astype(np.float32)
    kt[:, :, 1] = 7
    kt = np.stack([kt, -kt], axis=2).reshape(1, Lkv, d)
    koff = rng.integers(-20, 20, (1, 1, d)).astype(np.float32)
    return qt + qbar_val, kt + koff, qt, kt


def test_lossless_grid_codes_and_integer_product():
    """Z2: smoothed values that already lie on the INT4 grid quantize losslessly (scale 1, codes
    equal values) and the integer product equals numpy's exact integer matmul: catches a transposed
    operand or a wrong index in S."""
    rng = np.random.default_rng(31)
    Hq, Lq, Lkv, d = 2, 128, 64, 64
    qbar = (rng.integers(-16, 16, (Hq, 1, d)) / 8).astype(np.float32)
    q, k, qt, kt = _grid_inputs(rng, Hq, Lq, Lkv, d, qbar)
    v = rng.standard_normal((1, Lkv, d)).astype(np.float32)
    z = O.quantize(q, k, v)
    assert np.all(z.sq == 1.0) and np.all(z.sk == 1.0)
    assert np.array_equal(z.qcode, qt.astype(np.int8))
    assert np.array_equal(z.kcode, kt.astype(np.int8))
    S = O.qk_i32(z)
    ref = np.einsum("hid,jd->hij", qt.astype(np.int64), kt[0].astype(np.int64))
    assert np.array_equal(S, ref)


def test_q_correction_restores_logits():
    """I2: with lossless INT4 codes, the dequantized logits plus the correction q̄·k̃ equal the exact
    smoothed-K logits L·q·k̃, and differ from the unsmoothed L·q·k by a per-row constant L·q·k̄ that
    softmax ignores: catches a dropped correction term or a wrong sign."""
    rng = np.random.default_rng(32)
    Hq, Lq, Lkv, d = 2, 256, 96, 64
    qbar = (rng.integers(-24, 24, (Hq, 1, d)) / 8).astype(np.float32)
    q, k, qt, kt = _grid_inputs(rng, Hq, Lq, Lkv, d, qbar)
    v = rng.standard_normal((1, Lkv, d)).astype(np.float32)
    z = O.quantize(q, k, v)
    x = O.logits(z, False).astype(np.float64)
    L = float(_L(d))
    exact = L * np.einsum("hid,jd->hij", q.astype(np.float64), kt[0].astype(np.float64))
    assert np.max(np.abs(x - exact) / (np.abs(exact) + 1)) < 2 ** -20
    raw = L * np.einsum("hid,jd->hij", q.astype(np.float64), k[0].astype(np.float64))
    diff = x - raw
    assert np.max(np.abs(diff - diff[:, :, :1])) < 1e-3 * (1 + np.abs(raw).max())
    # the ablation without Q smoothing has no correction and a different grid: logits still close
    # to exact only up to quantization error; dropping the correction on its own would be far off
    x_no = x - np.repeat(z.delta, 128, axis=1)[:, :Lq].astype(np.float64)
    assert np.max(np.abs(x_no - exact)) > 1.0


def test_delta_is_mean_times_smoothed_k():
    """The stored correction equals L·(q̄·k̃), k̃ = f32(k - k̄), computed with numpy's fp64 matmul
    (library routine), within the error bound of an f32 multiply-add chain over d channels
    (gamma_d = d u / (1 - d u), u = 2^-24, times sum_c |q̄_c k̃_c|) plus the final f32 multiply's
    rounding. A dropped, repeated or sign-flipped channel term is far outside that bound."""
    w = W.custom(1, 4, 2, 300, 200, 64, torch.float16, seed=9, q_offset_std=2.0)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    kt = (k - z.kbar[:, None, :]).astype(np.float32).astype(np.float64)
    qb = z.qbar.astype(np.float64)
    ktr = np.repeat(kt, 2, axis=0)
    L = float(_L(64))
    ref = np.einsum("hbd,hjd->hbj", qb, ktr) * L
    sabs = np.einsum("hbd,hjd->hbj", np.abs(qb), np.abs(ktr)) * L
    u = 2.0 ** -24
    gamma = 64 * u / (1 - 64 * u)
    bound = gamma * sabs * (1 + u) + u * np.abs(ref) + 1e-30
    err = np.abs(z.delta.astype(np.float64) - ref)
    assert np.all(err <= bound)
    # the bound is tight enough to see one channel term: every |q̄_c k̃_c| of a random input is
    # larger than the allowed error for most entries
    one_term = np.abs(qb[:, :, :1]) * np.abs(ktr[:, None, :, 0]) * L
    assert np.mean(one_term > bound) > 0.9


def test_logits_within_int4_error_bound():
    """The dequantized logits differ from the exact smoothed logits L·q·(k - k̄) by no more than
    the closed-form INT4 bound L·sum_c(|q̃| s_k/2 + |k̃| s_q/2 + s_q s_k/4) (plus f32 slack):
    catches a scale taken from the wrong token or group."""
    w = W.custom(1, 2, 1, 256, 200, 128, torch.bfloat16, seed=10, n_outliers=3, outlier_scale=20.0,
                 k_offset_std=4.0, q_offset_std=1.0)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    x = O.logits(z, False).astype(np.float64)
    L = float(_L(128))
    qt = (q - np.repeat(z.qbar, 128, axis=1)[:, :q.shape[1]]).astype(np.float64)
    kt = (k - z.kbar[:, None, :]).astype(np.float64)
    kt2 = np.repeat(kt, 2, axis=0)
    exact = L * np.einsum("hid,hjd->hij", q.astype(np.float64), kt2)
    grp = np.array([O.kgroup(j) for j in range(k.shape[1])])
    skj = np.repeat(z.sk[:, grp], 2, axis=0).astype(np.float64)    # [Hq, Lkv]
    sq = z.sq.astype(np.float64)                                    # [Hq, Lq]
    bound = L * (np.abs(qt).sum(-1)[:, :, None] * skj[:, None, :] / 2
                 + np.abs(kt2).sum(-1)[:, None, :] * sq[:, :, None] / 2
                 + 128 * sq[:, :, None] * skj[:, None, :] / 4)
    err = np.abs(x - exact)
    assert np.all(err <= bound * (1 + 1e-5) + 1e-4 * (1 + np.abs(exact)))
    assert err.max() > 0  # not vacuous


# ------------------------------------------------------------------------------------------------
# online softmax and two-level accumulation


@pytest.mark.parametrize("causal", [False, True])
def test_online_equals_two_pass(causal):
    """I4: with P~ left unquantized, the tiled online softmax with the rescale-and-fold equals a
    two-pass softmax over the same logits for any tile size: catches a wrong rescale factor, a
    missing fold or a max that is not carried across tiles."""
    w = W.custom(1, 2, 1, 150, 150, 64, torch.float16, seed=14)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    x = O.logits(z, causal).astype(np.float64)
    dec = _dec_table()
    V = dec[z.v8[0]] * z.sv[0][None, :]
    M = x.max(axis=2, keepdims=True)
    wgt = np.exp2(x - M)
    ref = np.einsum("hij,jc->hic", wgt, V) / wgt.sum(axis=2, keepdims=True)
    for bn in (1, 16, 64, 150):
        out, _ = O.attn_quant(z, causal, bn=bn, flags=O.ATTN_NO_P8)
        assert np.max(np.abs(out - ref)) < 1e-5 * np.abs(V).max(), bn


def test_p8_rounding_effect_bounded():
    """B1: quantizing P~ to e4m3 changes each weight by at most 2^-4 relative (3 mantissa bits),
    so the output moves by at most 2^-4·max|v| against the unquantized form."""
    wl = W.WORKLOADS["tiny"]
    q, k, v = _seq(wl)
    z = O.quantize(q, k, v)
    a, _ = O.attn_quant(z, False)
    b, _ = O.attn_quant(z, False, flags=O.ATTN_NO_P8)
    vmax = (_dec_table()[z.v8] * z.sv[:, None, :]).max()
    diff = np.abs(a - b).max()
    assert 0 < diff <= 2 ** -4 * vmax


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_value_mean(causal):
    """Z1: Q = 0 makes every logit 0, so every P~ is exactly 448 and the output is the plain mean of
    the decoded values (the prefix mean under a causal mask)."""
    rng = np.random.default_rng(41)
    L, d = 100, 64
    q = np.zeros((2, L, d), np.float32)
    k = rng.standard_normal((1, L, d)).astype(np.float32)
    v = rng.standard_normal((1, L, d)).astype(np.float32)
    z = O.quantize(q, k, v)
    out, allow = O.attn_quant(z, causal)
    V = _dec_table()[z.v8[0]] * z.sv[0][None, :]
    if causal:
        ref = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None]
    else:
        ref = np.broadcast_to(V.mean(axis=0), (L, d))
    assert np.max(np.abs(out - ref[None])) < 1e-6 * np.abs(V).max()
    assert np.all(allow == 0)


def test_single_key_returns_its_value():
    """Z3: with one key the output is that key's value up to the FP8 step of V."""
    rng = np.random.default_rng(42)
    q = rng.standard_normal((2, 5, 64)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64)).astype(np.float32)
    v = rng.standard_normal((1, 1, 64)).astype(np.float32)
    z = O.quantize(q, k, v)
    out, _ = O.attn_quant(z, False)
    ref = _dec_table()[z.v8[0, 0]] * z.sv[0]
    assert np.max(np.abs(out - ref)) < 1e-6
    assert np.max(np.abs(out - v[0, 0])) <= np.abs(v).max() * 2 ** -4


def test_one_hot_attention():
    """Z4: a logit gap far beyond the FP8 range makes every other P~ zero: the output is the
    winning key's value."""
    rng = np.random.default_rng(43)
    L, d = 130, 64
    q = np.zeros((1, 4, d), np.float32)
    q[:, :, 0] = 30.0
    q[:, 1::2, 0] = 20.0
    k = (rng.standard_normal((1, L, d)) * 0.1).astype(np.float32)
    k[0, 77, 0] = 60.0
    v = rng.standard_normal((1, L, d)).astype(np.float32)
    z = O.quantize(q, k, v)
    out, _ = O.attn_quant(z, False)
    ref = _dec_table()[z.v8[0, 77]] * z.sv[0]
    # the winner's own weight is 448 in P~ but 2^t with t = x - (x - log2 448) in f32 in the row
    # sum: a relative difference of at most two f32 roundings at the logit's magnitude
    xmax = float(np.abs(O.logits(z, False)).max())
    tol = 2.0 ** -22 * (xmax + 16) * np.abs(ref).max()
    assert np.max(np.abs(out - ref)) <= tol


def test_gqa_equals_repeated_kv():
    """E1: grouped-query attention equals multi-head attention with each kv head repeated for its
    consecutive q heads, bit for bit: catches a wrong q-head -> kv-head map."""
    w = W.custom(1, 4, 2, 140, 170, 64, torch.float16, seed=15)
    q, k, v = _seq(w)
    z1 = O.quantize(q, k, v)
    z2 = O.quantize(q, np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0))
    for causal in (False, True):
        a, _ = O.attn_quant(z1, causal)
        b, _ = O.attn_quant(z2, causal)
        assert np.array_equal(a, b)


def test_fully_masked_rows_are_zero():
    """With Lq > Lkv and a bottom-right causal mask the first Lq - Lkv rows see no key and output 0."""
    rng = np.random.default_rng(44)
    q = rng.standard_normal((1, 80, 64)).astype(np.float32)
    k = rng.standard_normal((1, 50, 64)).astype(np.float32)
    v = rng.standard_normal((1, 50, 64)).astype(np.float32)
    z = O.quantize(q, k, v)
    out, _ = O.attn_quant(z, True)
    assert np.all(out[:, :30] == 0) and np.all(np.abs(out[:, 30:]).sum(-1) > 0)


# ------------------------------------------------------------------------------------------------
# whole method vs the exact rule


def test_quantized_pipeline_vs_exact_on_outliers():
    """Q1 on the tiny outlier workload: smoothing beats the naive pipeline (the pages show naive
    INT4 shifting softmax winners), and an independent numpy quantize-dequantize simulation of the
    same groups (fp64, library softmax) lands at the same accuracy. The outliers here are zero-mean
    channel multipliers, which a mean subtraction cannot remove, so INT4 keeps only about cos 0.93
    against the exact result; a value far from the simulation signals a mistake in the oracle."""
    wl = W.WORKLOADS["tiny"]
    q, k, v = _seq(wl)
    exact = O.attn_fp64(q, k, v, wl.causal)
    z = O.quantize(q, k, v)
    out, _ = O.attn_quant(z, wl.causal)
    zn = O.quantize(q, k, v, flags=O.NO_K_SMOOTH | O.NO_Q_SMOOTH)
    naive, _ = O.attn_quant(zn, wl.causal)
    c_s, c_n = _cos(out, exact), _cos(naive, exact)
    assert c_n < c_s, (c_n, c_s)
    # independent simulation: dequantized Q (block mean + per-token INT4) and K (per 16-key group)
    Q, K, V = (a.astype(np.float64) for a in (q, k, v))
    kt = K - K.mean(axis=1, keepdims=True)
    nb = (Q.shape[1] + 127) // 128
    qb = np.concatenate([np.repeat(Q[:, 128 * b:128 * b + 128].mean(1, keepdims=True),
                                   min(128, Q.shape[1] - 128 * b), 1) for b in range(nb)], 1)
    qt = Q - qb
    sq = np.abs(qt).max(-1, keepdims=True) / 7
    qd = np.round(qt / sq) * sq + qb
    grp = 2 * (np.arange(K.shape[1]) // 32) + ((np.arange(K.shape[1]) >> 2) & 1)
    kd = np.zeros_like(kt)
    for g in np.unique(grp):
        m = grp == g
        s = np.abs(kt[:, m]).max(axis=(1, 2), keepdims=True) / 7
        kd[:, m] = np.round(kt[:, m] / s) * s
    t = torch.from_numpy
    sim = torch.nn.functional.scaled_dot_product_attention(t(qd), t(kd), t(V)).numpy()
    c_sim = _cos(sim, exact)
    assert abs(c_s - c_sim) < 0.02, (c_s, c_sim)
    # the recorded accuracy floor of this workload (tests/golden/accuracy_budget.json)
    assert c_s >= _budget()["tiny"]["floor_cos_fp64"], c_s


def test_quantized_pipeline_close_to_exact_without_outliers():
    """Without channel multipliers (offsets only, which smoothing removes exactly) the pipeline
    reaches cos >= 0.99 against FP64 attention; dropping the Q correction term breaks it."""
    w = W.custom(1, 2, 2, 384, 384, 64, torch.float16, seed=17, n_outliers=0, k_offset_std=4.0,
                 q_offset_std=4.0)
    q, k, v = _seq(w)
    exact = O.attn_fp64(q, k, v, False)
    z = O.quantize(q, k, v)
    out, _ = O.attn_quant(z, False)
    assert _cos(out, exact) >= 0.99, _cos(out, exact)
    z.delta[:] = 0.0
    broken, _ = O.attn_quant(z, False)
    assert _cos(broken, exact) < 0.9


def test_q_smoothing_matters_with_q_offset():
    """With a large per-channel Q mean the Q smoothing plus correction improves accuracy over
    K smoothing alone."""
    w = W.custom(1, 2, 2, 256, 256, 64, torch.float16, seed=16, q_offset_std=4.0,
                 k_offset_rademacher=4.0, n_outliers=0, k_offset_std=0.0)
    q, k, v = _seq(w)
    exact = O.attn_fp64(q, k, v, False)
    full, _ = O.attn_quant(O.quantize(q, k, v), False)
    konly, _ = O.attn_quant(O.quantize(q, k, v, flags=O.NO_Q_SMOOTH), False)
    assert np.abs(full - exact).max() < np.abs(konly - exact).max()
    assert _cos(full, exact) > 0.99


def test_per_block_scales_are_block_maxima():
    """Per-block ablation ([VIZ: Per-Thread INT4 Geometry] contrasts per-block and per-thread
    scales): each 128-token Q block's scale is the largest per-token scale in it, each 64-key K
    block's scale the largest of its four 16-key group scales (amax/7 is monotone in amax and
    correctly rounded), and every code still round-trips within half its scale."""
    w = W.custom(1, 2, 1, 300, 200, 64, torch.float16, seed=21)
    q, k, v = _seq(w)
    zt = O.quantize(q, k, v)
    zb = O.quantize(q, k, v, flags=O.PER_BLOCK)
    for b0 in range(0, 300, 128):
        blk = slice(b0, min(300, b0 + 128))
        assert np.all(zb.sq[:, blk] == zt.sq[:, blk].max(axis=1, keepdims=True))
    ngk = zt.sk.shape[1]
    for g0 in range(0, ngk, 4):
        grp = slice(g0, min(ngk, g0 + 4))
        assert np.all(zb.sk[:, grp] == zt.sk[:, grp].max(axis=1, keepdims=True))
    # round trip within half a scale, for both operands
    qt = q - np.repeat(zb.qbar, 128, axis=1)[:, :300]
    assert np.all(np.abs(zb.qcode * zb.sq[..., None] - qt) <= zb.sq[..., None] / 2 * (1 + 1e-6))
    kt = k - zb.kbar[:, None, :]
    sk_key = zb.sk[:, [O.kgroup(j) for j in range(200)]]
    assert np.all(np.abs(zb.kcode * sk_key[..., None] - kt) <= sk_key[..., None] / 2 * (1 + 1e-6))
    assert np.array_equal(zb.v8, zt.v8) and np.array_equal(zb.delta, zt.delta)


def test_per_thread_scales_beat_per_block_on_outliers():
    """The pages' claim that thread-granularity scales recover accuracy lost by coarser ones."""
    w = W.WORKLOADS["tiny"]
    q, k, v = _seq(w)
    exact = O.attn_fp64(q, k, v, False)
    per_thread, _ = O.attn_quant(O.quantize(q, k, v), False)
    per_block, _ = O.attn_quant(O.quantize(q, k, v, flags=O.PER_BLOCK), False)
    assert _cos(per_thread, exact) > _cos(per_block, exact)


# ------------------------------------------------------------------------------------------------
# P~ codes, error-budget modes, accumulation ablations, the alternative correction-term reading


def _recipe(name, N, Hkv=1, causal=None):
    """A workload's value recipe (offsets, outliers, dtype, d) at a reduced length and head count."""
    import dataclasses
    w = W.WORKLOADS[name]
    grp = w.Hq // w.Hkv
    kw = dict(B=1, Hq=grp * Hkv, Hkv=Hkv, Nq=N, Nkv=N, seqlens=None, kv_seqlens=None)
    if causal is not None:
        kw["causal"] = causal
    return dataclasses.replace(w, **kw)


def test_p8_codes_match_library_cast():
    """The P~ codes the oracle reports are the e4m3 codes (torch's float8_e4m3fn cast, a library
    routine) of 2^t, t = x - (m - log2 448) in f32 with m the running max over 128-key tiles, on
    every entry the oracle does not flag as ambiguous; masked keys get code 0."""
    w = W.custom(1, 2, 1, 300, 300, 64, torch.float16, True, seed=51)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    rows = np.array([0, 5, 130, 299], np.int32)
    _, _, p8, amb = O.attn_quant(z, True, rows=rows, codes=True)
    x = O.logits(z, True, rows=rows)
    log2_448 = np.float32(8.80735492205760410750)
    n_checked = 0
    for h in range(2):
        for r_, i in enumerate(rows):
            m = np.float32(-np.inf)
            for t0 in range(0, 300, 128):
                xs = x[h, r_, t0:t0 + 128]
                m = np.maximum(m, xs.max())
                if m == -np.inf:
                    continue
                t = (xs - np.float32(m - log2_448)).astype(np.float32)
                p = np.exp2(t.astype(np.float64))
                ref = torch.from_numpy(p).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                ref = np.where(np.isneginf(xs), 0, ref)
                got = p8[h, r_, t0:t0 + 128]
                ok = amb[h, r_, t0:t0 + 128] == 0
                assert np.array_equal(got[ok], ref[ok]), (h, i, t0)
                n_checked += int(ok.sum())
    assert n_checked > 1000
    assert np.all(p8[:, 0, 1:] == 0)  # row 0 sees key 0 only under the causal mask


def test_p8_codes_of_zero_query():
    """Q = 0: every visible logit is 0, so every P~ code is 0x7E (448) and none is ambiguous."""
    rng = np.random.default_rng(52)
    q = np.zeros((1, 40, 64), np.float32)
    k = rng.standard_normal((1, 40, 64)).astype(np.float32)
    v = rng.standard_normal((1, 40, 64)).astype(np.float32)
    z = O.quantize(q, k, v)
    _, _, p8, amb = O.attn_quant(z, True, codes=True)
    vis = np.arange(40)[None, :] <= np.arange(40)[:, None]
    assert np.all(p8[0][vis] == 0x7E) and np.all(p8[0][~vis] == 0) and not amb.any()


def test_ambiguity_radius_is_exp2_error_bound():
    """An entry is flagged ambiguous exactly when e4m3(2^(t - r)) != e4m3(2^(t + r)) for
    r = 2^-22 (the hardware exp2's error bound in t), re-derived here with torch's e4m3 cast; on
    random data such entries are rare (about 16 r per key: e4m3 has about 8 rounding boundaries per
    binade, each with a window 2r wide)."""
    w = W.custom(1, 2, 1, 256, 512, 64, torch.float16, False, seed=53)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    rows = np.arange(0, 256, 3, dtype=np.int32)
    _, _, p8, amb = O.attn_quant(z, False, rows=rows, codes=True)
    x = O.logits(z, False, rows=rows)
    log2_448 = np.float32(8.80735492205760410750)
    r = 2.0 ** -22
    enc = lambda a: torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for h in range(2):
        for r_ in range(len(rows)):
            m = np.float32(-np.inf)
            for t0 in range(0, 512, 128):
                xs = x[h, r_, t0:t0 + 128]
                m = np.maximum(m, xs.max())
                t = (xs - np.float32(m - log2_448)).astype(np.float32).astype(np.float64)
                ref = enc(np.exp2(t - r)) != enc(np.exp2(t + r))
                assert np.array_equal(amb[h, r_, t0:t0 + 128].astype(bool), ref)
    frac = amb.mean()
    assert frac < 50 * 16 * r, frac


def test_exact_modes_reduce_to_fp64_attention():
    """With Q, K and V unquantized and P~ kept unquantized the pipeline is plain softmax attention:
    it equals the FP64 reference (itself pinned to torch SDPA) up to the f32 rounding of the
    logits (relative 2^-24 of |x| in each weight)."""
    w = W.custom(1, 4, 2, 200, 170, 64, torch.float16, True, seed=54)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v)
    flags = O.ATTN_NO_P8 | O.ATTN_V_EXACT | O.ATTN_QK_EXACT
    out, _ = O.attn_quant(z, True, flags=flags, exact=(q, k, v))
    ref = O.attn_fp64(q, k, v, True)
    assert np.max(np.abs(out - ref)) < 1e-5 * np.abs(v).max()
    # each exact mode on its own moves the result towards the reference
    full, _ = O.attn_quant(z, True)
    for f in (O.ATTN_V_EXACT, O.ATTN_QK_EXACT):
        part, _ = O.attn_quant(z, True, flags=f, exact=(q, k, v))
        assert np.abs(part - ref).max() != np.abs(full - ref).max()


def test_accumulation_ablation_models():
    """Narrow accumulator at 52 mantissa bits (fp64's own width) and the single-level form with
    exact accumulation both equal the default two-level result; with a narrow accumulator the
    single-level form loses more accuracy than the two-level form, whose fold is exact (the
    research record's reason for two levels); fewer bits lose more."""
    wl = _recipe("gqa16k", 1024)
    q, k, v = _seq(wl)
    z = O.quantize(q, k, v)
    rows = np.arange(0, 1024, 7, dtype=np.int32)
    base, _ = O.attn_quant(z, True, rows=rows)
    for flags, bits in ((O.ATTN_NARROW_ACC, 52), (O.ATTN_SINGLE_LEVEL, 0),
                        (O.ATTN_NARROW_ACC | O.ATTN_SINGLE_LEVEL, 52)):
        o, _ = O.attn_quant(z, True, rows=rows, flags=flags, acc_bits=bits)
        assert np.max(np.abs(o - base)) <= 1e-12 * np.abs(base).max(), flags
    errs = {}
    for bits in (6, 10):
        for single in (False, True):
            f = O.ATTN_NARROW_ACC | (O.ATTN_SINGLE_LEVEL if single else 0)
            o, _ = O.attn_quant(z, True, rows=rows, flags=f, acc_bits=bits)
            errs[bits, single] = np.abs(o - base).max()
    assert errs[6, True] > errs[6, False] and errs[10, True] > errs[10, False], errs
    assert errs[6, True] > errs[10, True] and errs[6, False] > errs[10, False], errs


def test_single_level_band_scales_with_its_rate():
    """The single-level error band is non-negative, zero where the output is zero, and halves with
    each extra bit of the per-step rate."""
    wl = W.WORKLOADS["tiny"]
    q, k, v = _seq(wl)
    z = O.quantize(q, k, v)
    _, _, b10 = O.attn_quant(z, False, flags=O.ATTN_SINGLE_LEVEL, band_log2=10)
    _, _, b11 = O.attn_quant(z, False, flags=O.ATTN_SINGLE_LEVEL, band_log2=11)
    assert np.all(b10 >= 0) and b10.max() > 0
    assert np.allclose(b11 * 2, b10, rtol=1e-12, atol=0)


def test_delta_f64_reading_is_correctly_rounded():
    """The alternative correction-term reading (one fp64 dot product, rounded once) equals numpy's
    fp64 matmul L*(q̄.k̃) to half an f32 ulp (plus the fp64 sum's own rounding)."""
    w = W.custom(1, 4, 2, 300, 200, 64, torch.float16, seed=55, q_offset_std=2.0)
    q, k, v = _seq(w)
    z = O.quantize(q, k, v, flags=O.DELTA_F64)
    kt = (k - z.kbar[:, None, :]).astype(np.float32).astype(np.float64)
    ref = np.einsum("hbd,hjd->hbj", z.qbar.astype(np.float64), np.repeat(kt, 2, axis=0)) * float(_L(64))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(z.delta - ref) <= 0.5 * ulp * (1 + 1e-9) + 1e-12 * np.abs(ref))


@pytest.mark.parametrize("name", ["tiny", "mha4k", "prefill8k", "gqa16k", "diffusion32k"])
def test_correction_chain_reading_moves_output_little(name):
    """The correction term is read as an f32 channel-order multiply-add chain (the kernel's
    arithmetic); the plain alternative is one fp64 dot product. On each workload's recipe (reduced
    to 1024 tokens and one kv-head group) the two readings give outputs within 1e-3 of each other,
    a tenth of the parity bar, and change only a small share of the P~ codes."""
    wl = W.WORKLOADS["tiny"] if name == "tiny" else _recipe(name, 1024)
    q, k, v = _seq(wl)
    rows = np.arange(0, q.shape[1], 5, dtype=np.int32)
    za = O.quantize(q, k, v)
    zb = O.quantize(q, k, v, flags=O.DELTA_F64)
    oa, _, pa, _ = O.attn_quant(za, wl.causal, rows=rows, codes=True)
    ob, _, pb, _ = O.attn_quant(zb, wl.causal, rows=rows, codes=True)
    diff = np.abs(oa - ob).max()
    changed = float((pa != pb).mean())
    print(f"[R5] {name}: max |out f32 chain - out fp64| = {diff:.3e}, P~ codes changed: "
          f"{changed:.2e} of {pa.size}, delta entries differing: {float((za.delta != zb.delta).mean()):.3f}")
    assert diff < 1e-3, diff
    assert changed < 1e-3, changed


def test_v_quantizer_half_step_and_amax_at_448():
    """V: every element is within half an e4m3 step (of the scaled value's binade) of its decoded
    code times the channel scale, and each channel's largest |v| over the whole sequence maps to
    exactly the code of +-448. An amax over the wrong token range breaks one or the other."""
    w = W.custom(1, 2, 2, 384, 384, 64, torch.bfloat16, seed=56)
    q, k, v = _seq(w)
    v[0, 300, 5] = 37.0  # one large value late in the sequence, in one channel
    z = O.quantize(q, k, v)
    dec = _dec_table()[z.v8]
    y = np.abs(v) / z.sv[:, None, :]
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    err = np.abs(v - dec * z.sv[:, None, :])
    assert np.all(err <= z.sv[:, None, :] * (step / 2 + 2.0 ** -20 * y))
    am = np.abs(v).argmax(axis=1)
    for g in range(2):
        for c in range(64):
            code = z.v8[g, am[g, c], c]
            assert code in (0x7E, 0xFE), (g, c, hex(code))
    assert np.all(np.abs(dec).max(axis=1) == 448.0)
    assert z.sv[0, 5] == np.float32(37.0) / np.float32(448.0)


@pytest.mark.parametrize("name", ["tiny", "prefill8k"])
def test_accuracy_budget_reproduces(name):
    """The stored accuracy budget is what the oracle computes now (a changed oracle must rewrite it
    with tests/golden/make_accuracy_budget.py), and it carries the structure the figures rest on:
    INT4 Q/K alone accounts for the method's error against FP64 (within 0.01 of the full method's
    cosine), FP8 V alone and FP8 P~ alone each keep cos >= 0.999, and with a narrow accumulator
    the two-level form stays closer to the full method than the single-level form (the research
    record's reason for the FP32 fold)."""
    import sys
    import os
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_accuracy_budget as MB
    stored = _budget()[name]
    now = MB.budget(W.WORKLOADS[name])
    for a, b in zip(stored["sequences"], now["sequences"]):
        assert a["rows"] == b["rows"]
        for k, v in a["settings"].items():
            assert abs(v["cos"] - b["settings"][k]["cos"]) < 1e-12, (k, v, b["settings"][k])
        st = a["settings"]
        assert abs(st["full"]["cos"] - st["int4_qk_only"]["cos"]) < 0.01
        assert st["fp8_v_only"]["cos"] >= 0.999 and st["fp8_p_only"]["cos"] >= 0.999
        for bits in (13, 10):
            assert (st[f"narrow{bits}_two_level"]["maxerr_vs_full"]
                    < st[f"narrow{bits}_single_level"]["maxerr_vs_full"])



@pytest.mark.parametrize("name", ["tiny", "gqa16k", "diffusion32k"])
def test_softmax_tile_size_reading(name):
    """The online softmax's key tile is part of the result (P~ is rounded against the running max
    of the tiles seen so far), so the oracle and the kernel share one: 128 keys. Other tile sizes
    give other, equally valid roundings: each is within 2^-4 max|v| of the unquantized-P~ result
    (pin B1), so two of them differ by at most max|v| / 8, and the accuracy against FP64 attention
    does not depend on the choice (cosines within 1e-4)."""
    wl = W.WORKLOADS["tiny"] if name == "tiny" else _recipe(name, 1024)
    q, k, v = _seq(wl)
    rows = np.arange(0, q.shape[1], 5, dtype=np.int32)
    z = O.quantize(q, k, v)
    exact = O.attn_fp64(q, k, v, wl.causal, rows=rows)
    ref, _ = O.attn_quant(z, wl.causal, rows=rows)
    vmax = float((_dec_table()[z.v8] * z.sv[:, None, :]).max())
    for bn in (32, 64, 256):
        out, _ = O.attn_quant(z, wl.causal, rows=rows, bn=bn)
        d = float(np.abs(out - ref).max())
        print(f"[R11] {name}: tile {bn} vs 128: max |diff| {d:.4f}, cos vs FP64 {_cos(out, exact):.5f} "
              f"vs {_cos(ref, exact):.5f}")
        assert d <= vmax / 8
        assert abs(_cos(out, exact) - _cos(ref, exact)) < 1e-4
