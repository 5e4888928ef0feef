"""Seeded synthetic attention inputs.

This module only draws random tensors; it holds none of the method's arithmetic, so the GPU path
and the CPU oracle can both be fed from it.

The pages measure on language, image and video models that are not available here; these recipes
stand in for them: LLM-prefill-like shapes at head dim 128 (bf16) and a diffusion-like long
sequence at head dim 64 (fp16), with the channel outliers and per-channel offsets that the
smoothing steps exist to handle (visual companion "SageAttention2 and Fast Exact INT4 Attention",
section "Channel Outlier Smoothing": a few channels dominate the range).

Draw order, all from one CPU torch.Generator seeded per workload: standard normal fp32 Q
[B, Nq, Hq, d], then K [B, Nkv, Hkv, d], then V, then the outlier channel indices (randperm(d)[:n]
per kv head), then the offset vectors. Outliers multiply the chosen channels of Q and K (the same
channels for a kv head and every q head that shares it) before any offset is added. Optional
deterministic terms follow (no random draws): `key_ramp` adds key_ramp * j / Nkv to every channel
of key j, and `q_shift` adds a constant to every channel of Q, so the logits of a row climb
steadily along the keys (a row whose running max keeps rising). The result is rounded to the input
dtype (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    d: int
    dtype: torch.dtype
    causal: bool
    seed: int
    k_offset_std: float = 0.0       # K += N(0, s^2) per (kv head, channel)
    q_offset_std: float = 0.0       # Q += N(0, s^2) per (q head, channel)
    k_offset_rademacher: float = 0.0  # K += a * (+-1) per (kv head, channel)
    n_outliers: int = 0
    outlier_scale: float = 1.0
    seqlens: list | None = None     # packed variable-length batch: per-sequence (query) lengths
    kv_seqlens: list | None = None  # per-sequence key/value lengths when they differ from seqlens
    key_ramp: float = 0.0           # K[j] += key_ramp * j / Nkv (all channels)
    q_shift: float = 0.0            # Q += q_shift (all channels)
    extra: dict = field(default_factory=dict)

    @property
    def varlen(self) -> bool:
        return self.seqlens is not None

    @property
    def kv_lens(self) -> list | None:
        return self.kv_seqlens if self.kv_seqlens is not None else self.seqlens

    def attention_ops(self) -> float:
        """4 * Nq * Nkv * d per (sequence, q head): one INT4 MAC and one FP8 MAC per (q, k, channel),
        two ops each; halved under a causal mask."""
        if self.varlen:
            tot = sum(4.0 * self.Hq * lq * lk * self.d for lq, lk in zip(self.seqlens, self.kv_lens))
        else:
            tot = 4.0 * self.B * self.Hq * self.Nq * self.Nkv * self.d
        return tot / 2 if self.causal else tot


def cu_seqlens(lens) -> torch.Tensor:
    """Offsets int32 [len(lens) + 1] of a packed batch with these per-sequence lengths."""
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int32), 0)
    return cu


def generate(w: Workload):
    """Returns (q, k, v, cu_seqlens) on the CPU. Dense: q [B, Nq, Hq, d], k/v [B, Nkv, Hkv, d].
    Variable length: q/k/v packed [total, H, d] and the query offsets cu_seqlens int32 [nseq + 1]
    (the key/value offsets are cu_seqlens(w.kv_lens))."""
    g = torch.Generator().manual_seed(w.seed)
    B = 1 if w.varlen else w.B
    Nq = sum(w.seqlens) if w.varlen else w.Nq
    Nkv = sum(w.kv_lens) if w.varlen else w.Nkv
    q = torch.randn(B, Nq, w.Hq, w.d, generator=g, dtype=torch.float32)
    k = torch.randn(B, Nkv, w.Hkv, w.d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Nkv, w.Hkv, w.d, generator=g, dtype=torch.float32)
    grp = w.Hq // w.Hkv
    if w.n_outliers:
        for hk in range(w.Hkv):
            ch = torch.randperm(w.d, generator=g)[: w.n_outliers]
            k[:, :, hk, ch] *= w.outlier_scale
            q[:, :, hk * grp:(hk + 1) * grp, ch] *= w.outlier_scale
    if w.k_offset_std:
        k += (torch.randn(w.Hkv, w.d, generator=g) * w.k_offset_std)[None, None]
    if w.q_offset_std:
        q += (torch.randn(w.Hq, w.d, generator=g) * w.q_offset_std)[None, None]
    if w.k_offset_rademacher:
        sign = torch.randint(0, 2, (w.Hkv, w.d), generator=g).float() * 2 - 1
        k += (sign * w.k_offset_rademacher)[None, None]
    if w.key_ramp:
        k += (torch.arange(Nkv, dtype=torch.float32) * (w.key_ramp / Nkv))[None, :, None, None]
    if w.q_shift:
        q += w.q_shift
    q, k, v = q.to(w.dtype), k.to(w.dtype), v.to(w.dtype)
    if w.varlen:
        return q[0].contiguous(), k[0].contiguous(), v[0].contiguous(), cu_seqlens(w.seqlens)
    return q, k, v, None


def _c1_like(name, B, H, N, causal, seed):
    return Workload(name, B, H, H, N, N, 128, torch.bfloat16, causal, seed,
                    k_offset_std=4.0, n_outliers=3, outlier_scale=20.0)


# The five workloads of the method's measurement plan plus the packed variable-length variant.
WORKLOADS = {
    # tiny sanity case: the oracle runs it whole in well under a second
    "tiny": Workload("tiny", 1, 2, 2, 256, 256, 64, torch.float16, False, 1000,
                     k_offset_std=3.0, n_outliers=2, outlier_scale=10.0),
    "mha4k": _c1_like("mha4k", 2, 32, 4096, False, 1001),
    "prefill8k": _c1_like("prefill8k", 1, 32, 8192, True, 1002),
    "gqa16k": Workload("gqa16k", 1, 32, 8, 16384, 16384, 128, torch.bfloat16, True, 1003,
                       k_offset_std=4.0, q_offset_std=4.0, n_outliers=4, outlier_scale=20.0),
    "diffusion32k": Workload("diffusion32k", 1, 24, 24, 32768, 32768, 64, torch.float16, False, 1004,
                             q_offset_std=2.0, k_offset_rademacher=4.0),
    "diffusion_varlen": Workload("diffusion_varlen", 4, 24, 24, 12288, 12288, 64, torch.float16, False,
                                 1005, q_offset_std=2.0, k_offset_rademacher=4.0,
                                 seqlens=[4096, 8192, 8192, 12288]),
}

# Head-dim-128 length sweep (N = 4K..32K, with and without the causal mask).
SWEEP = {
    f"sweep{N // 1024}k{'_causal' if c else ''}": _c1_like(
        f"sweep{N // 1024}k{'_causal' if c else ''}", 1, 32, N, c, 1100 + N // 4096)
    for N in (4096, 8192, 16384, 32768) for c in (False, True)
}


def custom(B, Hq, Hkv, Nq, Nkv, d, dtype=torch.bfloat16, causal=False, seed=0, seqlens=None,
           kv_seqlens=None, **kw) -> Workload:
    """Small cases for edge tests: same recipe family as the tiny workload unless overridden."""
    base = dict(k_offset_std=3.0, n_outliers=min(2, d), outlier_scale=10.0)
    base.update(kw)
    return Workload(f"custom_s{seed}", B, Hq, Hkv, Nq, Nkv, d, dtype, causal, seed,
                    seqlens=seqlens, kv_seqlens=kv_seqlens, **base)
