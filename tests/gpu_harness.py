"""Shared helpers for the GPU parity tests and the benchmark: run the HIP path through the C ABI,
decode the workspace into the oracle's canonical arrays, and compare with the oracle.

Decoding only reorders bytes (nibble unpacking, the V tile permutation); it does no arithmetic of
the method.
"""
from __future__ import annotations

import numpy as np
import torch

import quantized_exact_attention_token_amd as sage2
from quantized_exact_attention_token_amd import workloads as W

OUT_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


class DeviceRun:
    """Inputs on the device, params, workspace, output."""

    def __init__(self, w: W.Workload, out_dtype=None, layout: str = "bnhd", device="cuda",
                 flags: int = 0, sm_scale: float = 0.0, modify=None):
        """`modify(q, k, v)` may edit the generated CPU tensors in place (special-case inputs)."""
        self.w = w
        self.flags = flags
        self.sm_scale = sm_scale  # 0: the library default 1/sqrt(d)
        q, k, v, cu = W.generate(w)
        if modify is not None:
            modify(q, k, v)
        self.q_cpu, self.k_cpu, self.v_cpu, self.cu_cpu = q, k, v, cu
        self.cu_kv_cpu = None if cu is None else W.cu_seqlens(w.kv_lens)
        dev = torch.device(device)
        if layout == "bhnd" and cu is None:  # same values, [B, H, N, d] storage seen through strides
            q, k, v = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        odt = out_dtype or w.dtype
        self.o = torch.full(self.q.shape, float("nan"), dtype=odt, device=dev)
        if layout == "bhnd" and cu is None:  # the output in [B, H, N, d] storage as well
            B_, N_, H_, d_ = self.q.shape
            self.o = torch.full((B_, H_, N_, d_), float("nan"), dtype=odt, device=dev).permute(0, 2, 1, 3)
        self.cu = None if cu is None else cu.to(dev)
        self.cu_kv = None if cu is None else self.cu_kv_cpu.to(dev)
        self.p = sage2.make_params(self.q, self.k, self.v, self.o, w.causal, sm_scale=sm_scale,
                                   cu_seqlens_q=self.cu, cu_seqlens_kv=self.cu_kv,
                                   max_seqlen_q=w.Nq if cu is not None else None,
                                   max_seqlen_kv=w.Nkv if cu is not None else None,
                                   flags=flags)
        self.ws = torch.empty(sage2.workspace_size(self.p), dtype=torch.uint8, device=dev)
        self.lay = sage2.workspace_layout(self.p)

    def prepass(self):
        sage2.quantize_smooth(self.p, self.q, self.k, self.v, self.ws)

    def attn(self):
        sage2.attn_fwd(self.p, self.ws, self.o)

    def run(self):
        self.prepass()
        self.attn()
        torch.cuda.synchronize()
        return self.o

    def attn_as(self, dtype):
        """The attention output from the same workspace into a fresh tensor of another dtype."""
        o = torch.full(self.q.shape, float("nan"), dtype=dtype, device=self.q.device)
        p = sage2.make_params(self.q, self.k, self.v, o, self.w.causal, sm_scale=self.sm_scale,
                              cu_seqlens_q=self.cu, cu_seqlens_kv=self.cu_kv,
                              max_seqlen_q=self.w.Nq if self.cu is not None else None,
                              max_seqlen_kv=self.w.Nkv if self.cu is not None else None,
                              flags=self.flags)
        sage2.attn_fwd(p, self.ws, o)
        torch.cuda.synchronize()
        return o

    def debug_tiles(self, q_begin, q_count, with_output=False):
        """INT32 S and P~ codes of rows [q_begin, q_begin + q_count) from the attention kernel's own
        tiles: ([B, Hq, q_count, N_kv] int32, uint8) numpy arrays; entries the kernel does not
        visit keep the fill values (int32 min, 0xFF). With with_output the kernel also writes a
        fresh output tensor, returned third."""
        w = self.w
        shape = (self.p.B, w.Hq, q_count, self.p.N_kv)
        s = torch.full(shape, -(2 ** 31), dtype=torch.int32, device=self.q.device)
        p8 = torch.full(shape, 0xFF, dtype=torch.uint8, device=self.q.device)
        o = torch.full_like(self.o, float("nan")) if with_output else None
        sage2.debug_attn_tiles(self.p, self.ws, q_begin, q_count, s, p8, o)
        torch.cuda.synchronize()
        res = (s.cpu().numpy(), p8.cpu().numpy())
        return res + (o,) if with_output else res

    # ---- workspace decoding -------------------------------------------------------------------
    def ws_host(self):
        torch.cuda.synchronize()
        return self.ws.cpu().numpy()

    def sequences(self):
        """[(q_len, kv_len)] per sequence."""
        if self.cu_cpu is None:
            return [(self.w.Nq, self.w.Nkv)] * self.w.B
        cq, ck = self.cu_cpu.numpy(), self.cu_kv_cpu.numpy()
        return [(int(cq[i + 1] - cq[i]), int(ck[i + 1] - ck[i])) for i in range(len(cq) - 1)]

    def decode(self, ws: np.ndarray, b: int):
        """Canonical pre-pass outputs of sequence b, shaped like the oracle's (the head dim's zero
        padding inside the workspace is checked and cut off)."""
        lay, w = self.lay, self.w
        dt, Hq, Hkv = w.d, w.Hq, w.Hkv
        d = 64 if dt <= 64 else 128  # head dim inside the workspace
        if self.cu_cpu is None:
            # no table without cu_seqlens: sequence b sits after b full sequences
            nqb_, kvpad_ = (w.Nq + 127) // 128, (w.Nkv + 127) // 128 * 128
            qs, lq, ks, lk = 0, w.Nq, 0, w.Nkv
            qrow0, kvrow0, qblk0 = b * nqb_ * 128, b * kvpad_, b * nqb_
            delta0 = b * sum(delta_row_keys(w.causal, w.Nq, w.Nkv))
        else:
            tab = ws[lay.seq_table:lay.seq_table + 4 * 8 * self.p.B].view(np.int32).reshape(-1, 8)
            qs, lq, ks, lk, qrow0, kvrow0, qblk0, delta0 = (int(x) for x in tab[b])
        nqb = (lq + 127) // 128
        kvpad = (lk + 127) // 128 * 128

        def arr(off, dtype, count):
            nbytes = count * np.dtype(dtype).itemsize
            return ws[off:off + nbytes].view(dtype)

        def unpack(raw):  # [..., 3d/4] u8 of packed e2m3 fields -> [..., d] int8 codes
            bits = np.unpackbits(raw, axis=-1, bitorder="little")
            f = bits.reshape(raw.shape[:-1] + (raw.shape[-1] * 8 // 6, 6))
            v = (f * (1 << np.arange(6))).sum(-1)
            table = {0: 0, 8: 1, 16: 2, 20: 3, 24: 4, 26: 5, 28: 6, 30: 7}
            mag = np.full(v.shape, 99, np.int8)
            for k_, m_ in table.items():
                mag[(v & 31) == k_] = m_
            assert not (mag == 99).any(), "field that is not an INT4 code in e2m3"
            out = np.where(v & 32, -mag, mag).astype(np.int8)
            assert not ((v == 32).any()), "negative zero code"
            return out

        out = {"table": (qs, lq, ks, lk, qrow0, kvrow0, qblk0, delta0)}
        out["kbar"] = arr(lay.kbar, np.float32, self.p.B * Hkv * d).reshape(self.p.B, Hkv, d)[b]
        out["sv"] = arr(lay.sv, np.float32, self.p.B * Hkv * d).reshape(self.p.B, Hkv, d)[b]
        qbar = arr(lay.qbar, np.float32, Hq * lay.q_blocks * d).reshape(Hq, lay.q_blocks, d)
        # stored in MFMA order within each 8-channel group: channel c at 4*(c%2) + (c%8)/2
        cc = np.arange(d)
        out["qbar"] = qbar[:, qblk0:qblk0 + nqb][:, :, (cc & ~7) | ((cc & 1) << 2) | ((cc >> 1) & 3)]
        qc = arr(lay.qcode, np.uint8, Hq * lay.q_rows * 3 * d // 4).reshape(Hq, lay.q_rows, 3 * d // 4)
        out["qcode"] = unpack(qc[:, qrow0:qrow0 + lq])
        out["qcode_pad"] = unpack(qc[:, qrow0 + lq:qrow0 + nqb * 128])
        sq = arr(lay.sq, np.float32, Hq * lay.q_rows).reshape(Hq, lay.q_rows)
        out["sq"] = sq[:, qrow0:qrow0 + lq]
        kc = arr(lay.kcode, np.uint8, Hkv * lay.kv_rows * 3 * d // 4).reshape(Hkv, lay.kv_rows, 3 * d // 4)
        out["kcode"] = unpack(kc[:, kvrow0:kvrow0 + lk])
        sk = arr(lay.sk, np.float32, Hkv * lay.kv_rows // 16).reshape(Hkv, lay.kv_rows // 16)
        out["sk"] = sk[:, kvrow0 // 16:kvrow0 // 16 + 2 * ((lk + 31) // 32)]
        v8 = arr(lay.v8, np.uint8, Hkv * lay.kv_rows * d).reshape(Hkv, lay.kv_rows // 64, d, 2, 32)
        v8 = v8[:, kvrow0 // 64:(kvrow0 + kvpad) // 64]
        canon = np.empty((Hkv, v8.shape[1] * 64, d), np.uint8)
        for h in range(2):
            for s in range(32):
                key = 32 * (s // 16) + 8 * ((s % 16) // 4) + 4 * h + s % 4
                canon[:, key::64, :] = v8[:, :, :, h, s]
        out["v8"] = canon[:, :lk]
        dl = arr(lay.delta, np.float32, Hq * lay.delta_len).reshape(Hq, lay.delta_len)
        # one row per Q block, back to back; keys past a row's stored range read as NaN
        full = np.full((Hq, nqb, kvpad), np.nan, np.float32)
        at = delta0
        for qb, n in enumerate(delta_row_keys(w.causal, lq, lk)):
            full[:, qb, :n] = dl[:, at:at + n]
            at += n
        out["delta"] = full[:, :, :lk]
        if dt < d:
            for name in ("kbar", "sv", "qbar", "qcode", "qcode_pad", "kcode", "v8"):
                pad = out[name][..., dt:]
                assert not pad.any(), f"{name}: head-dim padding channels are not zero"
                out[name] = np.ascontiguousarray(out[name][..., :dt])
        return out

    def seq_inputs(self, b: int, heads=None):
        """Head-major float32 inputs of sequence b for the oracle ([Hq, L, d], [Hkv, L, d]);
        `heads` = (first kv head, number of kv heads) limits them to a kv-head group range."""
        if self.cu_cpu is None:
            q, k, v = self.q_cpu[b], self.k_cpu[b], self.v_cpu[b]
        else:
            s, e = int(self.cu_cpu[b]), int(self.cu_cpu[b + 1])
            sk, ek = int(self.cu_kv_cpu[b]), int(self.cu_kv_cpu[b + 1])
            q, k, v = self.q_cpu[s:e], self.k_cpu[sk:ek], self.v_cpu[sk:ek]
        if heads is not None:
            g0, ng = heads
            grp = self.w.Hq // self.w.Hkv
            q = q[:, g0 * grp:(g0 + ng) * grp]
            k, v = k[:, g0:g0 + ng], v[:, g0:g0 + ng]
        f = lambda t: t.float().permute(1, 0, 2).contiguous().numpy()
        return f(q), f(k), f(v)

    def out_seq(self, b: int, o=None):
        """GPU output of sequence b as float64 [Hq, L, d] (of `o`, default the run's output)."""
        o = (self.o if o is None else o).float().cpu()
        if self.cu_cpu is None:
            o = o[b]
        else:
            o = o[int(self.cu_cpu[b]):int(self.cu_cpu[b + 1])]
        return o.permute(1, 0, 2).double().numpy()


def delta_row_keys(causal: bool, lq: int, lk: int) -> list:
    """Keys stored per Q block in the correction table of one sequence: all keys rounded up to 128
    without a causal mask; with one, the block's last visible key + 1 rounded up to 128."""
    kvpad = (lk + 127) // 128 * 128
    rows = []
    for qb in range((lq + 127) // 128):
        if not causal:
            rows.append(kvpad)
            continue
        last = min(lq, 128 * (qb + 1)) - 1 + (lk - lq)  # last visible key of the block
        rows.append(min(kvpad, max(0, (last + 1 + 127) // 128 * 128)))
    return rows


def half_ulp(ref: np.ndarray, dtype) -> np.ndarray:
    """Half a unit in the last place of `dtype` at |ref|: the rounding the output format itself
    adds to any correctly computed value."""
    if dtype == torch.float32:
        mant, emin = 23, -126
    elif dtype == torch.bfloat16:
        mant, emin = 7, -126
    else:
        mant, emin = 10, -14
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** emin)))
    return 0.5 * 2.0 ** (e - mant)


def cos(a, b) -> float:
    a, b = np.ravel(a).astype(np.float64), np.ravel(b).astype(np.float64)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


MAX_ABS_TOL = 1e-2   # output max-abs error against the oracle's quantized pipeline
COS_TOL = 0.9999     # cosine similarity against the oracle's quantized pipeline


def check_output(gpu: np.ndarray, ref: np.ndarray, allow: np.ndarray, dtype, what=""):
    """Element-wise |gpu - ref| <= 1e-2 + allowance for ambiguous FP8 roundings of P~ + half an
    ulp of the output format; cos >= 0.9999. Returns a dict of the measured figures."""
    err = np.abs(gpu - ref)
    base = MAX_ABS_TOL + half_ulp(ref, dtype)
    tol = base + allow
    bad = err > tol
    c = cos(gpu, ref)
    info = dict(max_abs=float(err.max()) if err.size else 0.0, cos=c,
                n_bad=int(bad.sum()), allow_max=float(allow.max()) if allow.size else 0.0,
                n_needed_allowance=int((err > base).sum()))
    assert not np.isnan(gpu).any(), f"{what}: NaN in GPU output"
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, worst {err.max():.3e} {info}"
    assert c >= COS_TOL, f"{what}: cos {c} < {COS_TOL}"
    return info
