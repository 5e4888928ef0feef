// SageAttention2 attention kernel for gfx950 (CDNA4, wave64).
//
// Sources: PMLR vol. 267 page "SageAttention2: Efficient Attention with Thorough Outlier Smoothing
// and Per-thread INT4 Quantization", Abstract (INT4 QK^T, FP8 P~V, two-level accumulation of P~V);
// research record of the same title, "Three components" (per-thread scales kept in registers; FP8
// PV accumulation loses accuracy, recovered by two levels); visual companion "SageAttention2 and
// Fast Exact INT4 Attention", "Numerical Repair Stack" (exact INT4 fragments, FP8 value mixing,
// periodic FP32 foldback) and "Per-Thread INT4 Geometry" (scale groups follow thread ownership).
//
// gfx950 form of the method:
//  - S^T = K Q^T on the 32x32 MFMA. A lane owns one query (column) and, in each 32-key subtile,
//    the 16 keys whose index has bit 2 equal to its half-wave index. So one Q scale and one K scale
//    per lane and subtile dequantize all 16 accumulators: the per-thread scale groups.
//    gfx950 has no INT4 MFMA. The INT4 codes ride in 6-bit e2m3 fields, in which every integer in
//    [-7, 7] is exact, on v_mfma_scale_f32_32x32x64_f8f6f4 (fp6 x fp6, unit scales): the products
//    are small integers and the f32 accumulation of them is exact (|S| <= 49 d), so the accumulator
//    holds the INT32 product S exactly, at twice the K depth per instruction of the i8 MFMA and
//    with no integer-to-float conversion.
//  - logits in base 2: x = S * (s_q * sm_scale * log2 e * s_k) + delta (one fused rounding).
//  - online softmax per 128-key tile: p = 2^(x - (m - log2 448)), so P~ = e4m3(p) uses the whole
//    FP8 range; the row max is reduced within the lane and across the two half-waves.
//  - O^T += V^T P~^T on v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x fp8, unit scales). The P~ operand
//    is the S^T accumulator itself after conversion; V is stored in the matching key order.
//    The fp8 MFMA's internal accumulation is not exact FP32 on gfx950 (measured error up to about
//    2^-11 of the largest product's binade per instruction), so each tile's product is formed from
//    zero, accumulated in the MFMA over the tile's two 64-key halves, and folded into the FP32
//    output registers: O = alpha*O + inner (two-level accumulation).
//  - epilogue: O * s_v / l, rounded to the output dtype.
#include "device_common.h"

namespace sage2 {
namespace {

constexpr float kLog2_448 = 8.80735492205760410750f;

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int OUT>
__device__ inline void store4(char* dst, float a, float b, float c, float d) {
  if constexpr (OUT == SAGE2_F32) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
  } else if constexpr (OUT == SAGE2_BF16) {
    const uint32_t lo = f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
    const uint32_t hi = f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  } else {
    _Float16 h[4] = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    uint2 w;
    __builtin_memcpy(&w, h, 8);
    *reinterpret_cast<uint2*>(dst) = w;
  }
}

// Workgroup -> (q head, 128-query block) of one sequence. Work is ordered longest causal block
// first, and within a block index the q heads that share a kv head are consecutive; dispatches go
// round-robin over the 8 XCDs, so each run of `grp` consecutive work items is placed on one XCD
// (its q heads then read the same K/V through that XCD's L2).
__device__ inline void decode_work(int L, int nqb, int Hq, int grp, int* qb, int* h) {
  const int total = nqb * Hq;
  const int round = 8 * grp;
  int w = L;
  if (L < total / round * round) w = (L / round) * round + (L % 8) * grp + (L / 8) % grp;
  *qb = nqb - 1 - w / Hq;
  *h = w % Hq;
}

constexpr int kBN = 128;  // keys per tile of the online softmax

// LDS staging of one 128-key tile: K as packed e2m3 code rows (8-byte padded: conflict-free 8-byte
// reads), V as two 64-key tiles in their layout with padded channel rows, the tile's 128
// correction values and its 8 K group scales.
template <int D>
struct Stage {
  static constexpr int CB = 3 * D / 4;                  // bytes of one packed code row
  static constexpr int KROW = CB + 8;
  static constexpr int VCH = 80;                        // bytes per V channel (64 keys + padding)
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = (kBN * KROW + 15) / 16 * 16;
  static constexpr int VHALF = D * VCH;
  static constexpr int D_OFF = V_OFF + 2 * VHALF;
  static constexpr int S_OFF = D_OFF + kBN * 4;
  static constexpr int BYTES = S_OFF + 32;
  static constexpr int K_BYTES = kBN * CB / 256;        // staged per thread
  static constexpr int V_BYTES = 2 * 64 * D / 256;
};

template <int D>
struct TileK {  // K codes, correction values and group scales of one tile
  uint2 k[Stage<D>::K_BYTES / 8];
  uint4 dl;
};
template <int D>
struct TileV {  // V codes of one tile
  uint4 v[Stage<D>::V_BYTES / 16];
};

template <int D>
__device__ inline void load_k(TileK<D>& r, int tid, int t, const uint8_t* kcode, const float* drow,
                              const float* skp) {
  using S = Stage<D>;
  const uint2* ks = reinterpret_cast<const uint2*>(kcode + (int64_t)t * kBN * S::CB + tid * S::K_BYTES);
#pragma unroll
  for (int u = 0; u < S::K_BYTES / 8; ++u) r.k[u] = ks[u];
  if (tid < 32) r.dl = *reinterpret_cast<const uint4*>(drow + t * kBN + tid * 4);
  else if (tid < 34) r.dl = *reinterpret_cast<const uint4*>(skp + 8 * t + 4 * (tid - 32));
}

template <int D>
__device__ inline void store_k(const TileK<D>& r, int tid, uint8_t* st) {
  using S = Stage<D>;
  const int ko = tid * S::K_BYTES;  // K_BYTES divides CB: a thread's bytes stay in one row
  uint2* kd = reinterpret_cast<uint2*>(st + S::K_OFF + (ko / S::CB) * S::KROW + ko % S::CB);
#pragma unroll
  for (int u = 0; u < S::K_BYTES / 8; ++u) kd[u] = r.k[u];
  if (tid < 32) *reinterpret_cast<uint4*>(st + S::D_OFF + tid * 16) = r.dl;
  else if (tid < 34) *reinterpret_cast<uint4*>(st + S::S_OFF + (tid - 32) * 16) = r.dl;
}

template <int D>
__device__ inline void load_v(TileV<D>& r, int tid, int t, const uint8_t* v8) {
  using S = Stage<D>;
  const uint4* vs = reinterpret_cast<const uint4*>(v8 + (int64_t)t * kBN * D + tid * S::V_BYTES);
#pragma unroll
  for (int u = 0; u < S::V_BYTES / 16; ++u) r.v[u] = vs[u];
}

template <int D>
__device__ inline void store_v(const TileV<D>& r, int tid, uint8_t* st) {
  using S = Stage<D>;
  const int vo = tid * S::V_BYTES;  // V_BYTES divides 64: a thread's bytes stay in one channel row
  const int vhalf = vo / (64 * D), vr = vo % (64 * D);
  uint4* vd = reinterpret_cast<uint4*>(st + S::V_OFF + vhalf * S::VHALF + (vr / 64) * S::VCH + vr % 64);
#pragma unroll
  for (int u = 0; u < S::V_BYTES / 16; ++u) vd[u] = r.v[u];
}

// One fp6 MFMA operand: 32 e2m3 fields (24 bytes) read as three 8-byte words.
__device__ inline v8i load_fp6_op(const uint8_t* p) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  const uint2 b = *reinterpret_cast<const uint2*>(p + 8);
  const uint2 c = *reinterpret_cast<const uint2*>(p + 16);
  return v8i{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
}

__device__ inline v16f mfma_fp6(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, 0, 0, 0);
}

__device__ inline v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One workgroup = one (sequence, q head, 128-query block); 4 waves x 32 queries. K/V tiles of 128
// keys are staged once per workgroup in LDS (double-buffered, next tile's global loads in flight
// while the current tile is computed).
template <int D, int CAUSAL, int OUT>
__global__ __launch_bounds__(256, 2) void k_attn(KArgs a) {
  constexpr int NC6 = D / 64;   // fp6 MFMAs per 32-key subtile (64 channels each)
  constexpr int NCB = D / 32;   // 32-channel blocks of the output
  using S = Stage<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::BYTES];

  const int b = blockIdx.y;
  const int nqb_grid = (a.Nq + kQBlock - 1) / kQBlock;
  int qb, h;
  decode_work(blockIdx.x, nqb_grid, a.Hq, a.Hq / a.Hkv, &qb, &h);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const Seq s = load_seq(a, b);
  if (qb * kQBlock >= s.q_len) return;
  const int g = h / (a.Hq / a.Hkv);
  const int i = qb * kQBlock + 32 * wave + n;  // this lane's query row within the sequence
  const int64_t prow = (int64_t)h * a.lay.q_rows + s.q_row0 + i;
  const int kvpad = (s.kv_len + kKVPad - 1) / kKVPad * kKVPad;
  const int koff = s.kv_len - s.q_len;

  v8i qop[NC6];
  {
    const uint8_t* qrow = ws_ptr<uint8_t>(a, a.lay.qcode) + prow * S::CB + hh * (S::CB / 2);
#pragma unroll
    for (int cb = 0; cb < NC6; ++cb) qop[cb] = load_fp6_op(qrow + 24 * cb);
  }
  const float cq = ws_ptr<float>(a, a.lay.sq)[prow] * a.L;

  // tiles for the workgroup (all waves stage) and for this wave (causal: up to its last row)
  int nt = (s.kv_len + kBN - 1) / kBN;
  int nt_w = nt;
  const int wave_row0 = qb * kQBlock + 32 * wave;
  if (CAUSAL) {
    const int kmax = min(s.q_len, qb * kQBlock + kQBlock) - 1 + koff;
    nt = kmax < 0 ? 0 : min(nt, kmax / kBN + 1);
    const int kmax_w = min(s.q_len, wave_row0 + 32) - 1 + koff;
    nt_w = kmax_w < 0 ? 0 : min(nt_w, kmax_w / kBN + 1);
  }
  const uint8_t* kcode = ws_ptr<uint8_t>(a, a.lay.kcode) + ((int64_t)g * a.lay.kv_rows + s.kv_row0) * S::CB;
  const float* skp = ws_ptr<float>(a, a.lay.sk) + (int64_t)g * (a.lay.kv_rows / 16) + s.kv_row0 / 16;
  const uint8_t* v8 = ws_ptr<uint8_t>(a, a.lay.v8) + ((int64_t)g * a.lay.kv_rows + s.kv_row0) * D;
  const float* drow = ws_ptr<float>(a, a.lay.delta) + (int64_t)h * a.lay.delta_len + s.delta0 +
                      (int64_t)qb * kvpad;

  float m = kNegInf, lsum = 0.0f;
  v16f o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = v16f{};

  TileK<D> tk;
  TileV<D> tv;
  if (nt > 0) {
    load_k<D>(tk, tid, 0, kcode, drow, skp);
    load_v<D>(tv, tid, 0, v8);
    store_k<D>(tk, tid, smem);
    store_v<D>(tv, tid, smem);
  }
  __syncthreads();

#pragma unroll 1
  for (int t = 0; t < nt; ++t) {
    uint8_t* st = smem + (t & 1) * S::BYTES;
    const bool more = t + 1 < nt;
    uint8_t* nxt = smem + ((t + 1) & 1) * S::BYTES;  // last read before the previous barrier
    // next tile's K part: loads issued now, written to LDS after this tile's QK^T products
    if (more) load_k<D>(tk, tid, t + 1, kcode, drow, skp);
    if (t < nt_w) {
      // the wave needs masking only on a ragged last tile or where the causal edge crosses
      const bool need_mask = (t * kBN + kBN > s.kv_len) ||
                             (CAUSAL && t * kBN + kBN - 1 > wave_row0 + koff);
      const float* sks = reinterpret_cast<const float*>(st + S::S_OFF);
      float x[64];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const uint8_t* krow = st + S::K_OFF + (32 * sub + n) * S::KROW + hh * (S::CB / 2);
        v16f acc = v16f{};
#pragma unroll
        for (int cb = 0; cb < NC6; ++cb) acc = mfma_fp6(load_fp6_op(krow + 24 * cb), qop[cb], acc);
        __builtin_amdgcn_sched_barrier(0);
        const float cs = cq * sks[2 * sub + hh];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const float4 dl = *reinterpret_cast<const float4*>(st + S::D_OFF + (32 * sub + 8 * a4 + 4 * hh) * 4);
          const float dv[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) x[16 * sub + 4 * a4 + e] = __builtin_fmaf(acc[4 * a4 + e], cs, dv[e]);
        }
      }
      if (more) store_k<D>(tk, tid, nxt);
      if (need_mask) {
#pragma unroll
        for (int k = 0; k < 64; ++k) {
          const int key = t * kBN + 32 * (k >> 4) + 8 * ((k & 15) >> 2) + 4 * hh + (k & 3);
          const bool vis = key < s.kv_len && (!CAUSAL || key <= i + koff);
          x[k] = vis ? x[k] : kNegInf;
        }
      }
      float mt = x[0];
#pragma unroll
      for (int k = 1; k < 64; ++k) mt = fmaxf(mt, x[k]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mnew = fmaxf(m, mt);
      const float alpha = (m == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m - mnew);
      const float mb = (mnew == kNegInf) ? 0.0f : mnew - kLog2_448;
      float ps = 0.0f;
#pragma unroll
      for (int k = 0; k < 64; ++k) {
        x[k] = __builtin_amdgcn_exp2f(x[k] - mb);
        ps += x[k];
      }
      lsum = alpha * lsum + ps;
      v8i pop[2];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int w = cvt_fp8x2(x[4 * q], x[4 * q + 1], 0, false);
        pop[q >> 3][q & 7] = cvt_fp8x2(x[4 * q + 2], x[4 * q + 3], w, true);
      }
      // next tile's V part: loads land during the PV products
      if (more) load_v<D>(tv, tid, t + 1, v8);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        v16f inner = v16f{};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint8_t* vrow = st + S::V_OFF + half * S::VHALF + (32 * cb + n) * S::VCH + hh * 32;
          const uint4 v0 = *reinterpret_cast<const uint4*>(vrow);
          const uint4 v1 = *reinterpret_cast<const uint4*>(vrow + 16);
          const v8i vop = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
          inner = mfma_fp8(vop, pop[half], inner);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] = __builtin_fmaf(alpha, o[cb][r], inner[r]);
        // one channel block at a time: keeps the V operands and partial products of the other
        // blocks out of registers
        __builtin_amdgcn_sched_barrier(0);
      }
      m = mnew;
      if (more) store_v<D>(tv, tid, nxt);
    } else if (more) {
      store_k<D>(tk, tid, nxt);
      load_v<D>(tv, tid, t + 1, v8);
      store_v<D>(tv, tid, nxt);
    }
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 32, 64);
  if (i >= s.q_len) return;
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  const float* svp = ws_ptr<float>(a, a.lay.sv) + ((int64_t)b * a.Hkv + g) * D;
  constexpr int ES = OUT == SAGE2_F32 ? 4 : 2;
  char* orow = reinterpret_cast<char*>(a.o) + ES * row_index(a.os, b, s.q_start + i, h);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int c0 = 32 * cb + 8 * a4 + 4 * hh;
      const float4 sv = *reinterpret_cast<const float4*>(svp + c0);
      store4<OUT>(orow + ES * c0, o[cb][4 * a4] * sv.x * inv, o[cb][4 * a4 + 1] * sv.y * inv,
                  o[cb][4 * a4 + 2] * sv.z * inv, o[cb][4 * a4 + 3] * sv.w * inv);
    }
  }
}

// Test-only: the same fp6 MFMA path, dumping S for rows [dbg_q0, dbg_q0 + dbg_qn).
template <int D>
__global__ __launch_bounds__(256) void k_debug_qk(KArgs a) {
  constexpr int NC6 = D / 64;
  constexpr int CB = 3 * D / 4;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  if (qb * kQBlock + kQBlock <= a.dbg_q0 || qb * kQBlock >= a.dbg_q0 + a.dbg_qn) return;
  const Seq s = load_seq(a, b);
  const bool blk_ok = qb * kQBlock < s.q_len;
  const int g = h / (a.Hq / a.Hkv);
  const int i = qb * kQBlock + 32 * wave + n;
  const bool row_out = i >= a.dbg_q0 && i < a.dbg_q0 + a.dbg_qn;
  const int kvpad = (s.kv_len + kKVPad - 1) / kKVPad * kKVPad;
  v8i qop[NC6];
#pragma unroll
  for (int cb = 0; cb < NC6; ++cb) qop[cb] = v8i{};
  if (blk_ok) {
    const uint8_t* qrow = ws_ptr<uint8_t>(a, a.lay.qcode) + ((int64_t)h * a.lay.q_rows + s.q_row0 + i) * CB + hh * (CB / 2);
#pragma unroll
    for (int cb = 0; cb < NC6; ++cb) qop[cb] = load_fp6_op(qrow + 24 * cb);
  }
  const uint8_t* kcode = ws_ptr<uint8_t>(a, a.lay.kcode) + ((int64_t)g * a.lay.kv_rows + s.kv_row0) * CB;
  int32_t* out = a.dbg_out + (((int64_t)b * a.Hq + h) * a.dbg_qn + (i - a.dbg_q0)) * a.Nkv;
  const int nsub = (a.Nkv + 31) / 32;
  for (int sub = 0; sub < nsub; ++sub) {
    const int key0 = 32 * sub;
    v16f acc = v16f{};
    if (blk_ok && key0 < kvpad) {
      const uint8_t* krow = kcode + (int64_t)(key0 + n) * CB + hh * (CB / 2);
#pragma unroll
      for (int cb = 0; cb < NC6; ++cb) acc = mfma_fp6(load_fp6_op(krow + 24 * cb), qop[cb], acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (row_out && key < a.Nkv) out[key] = (i < s.q_len && key < s.kv_len) ? (int32_t)acc[r] : 0;
    }
  }
}

template <int D, int CAUSAL>
int launch_attn_d(const KArgs& a, hipStream_t st) {
  const dim3 grid((a.Nq + kQBlock - 1) / kQBlock * a.Hq, a.B);
  switch (a.out_dtype) {
    case SAGE2_F32: k_attn<D, CAUSAL, SAGE2_F32><<<grid, 256, 0, st>>>(a); break;
    case SAGE2_BF16: k_attn<D, CAUSAL, SAGE2_BF16><<<grid, 256, 0, st>>>(a); break;
    default: k_attn<D, CAUSAL, SAGE2_F16><<<grid, 256, 0, st>>>(a); break;
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_attn(const KArgs& a, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.d == 64) return a.causal ? launch_attn_d<64, 1>(a, st) : launch_attn_d<64, 0>(a, st);
  return a.causal ? launch_attn_d<128, 1>(a, st) : launch_attn_d<128, 0>(a, st);
}

int launch_debug_qk(const KArgs& a, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 grid((a.Nq + kQBlock - 1) / kQBlock, a.Hq, a.B);
  if (a.d == 64) k_debug_qk<64><<<grid, 256, 0, st>>>(a);
  else k_debug_qk<128><<<grid, 256, 0, st>>>(a);
  return (int)hipGetLastError();
}

}  // namespace sage2
