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
//  - S^T = K Q^T on v_mfma_i32_32x32x32_i8. A lane owns one query (column) and, in each 32-key
//    subtile, the 16 keys whose index has bit 2 equal to its half-wave index. So one Q scale and one
//    K scale per lane and subtile dequantize all 16 accumulators: the per-thread scale groups.
//    INT4 codes are carried as 16*code in the i8 operands (a nibble mask unpacks them), so the
//    INT32 accumulator holds 256*S exactly.
//  - logits in base 2: x = S * (s_q * sm_scale * log2 e * s_k) + delta (one fused rounding).
//  - online softmax per 64-key tile: p = 2^(x - (m - log2 448)), so P~ = e4m3(p) uses the whole
//    FP8 range; the row max is reduced within the lane and across the two half-waves.
//  - O^T += V^T P~^T on v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x fp8, unit scales). The P~ operand
//    is the S^T accumulator itself after conversion; V is stored in the matching key order.
//    The fp8 MFMA's internal accumulation is not exact FP32 on gfx950 (measured error up to about
//    2^-11 of the largest product's binade per instruction), so each tile's product is formed from
//    zero and folded into the FP32 output registers: O = alpha*O + inner (two-level accumulation).
//  - epilogue: O * s_v / l, rounded to the output dtype.
#include "device_common.h"

namespace sage2 {
namespace {

constexpr float kLog2_448 = 8.80735492205760410750f;

// 8 packed bytes (16 INT4 codes, channel 2i in the low nibble of byte i) -> MFMA i8 operand holding
// 16*code. Q and K use the same routine, so their slot orders agree.
__device__ inline v4i unpack16(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(w0 & 0xF0F0F0F0u);
  r[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(w1 & 0xF0F0F0F0u);
  return r;
}

// Loads this lane-half's D/4 packed bytes of one code row and unpacks them into D/32 operands.
template <int D>
__device__ inline void load_codes(const uint8_t* row, int hh, v4i (&op)[D / 32]) {
  const uint4* src = reinterpret_cast<const uint4*>(row + hh * (D / 4));
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    const uint4 w = src[u];
    op[2 * u] = unpack16(w.x, w.y);
    op[2 * u + 1] = unpack16(w.z, w.w);
  }
}

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

// One workgroup = one (sequence, q head, 128-query block); 4 waves x 32 queries.
// Causal grids run the longest blocks (highest qb) first.
template <int D, int CAUSAL, int OUT>
__global__ __launch_bounds__(256) void k_attn(KArgs a) {
  constexpr int NCH = D / 32;
  const int qb = gridDim.x - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  const Seq s = load_seq(a, b);
  if (qb * kQBlock >= s.q_len) return;
  const int g = h / (a.Hq / a.Hkv);
  const int i = qb * kQBlock + 32 * wave + n;  // this lane's query row within the sequence
  const int64_t prow = (int64_t)h * a.lay.q_rows + s.q_row0 + i;
  const int kvpad = (s.kv_len + kKVPad - 1) / kKVPad * kKVPad;

  v4i qop[NCH];
  load_codes<D>(ws_ptr<uint8_t>(a, a.lay.qcode) + prow * (D / 2), hh, qop);
  // (s_q * L) * 2^-8: the 2^-8 undoes the 16*16 carried by the two operands (exact).
  const float cq = (ws_ptr<float>(a, a.lay.sq)[prow] * a.L) * 0.00390625f;

  int ntile = (s.kv_len + kKVTile - 1) / kKVTile;
  const int koff = s.kv_len - s.q_len;
  if (CAUSAL) {
    const int kmax = min(s.q_len, qb * kQBlock + 32 * wave + 32) - 1 + koff;
    ntile = kmax < 0 ? 0 : min(ntile, kmax / kKVTile + 1);
  }
  const uint8_t* kcode = ws_ptr<uint8_t>(a, a.lay.kcode) + ((int64_t)g * a.lay.kv_rows + s.kv_row0) * (D / 2);
  const float* skp = ws_ptr<float>(a, a.lay.sk) + (int64_t)g * (a.lay.kv_rows / 16) + s.kv_row0 / 16;
  const uint8_t* v8 = ws_ptr<uint8_t>(a, a.lay.v8) + ((int64_t)g * a.lay.kv_rows + s.kv_row0) * D;
  const float* drow = ws_ptr<float>(a, a.lay.delta) + (int64_t)h * a.lay.delta_len + s.delta0 +
                      (int64_t)qb * kvpad;

  float m = kNegInf, lsum = 0.0f;
  v16f o[NCH];
#pragma unroll
  for (int cb = 0; cb < NCH; ++cb) o[cb] = v16f{};

  for (int t = 0; t < ntile; ++t) {
    float x[32];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key0 = t * kKVTile + 32 * st;
      v4i kop[NCH];
      load_codes<D>(kcode + (int64_t)(key0 + n) * (D / 2), hh, kop);
      v16i acc = v16i{};
#pragma unroll
      for (int cb = 0; cb < NCH; ++cb) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[cb], qop[cb], acc, 0, 0, 0);
      const float cs = cq * skp[2 * (key0 / 32) + hh];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 dl = *reinterpret_cast<const float4*>(drow + key0 + 8 * a4 + 4 * hh);
        const float dv[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * a4 + e;
          const int key = key0 + 8 * a4 + 4 * hh + e;
          const float xv = __builtin_fmaf((float)acc[r], cs, dv[e]);
          const bool vis = key < s.kv_len && (!CAUSAL || key <= i + koff);
          x[16 * st + r] = vis ? xv : kNegInf;
        }
      }
    }
    float mt = x[0];
#pragma unroll
    for (int k = 1; k < 32; ++k) mt = fmaxf(mt, x[k]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mnew = fmaxf(m, mt);
    const float alpha = (m == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m - mnew);
    const float mb = (mnew == kNegInf) ? 0.0f : mnew - kLog2_448;
    float p[32];
    float ps = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      p[k] = __builtin_amdgcn_exp2f(x[k] - mb);
      ps += p[k];
    }
    lsum = alpha * lsum + ps;
    v8i pop;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int w = cvt_fp8x2(p[4 * q], p[4 * q + 1], 0, false);
      pop[q] = cvt_fp8x2(p[4 * q + 2], p[4 * q + 3], w, true);
    }
    const uint8_t* vt = v8 + (int64_t)t * kKVTile * D;
#pragma unroll
    for (int cb = 0; cb < NCH; ++cb) {
      const uint4* src = reinterpret_cast<const uint4*>(vt + ((32 * cb + n) * 2 + hh) * 32);
      const uint4 v0 = src[0], v1 = src[1];
      const v8i vop = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      const v16f inner = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop, v16f{}, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][r] = __builtin_fmaf(alpha, o[cb][r], inner[r]);
    }
    m = mnew;
  }

  lsum += __shfl_xor(lsum, 32, 64);
  if (i >= s.q_len) return;
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  const float* svp = ws_ptr<float>(a, a.lay.sv) + ((int64_t)b * a.Hkv + g) * D;
  constexpr int ES = OUT == SAGE2_F32 ? 4 : 2;
  char* orow = reinterpret_cast<char*>(a.o) + ES * row_index(a.os, b, s.q_start + i, h);
#pragma unroll
  for (int cb = 0; cb < NCH; ++cb) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int c0 = 32 * cb + 8 * a4 + 4 * hh;
      const float4 sv = *reinterpret_cast<const float4*>(svp + c0);
      store4<OUT>(orow + ES * c0, o[cb][4 * a4] * sv.x * inv, o[cb][4 * a4 + 1] * sv.y * inv,
                  o[cb][4 * a4 + 2] * sv.z * inv, o[cb][4 * a4 + 3] * sv.w * inv);
    }
  }
}

// Test-only: the same INT4 MFMA path, dumping S = acc / 256 for rows [dbg_q0, dbg_q0 + dbg_qn).
template <int D>
__global__ __launch_bounds__(256) void k_debug_qk(KArgs a) {
  constexpr int NCH = D / 32;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
  if (qb * kQBlock + kQBlock <= a.dbg_q0 || qb * kQBlock >= a.dbg_q0 + a.dbg_qn) return;
  const Seq s = load_seq(a, b);
  const bool blk_ok = qb * kQBlock < s.q_len;
  const int g = h / (a.Hq / a.Hkv);
  const int i = qb * kQBlock + 32 * wave + n;
  const bool row_out = i >= a.dbg_q0 && i < a.dbg_q0 + a.dbg_qn;
  const int kvpad = (s.kv_len + kKVPad - 1) / kKVPad * kKVPad;
  v4i qop[NCH];
  if (blk_ok) {
    load_codes<D>(ws_ptr<uint8_t>(a, a.lay.qcode) + ((int64_t)h * a.lay.q_rows + s.q_row0 + i) * (D / 2), hh, qop);
  } else {
#pragma unroll
    for (int cb = 0; cb < NCH; ++cb) qop[cb] = v4i{};
  }
  const uint8_t* kcode = ws_ptr<uint8_t>(a, a.lay.kcode) + ((int64_t)g * a.lay.kv_rows + s.kv_row0) * (D / 2);
  int32_t* out = a.dbg_out + (((int64_t)b * a.Hq + h) * a.dbg_qn + (i - a.dbg_q0)) * a.Nkv;
  const int nt = (a.Nkv + kKVTile - 1) / kKVTile;
  for (int t = 0; t < nt; ++t) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key0 = t * kKVTile + 32 * st;
      v16i acc = v16i{};
      if (blk_ok && key0 < kvpad) {
        v4i kop[NCH];
        load_codes<D>(kcode + (int64_t)(key0 + n) * (D / 2), hh, kop);
#pragma unroll
        for (int cb = 0; cb < NCH; ++cb) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[cb], qop[cb], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row_out && key < a.Nkv) out[key] = (i < s.q_len && key < s.kv_len) ? (acc[r] >> 8) : 0;
      }
    }
  }
}

template <int D, int CAUSAL>
int launch_attn_d(const KArgs& a, hipStream_t st) {
  const dim3 grid((a.Nq + kQBlock - 1) / kQBlock, a.Hq, a.B);
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
