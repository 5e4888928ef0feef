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
//    output registers (two-level accumulation). The FP32 buffer is kept in a fixed reference
//    frame, o = O * 2^(ref - mb): the fold is o += 2^(mb - ref) * inner (an in-place fused
//    multiply-add, the same as rescaling O by alpha = 2^(m_prev - m) up to f32 rounding), and o, l
//    are renormalized only when that factor would pass 2^64. The frame cancels in O = o / l.
//  - epilogue: O * s_v / l, rounded to the output dtype.
#include "device_common.h"

namespace sage2 {
namespace {

constexpr float kLog2_448 = 8.80735492205760410750f;
// largest fold factor exponent before the running output is renormalized: o and l then stay below
// 2^(64 + 27) for any sequence the ABI accepts
constexpr float kFrameLimit = 64.0f;
// start (and floor) of the running row max: a row with no visible key yet keeps this finite max
// (its p are exact zeros), and the output frame starts at its frame, so the first tile with a visible
// key always takes the renormalization (o and l are still zero then); for the single-level ablation
// its alpha 2^(m_prev - m) is 0 there. Logits below -2^100 are outside the supported range.
constexpr float kMaxFloor = -0x1p100f;

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// v_max3_f32 written out. Through fmaxf the compiler quiets every operand that it cannot prove to be
// the result of arithmetic (here the two permlane results): one extra instruction each on the
// softmax's critical path. (Not used for the long in-lane chain: after each inline asm the compiler
// adds a wait state.)
__device__ inline float max3(float a, float b, float c) {
  float y;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(y) : "v"(a), "v"(b), "v"(c));
  return y;
}

// max over lanes l and l ^ 32 (the two half-waves hold the two key halves of a query's row):
// v_permlane32_swap exchanges the half-waves, and whichever of its two results holds the other
// half's value, the max over both and the lane's own value is the pair max
__device__ inline float half_wave_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(x, __uint_as_float(r[0]), __uint_as_float(r[1]));
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

// LDS staging of one 128-key tile, filled by global->LDS DMA (global_load_lds_dwordx4: lane i of
// an instruction writes 16 bytes at base + 16 i, from any global address). Each region is a
// permutation of 16-byte blocks chosen so that the compute reads hit distinct banks:
//  - K: 128 packed e2m3 rows of R = 3D/64 blocks. For D = 128 the two 3-block halves of a row swap
//    places every 8 keys (block j of key k at 6k + ((j + 3*((k>>3)&1)) mod 6)), so 16 lanes reading
//    one block each of 16 consecutive keys land on 16 different 16-byte bank groups; for D = 64
//    rows of 3 blocks already do.
//  - V: two 64-key tiles, D channels x 4 blocks (the layout of the workspace's v8 tiles), block j
//    of channel c at 4c + (j ^ ((c>>2)&3)).
//  - the tile's 128 correction values and its 8 K group scales, contiguous, in a 1 KB region
//    written by one full-wave DMA (lanes past the 34 that carry data refetch correction values).
template <int D>
struct Stage {
  static constexpr int CB = 3 * D / 4;         // bytes of one packed code row
  static constexpr int R = CB / 16;            // 16-byte blocks per code row
  static constexpr int KB = kBN * R;           // K blocks
  static constexpr int VB = 2 * D * 4;         // V blocks
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KB * 16;
  static constexpr int D_OFF = V_OFF + VB * 16;
  static constexpr int S_OFF = D_OFF + kBN * 4;
  static constexpr int BYTES = D_OFF + 1024;
  static constexpr int K_INSTR = KB / 64;      // DMA instructions per region (64 blocks each)
  static constexpr int V_INSTR = VB / 64;
};

// LDS block of K (key k, row block j)
template <int D>
__device__ inline int k_block(int k, int j) {
  if constexpr (Stage<D>::R == 6) return 6 * k + (j + 3 * ((k >> 3) & 1)) % 6;
  else return Stage<D>::R * k + j;
}
// LDS block of V (64-key half h2, channel c, block j)
template <int D>
__device__ inline int v_block(int h2, int c, int j) {
  return h2 * (4 * D) + 4 * c + (j ^ ((c >> 2) & 3));
}

// Per-lane byte offsets (relative to a tile's global base) of the blocks this lane fetches.
template <int D>
struct DmaPlan {
  uint32_t k[(Stage<D>::K_INSTR + 3) / 4];
  uint32_t v[(Stage<D>::V_INSTR + 3) / 4];
};

template <int D>
__device__ inline DmaPlan<D> make_dma_plan(int wave, int lane) {
  using S = Stage<D>;
  DmaPlan<D> pl;
#pragma unroll
  for (int u = 0; u < (S::K_INSTR + 3) / 4; ++u) {
    const int p = (wave + 4 * u) * 64 + lane;   // LDS block written by this lane
    int k = p / S::R, jj = p % S::R, j = jj;
    if constexpr (S::R == 6) j = (jj + 6 - 3 * ((k >> 3) & 1)) % 6;
    pl.k[u] = k * S::CB + 16 * j;
  }
#pragma unroll
  for (int u = 0; u < (S::V_INSTR + 3) / 4; ++u) {
    const int p = (wave + 4 * u) * 64 + lane;
    const int h2 = p / (4 * D), r = p % (4 * D), c = r / 4, j = (r % 4) ^ ((c >> 2) & 3);
    pl.v[u] = h2 * (64 * D) + c * 64 + 16 * j;
  }
  return pl;
}

// 16-byte global->LDS DMA through a buffer descriptor over one tile: the tile's base sits in scalar
// registers and the lane's byte offset in one loop-invariant VGPR, so issuing it needs no vector
// address arithmetic. 0x00020000 is the gfx9-family descriptor word 3 (32-bit data format, no
// swizzle); offsets are checked against `bytes` (out of range reads return zero).
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, off, 0, 0, 0);
}

// Issues the DMA of tile t into stage `st` (every wave its share).
template <int D>
__device__ inline void issue_tile(const DmaPlan<D>& pl, int wave, int lane, int t, uint8_t* st,
                                  const uint8_t* kcode, const uint8_t* v8, const float* drow,
                                  const float* skp) {
  using S = Stage<D>;
  const auto kr = tile_rsrc(kcode + (int64_t)t * kBN * S::CB, kBN * S::CB);
  const auto vr = tile_rsrc(v8 + (int64_t)t * kBN * D, kBN * D);
#pragma unroll
  for (int u = 0; u < (S::K_INSTR + 3) / 4; ++u)
    if (wave + 4 * u < S::K_INSTR) dma16(kr, pl.k[u], st + S::K_OFF + (wave + 4 * u) * 1024);
#pragma unroll
  for (int u = 0; u < (S::V_INSTR + 3) / 4; ++u)
    if (wave + 4 * u < S::V_INSTR) dma16(vr, pl.v[u], st + S::V_OFF + (wave + 4 * u) * 1024);
  if (wave == 0) {
    // one select of two in-bounds addresses (no divergent branch around the DMA)
    const float* dsrc = drow + t * kBN + 4 * (lane & 31);
    const float* ssrc = skp + 8 * t + 4 * (lane & 1);
    __builtin_amdgcn_global_load_lds((unsigned)(lane - 32) < 2u ? ssrc : dsrc,
                                     (__attribute__((address_space(3))) void*)(st + S::D_OFF), 16, 0, 0);
  }
}

__device__ inline void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
// NOFOLD = 1 is the ablation without the two-level accumulation: the output accumulates across
// tiles inside the FP8 MFMA (rescaled by alpha in registers each tile), which on gfx950 adds its C
// input with less than FP32 precision.
// DUMP = 1 (tests only) also writes, for the rows of KArgs::dbg_*, the INT32 S of every key tile the
// wave computes (from the same LDS-staged operands and MFMAs) and the e4m3 P~ codes it feeds to the
// P~V MFMA; with a.o null it writes no output.
template <int D, int CAUSAL, int OUT, int NOFOLD, int DUMP = 0>
__global__ __launch_bounds__(256, 2) void k_attn(KArgs a) {
  constexpr int NC6 = D / 64;   // fp6 MFMAs per 32-key subtile (64 channels each)
  constexpr int NCB = D / 32;   // 32-channel blocks of the output
  using S = Stage<D>;
  // two separate stage arrays (not one array with offsets): the compiler then knows that the DMA
  // filling one stage never aliases the LDS reads of the other, and does not wait on it early
  __shared__ __attribute__((aligned(16))) uint8_t stage0[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[S::BYTES];

  const int b = blockIdx.y;
  const int nqb_grid = (a.Nq + kQBlock - 1) / kQBlock;
  int qb, h;
  decode_work(blockIdx.x, nqb_grid, a.Hq, a.Hq / a.Hkv, &qb, &h);
  // the wave index in an SGPR: the DMA share of each wave is then decided by scalar code
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63,
            n = lane & 31, hh = lane >> 5;
  __builtin_assume(wave >= 0 && wave < 4);
  const Seq s = load_seq(a, b);
  if (qb * kQBlock >= s.q_len) return;
  const int g = h / (a.Hq / a.Hkv);
  const int i = qb * kQBlock + 32 * wave + n;  // this lane's query row within the sequence
  const int64_t prow = (int64_t)h * a.lay.q_rows + s.q_row0 + i;
  const int koff = s.kv_len - s.q_len;
  // tile dump (tests only): this lane's row, when it is one of the dumped rows
  const bool dump_row = DUMP && i < s.q_len && i >= a.dbg_q0 && i < a.dbg_q0 + a.dbg_qn;
  const int64_t dump_at = DUMP ? (((int64_t)b * a.Hq + h) * a.dbg_qn + (i - a.dbg_q0)) * a.Nkv : 0;

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
                      DeltaRows(CAUSAL, s.q_len, s.kv_len).offset(qb);

  float m = kMaxFloor, lsum = 0.0f, ref = kMaxFloor - kLog2_448;
  v16f o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = v16f{};

  const DmaPlan<D> plan = make_dma_plan<D>(wave, lane);
  // per-lane LDS byte offsets of the compute reads (loop invariant)
  int kofs[4], kofs24[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) kofs[sub] = S::K_OFF + 16 * k_block<D>(32 * sub + n, S::R / 2 * hh);
  // the same offsets + 24, computed where the compiler cannot see the relation (see the K operand
  // reads below)
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) asm("v_add_u32 %0, 24, %1" : "=v"(kofs24[sub]) : "v"(kofs[sub]));
  int vofs[NCB][2][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int u = 0; u < 2; ++u) vofs[cb][h2][u] = S::V_OFF + 16 * v_block<D>(h2, 32 * cb + n, 2 * hh + u);

  if (nt > 0) issue_tile<D>(plan, wave, lane, 0, stage0, kcode, v8, drow, skp);
  wait_dma();
  __syncthreads();

  // one tile: DMA of tile t+1 into `nxt`, compute of tile t from `st`, wait, barrier
  auto step = [&](const int t, uint8_t* st, uint8_t* nxt) __attribute__((always_inline)) {
    // next tile: DMA into the other stage (last read before the previous barrier); it has this
    // whole iteration to land
    if (t + 1 < nt) issue_tile<D>(plan, wave, lane, t + 1, nxt, kcode, v8, drow, skp);
    if (t < nt_w) {
      // the wave needs masking only on a ragged last tile or where the causal edge crosses
      const bool need_mask = (t * kBN + kBN > s.kv_len) ||
                             (CAUSAL && t * kBN + kBN - 1 > wave_row0 + koff);
      const float* sks = reinterpret_cast<const float*>(st + S::S_OFF);
      float x[64];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        v16f acc = v16f{};
        if constexpr (D == 128) {
          // this lane's 48 bytes of the key row (rows keep their 3-block halves contiguous), as
          // 16 + 8 bytes per operand. Addressed from the same base, the compiler merges the two
          // middle 8-byte reads into one 16-byte read and then splits it over the two operand
          // tuples with register copies (14 per tile); with the second one addressed from the
          // opaque kofs24 the reads stay apart and land in place
          const uint4 b0 = *reinterpret_cast<const uint4*>(st + kofs[sub]);
          const uint2 b1 = *reinterpret_cast<const uint2*>(st + kofs[sub] + 16);
          const uint2 b2 = *reinterpret_cast<const uint2*>(st + kofs24[sub]);
          const uint4 b3 = *reinterpret_cast<const uint4*>(st + kofs[sub] + 32);
          const v8i k0 = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, 0, 0};
          const v8i k1 = {(int)b2.x, (int)b2.y, (int)b3.x, (int)b3.y, (int)b3.z, (int)b3.w, 0, 0};
          acc = mfma_fp6(k0, qop[0], acc);
          acc = mfma_fp6(k1, qop[NC6 - 1], acc);
        } else {
          // D = 64: 24 bytes at byte 24*hh of a 48-byte row
          const uint8_t* kr = st + S::K_OFF + (32 * sub + n) * S::CB + 24 * hh;
          acc = mfma_fp6(load_fp6_op(kr), qop[0], acc);
        }
        if constexpr (DUMP) {
          if (dump_row && a.dbg_s) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = t * kBN + 32 * sub + 8 * (r >> 2) + 4 * hh + (r & 3);
              if (key < s.kv_len) a.dbg_s[dump_at + key] = (int32_t)acc[r];
            }
          }
        }
        const float cs = cq * sks[2 * sub + hh];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const float4 dl = *reinterpret_cast<const float4*>(st + S::D_OFF + (32 * sub + 8 * a4 + 4 * hh) * 4);
          const float dv[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) x[16 * sub + 4 * a4 + e] = __builtin_fmaf(acc[4 * a4 + e], cs, dv[e]);
        }
      }
      if (need_mask) {
        // register k holds key t*kBN + 4*hh + off(k), off(k) a constant: one compare of the
        // constant with the lane's last visible offset per element
        int lim = s.kv_len - 1 - t * kBN - 4 * hh;
        if (CAUSAL) lim = min(lim, i + koff - t * kBN - 4 * hh);
#pragma unroll
        for (int k = 0; k < 64; ++k) {
          const int off = 32 * (k >> 4) + 8 * ((k & 15) >> 2) + (k & 3);
          x[k] = off <= lim ? x[k] : kNegInf;
        }
      }
      // running max over the previous value and this tile's keys, then over the two half-waves
      float mt = m;
#pragma unroll
      for (int k = 0; k < 64; ++k) mt = fmaxf(mt, x[k]);
      const float mnew = half_wave_max(mt);
      const float mb = mnew - kLog2_448;
      // renormalize (rarely: at the first visible key, then on large rises of the max) before the
      // fold factor 2^(mb - ref) could leave the f32 range
      if (!NOFOLD && __any(mb - ref > kFrameLimit)) {
        const float r = __builtin_amdgcn_exp2f(ref - mb);
        lsum *= r;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[cb][e] *= r;
        ref = mb;
      }
      // fold factor (fixed frame), or for the ablation the usual rescale alpha = 2^(m_prev - m)
      const float factor = NOFOLD ? __builtin_amdgcn_exp2f(m - mnew) : __builtin_amdgcn_exp2f(mb - ref);
      // (each exp is followed by independent adds: the transcendental unit then overlaps them)
      float ps = 0.0f;
#pragma unroll
      for (int k = 0; k < 64; ++k) {
        x[k] = __builtin_amdgcn_exp2f(x[k] - mb);
        ps += x[k];
      }
      lsum = NOFOLD ? __builtin_fmaf(factor, lsum, ps) : __builtin_fmaf(ps, factor, lsum);
      v8i pop[2];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        // bytes 2-3 of the first conversion's "old" operand are overwritten by the second
        const int w = cvt_fp8x2(x[4 * q], x[4 * q + 1], __float_as_int(x[4 * q]), false);
        pop[q >> 3][q & 7] = cvt_fp8x2(x[4 * q + 2], x[4 * q + 3], w, true);
      }
      if constexpr (DUMP) {
        if (dump_row && a.dbg_p8) {
#pragma unroll
          for (int k = 0; k < 64; ++k) {
            const int key = t * kBN + 32 * (k >> 4) + 8 * ((k & 15) >> 2) + 4 * hh + (k & 3);
            if (key < s.kv_len) a.dbg_p8[dump_at + key] = (uint8_t)(pop[k >> 5][(k >> 2) & 7] >> (8 * (k & 3)));
          }
        }
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        v16f inner = v16f{};
        if constexpr (NOFOLD) {
#pragma unroll
          for (int r = 0; r < 16; ++r) inner[r] = o[cb][r] * factor;
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint4 v0 = *reinterpret_cast<const uint4*>(st + vofs[cb][h2][0]);
          const uint4 v1 = *reinterpret_cast<const uint4*>(st + vofs[cb][h2][1]);
          const v8i vop = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
          inner = mfma_fp8(vop, pop[h2], inner);
        }
        if constexpr (NOFOLD) {
          o[cb] = inner;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[cb][r] = __builtin_fmaf(inner[r], factor, o[cb][r]);
        }
      }
      m = mnew;
    }
    wait_dma();
    __syncthreads();
  };
#pragma unroll 1
  for (int t = 0; t < nt; t += 2) {
    step(t, stage0, stage1);
    if (t + 1 < nt) step(t + 1, stage1, stage0);
  }

  lsum += __shfl_xor(lsum, 32, 64);
  if (i >= s.q_len) return;
  if (DUMP && a.o == nullptr) return;
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  const float* svp = ws_ptr<float>(a, a.lay.sv) + ((int64_t)b * a.Hkv + g) * D;
  constexpr int ES = OUT == SAGE2_F32 ? 4 : 2;
  char* orow = reinterpret_cast<char*>(a.o) + ES * row_index(a.os, b, s.q_start + i, h);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int c0 = 32 * cb + 8 * a4 + 4 * hh;
      if (c0 >= a.dt) continue;  // zero padding of a smaller head dim (dt is a multiple of 8)
      const float4 sv = *reinterpret_cast<const float4*>(svp + c0);
      store4<OUT>(orow + ES * c0, o[cb][4 * a4] * sv.x * inv, o[cb][4 * a4 + 1] * sv.y * inv,
                  o[cb][4 * a4 + 2] * sv.z * inv, o[cb][4 * a4 + 3] * sv.w * inv);
    }
  }
}

template <int D, int CAUSAL, int NOFOLD, int DUMP>
int launch_attn_f(const KArgs& a, hipStream_t st) {
  const dim3 grid((a.Nq + kQBlock - 1) / kQBlock * a.Hq, a.B);
  switch (a.out_dtype) {
    case SAGE2_F32: k_attn<D, CAUSAL, SAGE2_F32, NOFOLD, DUMP><<<grid, 256, 0, st>>>(a); break;
    case SAGE2_BF16: k_attn<D, CAUSAL, SAGE2_BF16, NOFOLD, DUMP><<<grid, 256, 0, st>>>(a); break;
    default: k_attn<D, CAUSAL, SAGE2_F16, NOFOLD, DUMP><<<grid, 256, 0, st>>>(a); break;
  }
  return (int)hipGetLastError();
}

template <int D, int CAUSAL>
int launch_attn_d(const KArgs& a, hipStream_t st) {
  return (a.flags & SAGE2_NO_FP32_FOLD) ? launch_attn_f<D, CAUSAL, 1, 0>(a, st)
                                        : launch_attn_f<D, CAUSAL, 0, 0>(a, st);
}

}  // namespace

int launch_attn(const KArgs& a, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.d == 64) return a.causal ? launch_attn_d<64, 1>(a, st) : launch_attn_d<64, 0>(a, st);
  return a.causal ? launch_attn_d<128, 1>(a, st) : launch_attn_d<128, 0>(a, st);
}

int launch_attn_dump(const KArgs& a, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // the two-level (production) form only
  if (a.d == 64) return a.causal ? launch_attn_f<64, 1, 0, 1>(a, st) : launch_attn_f<64, 0, 0, 1>(a, st);
  return a.causal ? launch_attn_f<128, 1, 0, 1>(a, st) : launch_attn_f<128, 0, 0, 1>(a, st);
}

}  // namespace sage2
