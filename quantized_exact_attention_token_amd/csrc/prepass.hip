// Pre-pass of the SageAttention2 forward pass on gfx950: smoothing statistics, INT4 codes and
// scales for Q and K, FP8 codes and scales for V, and the Q-smoothing correction table.
//
// Sources: PMLR vol. 267 page "SageAttention2: Efficient Attention with Thorough Outlier Smoothing
// and Per-thread INT4 Quantization", Abstract (Q,K to INT4 at thread granularity, P~,V to FP8, Q
// smoothing); research record of the same title, "Three components" (Q smoothing; per-thread scales);
// visual companion "SageAttention2 and Fast Exact INT4 Attention", "Channel Outlier Smoothing"
// (K smoothing) and "Per-Thread INT4 Geometry" (scale groups follow thread ownership).
//
// Every step that produces a code or a statistic uses a fixed order of IEEE operations (fp64 sums
// in token order over 128-token chunks, then chunks in order; f32 products and divisions, round to
// nearest even), so its result is reproducible bit for bit. Built with -ffp-contract=off.
//
// The pre-pass streams Q, K and V (HBM-bound); the correction table is an f32 MFMA product.
#include "device_common.h"

namespace sage2 {
namespace {

// ---- plan: per-sequence offsets into the padded workspace buffers ------------------------------
// Launched for variable-length batches only. One thread walks the sequences in order. A sequence whose device lengths disagree with what the
// host sized the workspace for (lengths above N, or totals past the layout) gets length 0, so no
// kernel touches memory outside the workspace.
__global__ void k_plan(KArgs a) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int32_t* t = ws_ptr<int32_t>(a, a.lay.seq_table);
  int64_t q_row = 0, kv_row = 0, qblk = 0, delta = 0;
  for (int b = 0; b < a.B; ++b) {
    int64_t qs = 0, ks = 0, lq = a.Nq, lk = a.Nkv;
    if (a.varlen) {
      qs = a.cu_q[b];
      ks = a.cu_kv[b];
      lq = a.cu_q[b + 1] - qs;
      lk = a.cu_kv[b + 1] - ks;
    }
    int64_t nqb = (lq + kQBlock - 1) / kQBlock;
    int64_t kvpad = (lk + kKVPad - 1) / kKVPad * kKVPad;
    // (lengths within the bounds the host validated, so the table size fits in int)
    const bool len_ok = lq >= 0 && lk >= 0 && lq <= a.Nq && lk <= a.Nkv;
    const int64_t dlen = len_ok ? DeltaRows(a.causal, (int)lq, (int)lk).total((int)lq) : 0;
    const bool ok = len_ok && q_row + nqb * kQBlock <= a.lay.q_rows &&
                    kv_row + kvpad <= a.lay.kv_rows && delta + dlen <= a.lay.delta_len;
    if (!ok) lq = lk = nqb = kvpad = 0;
    int32_t* r = t + b * kSeqCols;
    r[kQStart] = (int32_t)qs; r[kQLen] = (int32_t)lq;
    r[kKVStart] = (int32_t)ks; r[kKVLen] = (int32_t)lk;
    r[kQRow0] = (int32_t)q_row; r[kKVRow0] = (int32_t)kv_row;
    r[kQBlk0] = (int32_t)qblk; r[kDelta0] = (int32_t)delta;
    q_row += nqb * kQBlock;
    kv_row += kvpad;
    qblk += nqb;
    delta += ok ? dlen : 0;
  }
}

// Widening of one raw fp16 / bf16 element (exact).
template <int IN>
__device__ inline float widen16(uint32_t raw) {
  if constexpr (IN == SAGE2_BF16) {
    return __uint_as_float(raw << 16);
  } else {
    _Float16 h;
    const uint16_t r16 = (uint16_t)raw;
    __builtin_memcpy(&h, &r16, 2);
    return (float)h;
  }
}

// The 8 elements of a 16-byte chunk, widened.
template <int IN>
__device__ inline void widen8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = widen16<IN>(w[e] & 0xFFFFu);
    f[2 * e + 1] = widen16<IN>(w[e] >> 16);
  }
}

// Position of channel c in a row of the correction MFMA's operands (the block means in the
// workspace, the smoothed K tile in LDS): within each 8-channel group, the channels c, c+2, c+4,
// c+6 that one lane feeds to four consecutive k-steps sit side by side.
__device__ constexpr int mma_pos(int c) { return (c & ~7) | ((c & 1) << 2) | ((c >> 1) & 3); }

// Rows [tok0, tok0 + n) of one head of a strided input, as 16-byte chunks for a block of 256
// threads: chunk k of thread x is row (x + 256 k) / (D/8), channels 8 ((x + 256 k) % (D/8)) + [0, 8).
// All of a thread's loads are issued before any is waited on; rows n..NROWS-1 and channels dt..D-1
// (the zero padding of a head dim below D) are zero: they reread row n-1 / the last real chunk,
// which exist whenever n > 0, and are then cleared.
template <int D, int NROWS>
__device__ inline void load_rows(uint4 (&v)[NROWS * D / 8 / 256], const void* base, const int64_t* strides,
                                 int b, int64_t tok0, int head, int n, int dt) {
  constexpr int RW = D / 8;
  constexpr int IT = NROWS * RW / 256;
  static_assert(NROWS * RW % 256 == 0, "tile must split evenly over the block");
#pragma unroll
  for (int k = 0; k < IT; ++k) v[k] = make_uint4(0, 0, 0, 0);
  if (n > 0) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int idx = threadIdx.x + 256 * k, r = idx / RW, ch = idx % RW;
      v[k] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) +
                                             row_index(strides, b, tok0 + min(r, n - 1), head) +
                                             8 * min(ch, dt / 8 - 1));
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int idx = threadIdx.x + 256 * k;
      if (idx / RW >= n || 8 * (idx % RW) >= dt) v[k] = make_uint4(0, 0, 0, 0);
    }
  }
}

// The same rows, raw, into LDS rows of P >= D elements.
template <int D, int NROWS, int P = D>
__device__ inline void stage_rows(uint16_t (*dst)[P], const void* base, const int64_t* strides, int b,
                                  int64_t tok0, int head, int n, int dt) {
  constexpr int RW = D / 8;
  uint4 v[NROWS * RW / 256];
  load_rows<D, NROWS>(v, base, strides, b, tok0, head, n, dt);
#pragma unroll
  for (int k = 0; k < NROWS * RW / 256; ++k) {
    const int idx = threadIdx.x + 256 * k;
    *reinterpret_cast<uint4*>(&dst[idx / RW][8 * (idx % RW)]) = v[k];
  }
}

// ---- K channel sums and V channel max over one 128-token chunk ---------------------------------
// One workgroup of 256 per (128-key chunk, kv head, sequence). The chunk's K rows are staged in LDS
// (zero rows past the sequence end add +0.0, which leaves an fp64 sum unchanged); threads c < D
// then sum channel c in token order. V's channel max needs no order: each thread keeps the max of
// the 8 channels it loads, and threads D..2D-1 combine them.
// LDS bytes: the chunk's K rows (kKVPad x D raw elements), then 256 / (D / 8) rows of D floats
template <int D>
constexpr int kKstatsLds = 2 * kKVPad * D + 4 * (256 / (D / 8)) * D;

template <int D, int IN>
__device__ inline void kstats_chunk(const KArgs& a, int u, int g, int b, uint8_t* lds) {
  constexpr int RW = D / 8;
  constexpr int RPP = 256 / RW;  // rows per pass of the block over the chunk
  const int tid = threadIdx.x;
  const Seq s = load_seq(a, b);
  if (u * kKVPad >= s.kv_len) return;
  const int j0 = u * kKVPad, n = min(kKVPad, s.kv_len - j0);
  uint16_t(*kr)[D] = reinterpret_cast<uint16_t(*)[D]>(lds);
  float(*vm)[D] = reinterpret_cast<float(*)[D]>(lds + 2 * kKVPad * D);
  stage_rows<D, kKVPad>(kr, a.k, a.ks, b, s.kv_start + j0, g, n, a.dt);
  {
    // V: this thread's chunks all share channels 8 (tid % RW) + [0, 8) (256 is a multiple of RW)
    const int ch = tid % RW, r0 = tid / RW;
    uint4 v[kKVPad * RW / 256];
    load_rows<D, kKVPad>(v, a.v, a.vs, b, s.kv_start + j0, g, n, a.dt);
    float m8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < kKVPad * RW / 256; ++k) {
      float f[8];
      widen8<IN>(v[k], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) m8[e] = fmaxf(m8[e], fabsf(f[e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vm[r0][8 * ch + e] = m8[e];
  }
  __syncthreads();
  const int64_t slot0 = ((int64_t)g * (a.lay.kv_rows / kKVPad) + s.kv_row0 / kKVPad + u) * D;
  if (tid < D) {
    double part = 0.0;
#pragma unroll 16
    for (int i = 0; i < kKVPad; ++i) part += (double)widen16<IN>(kr[i][tid]);
    ws_ptr<double>(a, a.lay.k_partial)[slot0 + tid] = part;
  } else if (tid < 2 * D) {
    const int c = tid - D;
    float vmax = 0.0f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) vmax = fmaxf(vmax, vm[r][c]);
    ws_ptr<float>(a, a.lay.v_partial)[slot0 + c] = vmax;
  }
}

// ---- K mean and V scale: chunks reduced in order -----------------------------------------------
// grid (D/32 channel groups, H_kv, B), block 256: the chunk partials of 32 channels are brought
// into LDS 64 chunks at a time (8 loads in flight per thread), then 32 threads add them in chunk
// order (missing chunks past the end add +0.0).
template <int D>
__global__ __launch_bounds__(256) void k_kreduce(KArgs a) {
  const int cg = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int cl = tid & 31, rr = tid >> 5;
  const Seq s = load_seq(a, b);
  __shared__ double kp[64][32];
  __shared__ float vp[64][32];
  const int nch = (s.kv_len + kKVPad - 1) / kKVPad;
  const int64_t base = ((int64_t)g * (a.lay.kv_rows / kKVPad) + s.kv_row0 / kKVPad) * D + 32 * cg + cl;
  double total = 0.0;
  float amax = 0.0f;
  for (int u0 = 0; u0 < nch; u0 += 64) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = u0 + rr + 8 * k;
      kp[rr + 8 * k][cl] = u < nch ? ws_ptr<double>(a, a.lay.k_partial)[base + (int64_t)u * D] : 0.0;
      vp[rr + 8 * k][cl] = u < nch ? ws_ptr<float>(a, a.lay.v_partial)[base + (int64_t)u * D] : 0.0f;
    }
    __syncthreads();
    if (tid < 32) {
#pragma unroll 16
      for (int k = 0; k < 64; ++k) {
        total += kp[k][tid];
        amax = fmaxf(amax, vp[k][tid]);
      }
    }
    __syncthreads();
  }
  if (tid < 32) {
    const int64_t out = ((int64_t)b * a.Hkv + g) * D + 32 * cg + tid;
    float kbar = 0.0f, sv = 0.0f, svinv = 0.0f;
    if (s.kv_len > 0) {
      kbar = (a.flags & SAGE2_NO_K_SMOOTH) ? 0.0f : (float)(total / (double)s.kv_len);
      if (amax != 0.0f) {
        sv = amax / 448.0f;     // V channel amax maps to 448, the largest e4m3 value
        svinv = 448.0f / amax;
      }
    }
    ws_ptr<float>(a, a.lay.kbar)[out] = kbar;
    ws_ptr<float>(a, a.lay.sv)[out] = sv;
    ws_ptr<float>(a, a.lay.sv_inv)[out] = svinv;
  }
}

// INT4 code of x given its group's inverse scale, as an exact small-integer float: round to nearest
// even, clamp to [-7, 7] (never active: |x| <= amax and inv = 7/amax rounded keep |x * inv| < 7.5),
// and + 0 so that a code 0 is +0 (no negative-zero field below).
__device__ inline float int4_codef(float x, float inv) {
  return __builtin_amdgcn_fmed3f(rintf(x * inv), -7.0f, 7.0f) + 0.0f;
}

// 32 INT4 codes of consecutive channels (exact integers in float) -> 6 dwords of e2m3 (FP6) fields,
// field i (channel i) at bits [6i, 6i + 6), little-endian across the dwords: the fp6 MFMA operand
// format. Every integer in [-7, 7] is exact in e2m3, so the conversion is exact; the attention
// kernel feeds these fields to the fp6 MFMA, whose f32 accumulation of such integer products is
// exact. v_cvt_scalef32_2xpk16_fp6_f32 (scale 1) takes field 2i from element i of its first source
// and field 2i + 1 from element i of its second (checked bit for bit against a software packing).
__device__ inline void store_fp6_32(uint8_t* dst, const float (&c)[32]) {
  v16f ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = c[2 * i];
    od[i] = c[2 * i + 1];
  }
  const auto w = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
  *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  *reinterpret_cast<uint2*>(dst + 8) = make_uint2(w[2], w[3]);
  *reinterpret_cast<uint2*>(dst + 16) = make_uint2(w[4], w[5]);
}

// max over the lanes of an aligned group of LPR lanes (LPR a power of two <= 64)
template <int LPR>
__device__ inline float group_max(float x) {
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// The 32 raw elements [c0, c0 + 32) of a staged LDS row, widened.
template <int IN>
__device__ inline void widen32(const uint16_t* p, float (&f)[32]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float g[8];
    widen8<IN>(*reinterpret_cast<const uint4*>(p + 8 * k), g);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[8 * k + e] = g[e];
  }
}

// Row pitch (elements) of the Q and K rows that lanes then read 32 channels at a time: 16 bytes
// more than a row, so the rows of consecutive keys start in different LDS banks (with a pitch of
// exactly D the lanes of one channel group would all hit the same banks).
template <int D>
constexpr int kPitch = D + 8;

// ---- Q: block mean, per-token INT4 codes -------------------------------------------------------
// One workgroup of 256 per (Q block, q head, sequence). The block's rows are read once, coalesced,
// into LDS (rows past the sequence end are zero and add +0.0 to the fp64 sums); thread c sums
// channel c in row order. The rows are then quantized with D/32 lanes per row and 32 channels per
// lane (one scale per token: on gfx950 a lane owns one query column of the S^T = K Q^T MFMA tile,
// so the per-thread group is one token).
// LDS bytes: the block's Q rows (kQBlock rows of kPitch raw elements), then the D block means (f32)
template <int D>
constexpr int kQuantQLds = 2 * kQBlock * kPitch<D> + 4 * D;

template <int D, int IN>
__device__ inline void quant_q_block(const KArgs& a, int qb, int h, int b, uint8_t* lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const Seq s = load_seq(a, b);
  if (qb * kQBlock >= s.q_len) return;
  const int i0 = qb * kQBlock, n = min(kQBlock, s.q_len - i0);
  uint16_t(*rows)[kPitch<D>] = reinterpret_cast<uint16_t(*)[kPitch<D>]>(lds);
  float* qbar = reinterpret_cast<float*>(lds + 2 * kQBlock * kPitch<D>);
  stage_rows<D, kQBlock, kPitch<D>>(rows, a.q, a.qs, b, s.q_start + i0, h, n, a.dt);
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
#pragma unroll 16
    for (int i = 0; i < kQBlock; ++i) sum += (double)widen16<IN>(rows[i][tid]);
    const float m = (a.flags & SAGE2_NO_Q_SMOOTH) ? 0.0f : (float)(sum / (double)n);
    qbar[tid] = m;
    const int64_t at = ((int64_t)h * a.lay.q_blocks + s.qblk0 + qb) * D + mma_pos(tid);
    ws_ptr<float>(a, a.lay.qbar)[at] = m;
  }
  __syncthreads();
  uint8_t* qcode = ws_ptr<uint8_t>(a, a.lay.qcode);
  float* sq = ws_ptr<float>(a, a.lay.sq);
  // LPR lanes per row, 32 channels each: rows [r0, r0 + 256 / LPR) per pass of the block
  constexpr int LPR = D / 32;
  constexpr int RPP = 256 / LPR;
  const int lr = lane % LPR, c0 = 32 * lr;
  float qm[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) qm[e] = qbar[c0 + e];
  // per-block ablation: one scale for the whole block (the largest |q - qbar| in it)
  const bool per_block = a.flags & SAGE2_PER_BLOCK_SCALES;
  float bmax = 0.0f;
  if (per_block) {
    __shared__ float wmax[4];
    for (int r0 = 0; r0 < kQBlock; r0 += RPP) {
      const int r = r0 + tid / LPR;
      float raw[32];
      widen32<IN>(&rows[r][c0], raw);
#pragma unroll
      for (int e = 0; e < 32; ++e) bmax = fmaxf(bmax, r < n ? fabsf(raw[e] - qm[e]) : 0.0f);
    }
    bmax = wave_max(bmax);
    if (lane == 0) wmax[wave] = bmax;
    __syncthreads();
    bmax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  }
  for (int r0 = 0; r0 < kQBlock; r0 += RPP) {
    const int r = r0 + tid / LPR;
    const int64_t prow = (int64_t)h * a.lay.q_rows + s.q_row0 + i0 + r;
    float qt[32];
    widen32<IN>(&rows[r][c0], qt);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      qt[e] = r < n ? qt[e] - qm[e] : 0.0f;
      amax = fmaxf(amax, fabsf(qt[e]));
    }
    amax = per_block ? bmax : group_max<LPR>(amax);
    const float inv = amax == 0.0f ? 0.0f : 7.0f / amax;
    const float scale = amax == 0.0f || r >= n ? 0.0f : amax / 7.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) qt[e] = int4_codef(qt[e], inv);
    store_fp6_32(qcode + prow * (3 * D / 4) + 24 * lr, qt);
    if (lr == 0) sq[prow] = scale;
  }
}

// Key index (within a 64-key tile) held in slot s of lane half h: the S^T accumulator of the
// 32x32 MFMA gives lane half h the rows 8*(r/4) + 4*h + r%4 of each 32-key subtile.
__device__ inline int tile_key(int h, int s) { return 32 * (s >> 4) + 8 * ((s & 15) >> 2) + 4 * h + (s & 3); }

// ---- the K/V statistics and the Q quantizer in one launch ---------------------------------------
// Both read only the inputs (and the sequence table): grid (128-key chunks x H_kv + Q blocks x
// H_q, 1, B), first the statistics workgroups (x = chunk * H_kv + kv head), then the Q blocks
// (x = block * H_q + q head).
template <int D, int IN>
__global__ __launch_bounds__(256) void k_stats_quant_q(KArgs a, int n_chunks) {
  constexpr int LDS = kKstatsLds<D> > kQuantQLds<D> ? kKstatsLds<D> : kQuantQLds<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
  const int n = n_chunks * a.Hkv, x = blockIdx.x;
  if (x < n) kstats_chunk<D, IN>(a, x / a.Hkv, x % a.Hkv, blockIdx.z, lds);
  else quant_q_block<D, IN>(a, (x - n) / a.Hq, (x - n) % a.Hq, blockIdx.z, lds);
}

// ---- K: per-16-key-group INT4 codes; V: FP8 codes in the attention kernel's tile layout -------
// One workgroup of 256 per (64-key tile, kv head, sequence). The tile's K rows are staged in LDS
// with 16-byte loads (zero past the sequence end); V is scaled and converted to FP8 in registers
// (each thread one 16-byte chunk of the keys of 4 or 2 consecutive output slots) and transposed
// through LDS as bytes, then copied out in 32-byte rows. Wave w quantizes K group w of the tile:
// the 16 keys of 32-key subtile w/2 whose index has bit 2 equal to w%2 (the keys one lane half
// owns), D/32 lanes per key with 32 channels each; the smoothed values stay in registers between
// the group max and the codes.
// LDS bytes of one K/V quantizer workgroup: kbar, 1/s_v (D floats each), the K rows (kKVTile rows
// of kPitch raw elements), and the V codes in the output order (for channel c and lane half h the
// 32 fp8 bytes of the keys tile_key(h, 0..31), at byte vrow(c, h))
template <int D>
constexpr int kQuantKvLds = 8 * D + 2 * kKVTile * kPitch<D> + 64 * D + 2 * D;

// Byte offset of the V code row of channel c, lane half h: rows of 32 bytes, with 16 more bytes
// after every 8 channels, so that the words the lanes of one wave write for the same channel index
// (channels 8 apart) fall in different LDS banks
__device__ inline int vrow(int c, int h) { return (2 * c + h) * 32 + 16 * (c >> 3); }

template <int D, int IN>
__device__ inline void quant_kv_tile(const KArgs& a, int t, int g, int b, uint8_t* lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const Seq s = load_seq(a, b);
  const int kvpad = (s.kv_len + kKVPad - 1) / kKVPad * kKVPad;
  if (t * kKVTile >= kvpad) return;
  float* kbar = reinterpret_cast<float*>(lds);
  float* svinv = kbar + D;
  uint16_t(*kr)[kPitch<D>] = reinterpret_cast<uint16_t(*)[kPitch<D>]>(lds + 8 * D);
  uint32_t* vt8 = reinterpret_cast<uint32_t*>(lds + 8 * D + 2 * kKVTile * kPitch<D>);
  const int64_t sidx = ((int64_t)b * a.Hkv + g) * D;
  if (tid < D) {
    kbar[tid] = ws_ptr<float>(a, a.lay.kbar)[sidx + tid];
    svinv[tid] = ws_ptr<float>(a, a.lay.sv_inv)[sidx + tid];
  }
  const int n = max(0, min(kKVTile, s.kv_len - t * kKVTile));
  stage_rows<D, kKVTile, kPitch<D>>(kr, a.k, a.ks, b, s.kv_start + t * kKVTile, g, n, a.dt);
  // V: this thread's 16-byte chunk (channels 8 ch + [0, 8)) of KPT keys that are consecutive both
  // in the tile and in the output order (slots s0 .. s0 + KPT - 1 of lane half h)
  constexpr int RW = D / 8;
  constexpr int KPT = kKVTile * RW / 256;
  constexpr int NG = 32 / KPT;
  const int ch = tid % RW, grp = tid / RW, h = grp / NG, s0 = KPT * (grp % NG);
  const int key0 = tile_key(h, s0);
  uint4 vr[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    vr[e] = make_uint4(0, 0, 0, 0);
    if (key0 + e < n && 8 * ch < a.dt)
      vr[e] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.v) +
                                              row_index(a.vs, b, s.kv_start + t * kKVTile + key0 + e, g) +
                                              8 * ch);
  }
  __syncthreads();
  {
    float f[KPT][8];
#pragma unroll
    for (int e = 0; e < KPT; ++e) widen8<IN>(vr[e], f[e]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 8 * ch + i;
      const float sc = svinv[c];
      const int w = cvt_fp8x2(f[0][i] * sc, f[1][i] * sc, 0, false);
      if constexpr (KPT == 4) {
        vt8[(vrow(c, h) + s0) / 4] = (uint32_t)cvt_fp8x2(f[2][i] * sc, f[3][i] * sc, w, true);
      } else {
        reinterpret_cast<uint16_t*>(vt8)[(vrow(c, h) + s0) / 2] = (uint16_t)w;
      }
    }
  }
  // K group of this wave: its 16 keys, LPR lanes per key with 32 channels each (for D = 64 the
  // upper half-wave repeats the lower one and does not store)
  {
    constexpr int LPR = D / 32;
    const int half = wave & 1, sub = wave >> 1;
    const int lr = lane % LPR, c0 = 32 * lr;
    const int e = (lane / LPR) & 15;
    const int key = 32 * sub + 8 * (e >> 2) + 4 * half + (e & 3);  // within the tile
    float val[32];
    widen32<IN>(&kr[key][c0], val);
    float amax = 0.0f;
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      val[x] = key < n ? val[x] - kbar[c0 + x] : 0.0f;
      amax = fmaxf(amax, fabsf(val[x]));
    }
    amax = wave_max(amax);
    if (a.flags & SAGE2_PER_BLOCK_SCALES) {
      // per-block ablation: one scale for the 64-key tile (the four groups' largest)
      __shared__ float gmax[4];
      if (lane == 0) gmax[wave] = amax;
      __syncthreads();
      amax = fmaxf(fmaxf(gmax[0], gmax[1]), fmaxf(gmax[2], gmax[3]));
    }
    const float inv = amax == 0.0f ? 0.0f : 7.0f / amax;
    const float scale = amax == 0.0f ? 0.0f : amax / 7.0f;
#pragma unroll
    for (int x = 0; x < 32; ++x) val[x] = int4_codef(val[x], inv);
    const int j = t * kKVTile + key;
    if (lane < 16 * LPR)
      store_fp6_32(ws_ptr<uint8_t>(a, a.lay.kcode) + ((int64_t)g * a.lay.kv_rows + s.kv_row0 + j) * (3 * D / 4) + 24 * lr,
                   val);
    if (lane == 0)
      ws_ptr<float>(a, a.lay.sk)[(int64_t)g * (a.lay.kv_rows / 16) + s.kv_row0 / 16 + 4 * t + wave] = scale;
  }
  __syncthreads();
  uint8_t* v8 = ws_ptr<uint8_t>(a, a.lay.v8) +
                ((int64_t)g * (a.lay.kv_rows / kKVTile) + s.kv_row0 / kKVTile + t) * (kKVTile * D);
  for (int p = tid; p < 2 * D; p += 256) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(vt8) + vrow(p >> 1, p & 1));
    uint4* dst = reinterpret_cast<uint4*>(v8 + (int64_t)p * 32);
    dst[0] = src[0];
    dst[1] = src[1];
  }
}

// ---- correction table: delta[qb][j] = (qbar_qb . ktilde_j) * sm_scale * log2(e) ---------------
// Q smoothing removes each block's mean from the INT4 product; this adds back its share with the
// unquantized smoothed K: an f32 fused multiply-add chain over the channels in order from +0,
// then one f32 multiply by sm_scale * log2(e).
// The chains run on v_mfma_f32_32x32x2_f32: on gfx950 it accumulates every output as two fused
// multiply-adds in k order on top of C (checked bit for bit against sequential fmaf() on
// 8.4 million outputs of random-sign inputs spread over 24 binades), so feeding it the channels
// two at a time, in order, is exactly the channel-order chain, at twice the fp64 MFMA's rate.
// Operand layouts: A[i][k] in lane i + 32k, B[k][j] in lane j + 32k, D[i][j] in lane
// j + 32 ((i / 4) % 2), register 4 (i / 8) + i % 4.
// One workgroup of 256 per (64-key tile, kv head, sequence): k~ of the tile in LDS (f32, a 4-float
// row skew, channels in MFMA order). Only the (q head, Q block) pairs that see a key of the tile
// are computed: they are numbered Q block major and dealt to the waves in blocks of 32 pairs x the
// 64 keys = 2 MFMA tiles, so a causal mask leaves no wave idle. Entries a causal mask hides from every row of a Q
// block are left unwritten (the attention kernel masks such keys by selection, never reads them
// into arithmetic that reaches the output) except within a computed tile, where they are stored as
// 0.
typedef float v4f __attribute__((ext_vector_type(4)));

// LDS bytes of one correction-table workgroup: the tile's k~ rows of D + 4 floats
template <int D>
constexpr int kDeltaLds = 4 * kKVTile * (D + 4);

// What a correction-table work item needs besides its pair block and key range.
struct DeltaItem {
  const KArgs& a;
  const Seq& s;
  const float* kt;  // k~ tile in LDS, rows of D + 4 floats
  DeltaRows rows;   // row offsets of the sequence's correction table
  const float* qbar;
  float* delta;
  float L;
  int t, g, grp, qbmin, nlive, koff, li, lk;
  int grp_log2;  // log2(grp) when grp is a power of two, else -1
};

// Correction values of 32 pairs (from p0) x 32 NKB keys (from key k0 of the tile): NKB f32 MFMA
// tiles of 32 x 32 over all D channels, then the stores.
template <int D, int NKB>
__device__ inline void delta_item(const DeltaItem& c, int p0, int k0) {
  constexpr int KS = D + 4;
  // A[i][k]: the mean of pair p0 + i (rows of pairs past the end read the clamped last pair: an
  // output row depends only on its own A row, and those rows are never stored)
  const float* qrow;
  {
    const int pc = min(p0 + c.li, c.nlive - 1);
    const int h = c.g * c.grp + pc % c.grp, qb = c.qbmin + pc / c.grp;
    qrow = c.qbar + ((int64_t)h * c.a.lay.q_blocks + c.s.qblk0 + qb) * D + 4 * c.lk;
  }
  v16f acc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) acc[kb] = v16f{};
  // channels in chunks of 8 (4 MFMA k-steps of 2 channels). Both operands are stored with the
  // channels of a chunk in MFMA order (mma_pos), so one 16-byte read gives a lane its operand for
  // all 4 k-steps. The next chunk's means are requested before the current chunk's MFMAs, so their
  // latency hides behind them.
  v4f a_cur = *reinterpret_cast<const v4f*>(qrow), a_nxt;
  const float* kr = c.kt + (k0 + c.li) * KS + 4 * c.lk;
#pragma unroll 1
  for (int ch = 0; ch < D; ch += 8) {
    const int nx = ch + 8 < D ? ch + 8 : 0;  // (the last prefetch rereads chunk 0, unused)
    a_nxt = *reinterpret_cast<const v4f*>(qrow + nx);
    // (an empty asm statement that clobbers memory keeps this load in this iteration: without it
    // the compiler moves it into the next one, next to its use, and waits on it there)
    asm volatile("" ::: "memory");
    v4f bv[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) bv[kb] = *reinterpret_cast<const v4f*>(kr + 32 * kb * KS + ch);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a_cur[u], bv[kb][u], acc[kb], 0, 0, 0);
    a_cur = a_nxt;
  }
  // D[i][j] in register r of lane l: pair p0 + 8 (r / 4) + 4 (l / 32) + r % 4, key
  // t*64 + k0 + 32 kb + l % 32. One store instruction writes two pairs' 32 consecutive keys.
  const int j0 = c.t * kKVTile + k0 + c.li;
  const int64_t dl = c.a.lay.delta_len;
  // last key that any row of Q block qb sees
  auto last_key = [&](int qb) __attribute__((always_inline)) {
    int jm = c.s.kv_len - 1;
    if (c.a.causal) jm = min(jm, min(c.s.q_len, (qb + 1) * kQBlock) - 1 + c.koff);
    return jm;
  };
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int pb = p0 + 8 * r4 + 4 * c.lk;  // pair of register 4 r4 (a multiple of 4)
    if (c.grp_log2 >= 2) {
      // grp a power of two >= 4: pairs pb .. pb + 3 are four consecutive q heads of one Q block
      // (and nlive, a multiple of grp, covers all four or none), so the row offset and the last
      // visible key are computed once for the four registers
      if (pb >= c.nlive) continue;
      const int qb = c.qbmin + (pb >> c.grp_log2);
      const int jm = last_key(qb);
      float* drow = c.delta + (int64_t)(c.g * c.grp + (pb & (c.grp - 1))) * dl + c.s.delta0 +
                    c.rows.offset(qb);
#pragma unroll
      for (int r1 = 0; r1 < 4; ++r1)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int j = j0 + 32 * kb;
          drow[r1 * dl + j] = j <= jm ? acc[kb][4 * r4 + r1] * c.L : 0.0f;
        }
    } else {
#pragma unroll
      for (int r1 = 0; r1 < 4; ++r1) {
        const int pair = pb + r1;
        if (pair >= c.nlive) continue;
        const int pq = c.grp_log2 >= 0 ? pair >> c.grp_log2 : pair / c.grp;
        const int h = c.g * c.grp + (pair - pq * c.grp), qb = c.qbmin + pq;
        const int jm = last_key(qb);
        float* drow = c.delta + (int64_t)h * dl + c.s.delta0 + c.rows.offset(qb);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int j = j0 + 32 * kb;
          drow[j] = j <= jm ? acc[kb][4 * r4 + r1] * c.L : 0.0f;
        }
      }
    }
  }
}

template <int D, int IN>
__device__ inline void delta_tile(const KArgs& a, int t, int g, int b, float* kt) {
  constexpr int KS = D + 4;  // floats per k~ row in LDS
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Seq s = load_seq(a, b);
  const int kvpad = (s.kv_len + kKVPad - 1) / kKVPad * kKVPad;
  if (t * kKVTile >= kvpad) return;
  const float* kbar = ws_ptr<float>(a, a.lay.kbar) + ((int64_t)b * a.Hkv + g) * D;
  {
    // k~ = k - kbar in f32 (keys past the sequence end: 0)
    constexpr int RW = D / 8;
    const int n = max(0, min(kKVTile, s.kv_len - t * kKVTile));
    uint4 v[kKVTile * RW / 256];
    load_rows<D, kKVTile>(v, a.k, a.ks, b, s.kv_start + t * kKVTile, g, n, a.dt);
#pragma unroll
    for (int k = 0; k < kKVTile * RW / 256; ++k) {
      const int idx = tid + 256 * k, key = idx / RW, ch = idx % RW;
      float f[8];
      widen8<IN>(v[k], f);
      const v4f m0 = *reinterpret_cast<const v4f*>(kbar + 8 * ch);
      const v4f m1 = *reinterpret_cast<const v4f*>(kbar + 8 * ch + 4);
      const float m[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
      // the chunk's 8 channels are one MFMA-order group: channel 8 ch + e at 8 ch + mma_pos(e),
      // the even channels first, then the odd ones
      v4f even, odd;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        even[u] = key < n ? f[2 * u] - m[2 * u] : 0.0f;
        odd[u] = key < n ? f[2 * u + 1] - m[2 * u + 1] : 0.0f;
      }
      static_assert(mma_pos(2) == 1 && mma_pos(1) == 4, "staging order must match mma_pos");
      *reinterpret_cast<v4f*>(kt + key * KS + 8 * ch) = even;
      *reinterpret_cast<v4f*>(kt + key * KS + 8 * ch + 4) = odd;
    }
  }
  __syncthreads();
  const int grp = a.Hq / a.Hkv;
  const int nqb = (s.q_len + kQBlock - 1) / kQBlock;
  const int koff = s.kv_len - s.q_len;
  const int li = lane & 31, lk = lane >> 5;
  float* delta = ws_ptr<float>(a, a.lay.delta);
  const float* qbar = ws_ptr<float>(a, a.lay.qbar);
  // first Q block that sees a key of this tile (the last key a Q block sees is non-decreasing in qb)
  int qbmin;
  if (t * kKVTile >= s.kv_len) {
    qbmin = nqb;
  } else if (!a.causal) {
    qbmin = 0;
  } else {
    const int T = t * kKVTile + 1 - koff;  // needs min(q_len, (qb + 1) * 128) >= T
    qbmin = T <= 0 ? 0 : (T > s.q_len ? nqb : (T + kQBlock - 1) / kQBlock - 1);
  }
  // live pairs, Q-block major: pair p -> Q block qbmin + p / grp, q head g * grp + p % grp. Work
  // items are blocks of 32 pairs x the tile's 64 keys, dealt round-robin to the waves; a tile with
  // fewer than 4 blocks (one or two q heads per kv head, or the last tiles under a causal mask)
  // splits each block's keys in two halves instead, so that up to twice as many waves have work
  const int nlive = (nqb - qbmin) * grp;
  const int nblk = (nlive + 31) / 32;
  const int grp_log2 = (grp & (grp - 1)) == 0 ? __builtin_ctz(grp) : -1;
  const DeltaItem it{a, s, kt, DeltaRows(a.causal, s.q_len, s.kv_len), qbar, delta, a.L, t, g, grp,
                     qbmin, nlive, koff, li, lk, grp_log2};
  if (nblk >= 4) {
    for (int w = wave; w < nblk; w += 4) delta_item<D, 2>(it, 32 * w, 0);
  } else {
    for (int w = wave; w < 2 * nblk; w += 4) delta_item<D, 1>(it, 32 * (w >> 1), 32 * (w & 1));
  }
}

// ---- the K/V quantizer and the correction table in one launch ----------------------------------
// The two read the statistics of the previous kernels and not each other's output; run side by
// side, the HBM-bound quantizer workgroups fill the CUs next to the MFMA-bound correction
// workgroups as the correction workgroups drain. grid (2 x 64-key tiles x H_kv, 1, B): first the
// correction workgroups, x = tile * H_kv + kv head (longest first under a causal mask), then the
// quantizer workgroups in the same order. (Quantizers first, or the two roles interleaved, measured
// slower: the interleaved order stretched the pre-pass by half.) At most 128 VGPRs: four
// workgroups per CU, as many as the correction tile's LDS allows.
template <int D, int IN>
__global__ __launch_bounds__(256, 4) void k_kv_delta(KArgs a, int n_tiles) {
  constexpr int LDS = kDeltaLds<D> > kQuantKvLds<D> ? kDeltaLds<D> : kQuantKvLds<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
  const int n = n_tiles * a.Hkv, x = blockIdx.x;
  if (x < n) delta_tile<D, IN>(a, x / a.Hkv, x % a.Hkv, blockIdx.z, reinterpret_cast<float*>(lds));
  else quant_kv_tile<D, IN>(a, (x - n) / a.Hkv, (x - n) % a.Hkv, blockIdx.z, lds);
}

template <int D, int IN>
int launch_all(const KArgs& a, hipStream_t st) {
  const int nch = (a.Nkv + kKVPad - 1) / kKVPad;
  const int nqb = (a.Nq + kQBlock - 1) / kQBlock;
  const int ntile = nch * (kKVPad / kKVTile);
  // without cu_seqlens the kernels compute each sequence's offsets from its index (load_seq)
  if (a.varlen) k_plan<<<1, 64, 0, st>>>(a);
  k_stats_quant_q<D, IN><<<dim3(nch * a.Hkv + nqb * a.Hq, 1, a.B), 256, 0, st>>>(a, nch);
  k_kreduce<D><<<dim3(D / 32, a.Hkv, a.B), 256, 0, st>>>(a);
  k_kv_delta<D, IN><<<dim3(2 * ntile * a.Hkv, 1, a.B), 256, 0, st>>>(a, ntile);
  return (int)hipGetLastError();
}

}  // namespace

int launch_prepass(const KArgs& a, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.d == 64) return a.in_dtype == SAGE2_BF16 ? launch_all<64, SAGE2_BF16>(a, st) : launch_all<64, SAGE2_F16>(a, st);
  return a.in_dtype == SAGE2_BF16 ? launch_all<128, SAGE2_BF16>(a, st) : launch_all<128, SAGE2_F16>(a, st);
}

}  // namespace sage2
