// Internal interface between the host library (argument checks, workspace layout) and the HIP
// launchers. Not installed; the public ABI is include/sage2.h.
#pragma once

#include <cstdint>

#include "sage2.h"

namespace sage2 {

constexpr int kQBlock = 128;   // Q smoothing block = attention workgroup Q tile (tokens)
constexpr int kKVPad = 128;    // per-sequence K/V row padding (K mean chunk size)
constexpr int kKVTile = 64;    // attention KV tile (keys)
constexpr int kSeqCols = 8;    // int32 columns of a sequence-table row

// Columns of the per-sequence table the plan kernel writes into the workspace.
enum SeqCol { kQStart = 0, kQLen, kKVStart, kKVLen, kQRow0, kKVRow0, kQBlk0, kDelta0 };

// Layout helpers shared by the host (workspace sizes) and the kernels (offsets).
#if defined(__HIPCC__)
#define SAGE2_HD __host__ __device__
#else
#define SAGE2_HD
#endif

// Smallest multiple of 128 that is >= x (x may be negative).
SAGE2_HD inline int64_t ceil128(int64_t x) { return x >= 0 ? (x + 127) / 128 * 128 : -((-x) / 128 * 128); }

// sum over b in [0, n) of min(K, max(0, 128 (b + 1) + c)), for c and K multiples of 128, K >= 0.
SAGE2_HD inline int64_t clamped_ramp_sum(int64_t n, int64_t c, int64_t K) {
  if (n <= 0) return 0;
  int64_t b0 = -c / 128;            // first b whose term is > 0
  if (b0 < 0) b0 = 0;
  int64_t b1 = (K - c) / 128 - 1;   // first b whose term is >= K
  if (b1 < b0) b1 = b0;
  const int64_t lo = b0 < n ? b0 : n, hi = b1 < n ? b1 : n;
  return 64 * (hi * (hi + 1) - lo * (lo + 1)) + c * (hi - lo) + (n - hi) * K;
}

// The correction table of one sequence (q_len queries, kv_len keys) is one row per 128-query block.
// Without a causal mask every row holds all kv_len keys rounded up to 128. With one, row qb holds
// only the keys [0, V(qb)), V(qb) = the block's last visible key + 1 rounded up to 128 (0 if it sees
// none): the attention kernel visits no other key tile, and the table shrinks to about half. For
// every block but the last, V(qb) = clamp(128 (qb + 1) + ceil128(kv_len - q_len), 0, kvpad); the
// last block sees every key.
// Offset of row qb within the sequence's table (qb <= number of blocks):
SAGE2_HD inline int64_t delta_row_offset(int causal, int64_t q_len, int64_t kv_len, int64_t qb) {
  const int64_t kvpad = ceil128(kv_len);
  if (!causal) return qb * kvpad;
  const int64_t nqb = (q_len + 127) / 128;
  if (qb >= nqb) return nqb == 0 ? 0 : clamped_ramp_sum(nqb - 1, ceil128(kv_len - q_len), kvpad) + kvpad;
  return clamped_ramp_sum(qb, ceil128(kv_len - q_len), kvpad);
}
// Entries of the sequence's whole table.
SAGE2_HD inline int64_t delta_seq_len(int causal, int64_t q_len, int64_t kv_len) {
  return delta_row_offset(causal, q_len, kv_len, (q_len + 127) / 128);
}

// Everything a kernel needs, passed by value.
struct KArgs {
  int32_t B, Hq, Hkv, Nq, Nkv, causal, in_dtype, out_dtype, varlen;
  int32_t d;      // head dim inside the workspace and kernels: 64 or 128
  int32_t dt;     // the caller's head dim (a multiple of 8, <= d); channels dt..d-1 are zero
  int32_t flags;  // sage2_flag bits
  float L;  // sm_scale * log2(e) in f32: logits are carried in base-2 units
  const void *q, *k, *v;
  void* o;
  int64_t qs[3], ks[3], vs[3], os[3];
  const int32_t *cu_q, *cu_kv;
  char* ws;
  sage2_ws_layout lay;
  // test-only dump of the attention kernel's own tiles (rows [dbg_q0, dbg_q0 + dbg_qn) of every
  // sequence and q head): INT32 S and e4m3 P~ codes, [B][Hq][dbg_qn][Nkv]; either may be null
  int32_t dbg_q0, dbg_qn;
  int32_t* dbg_s;
  uint8_t* dbg_p8;
};

// Launchers (defined in the .hip files). Return hipSuccess as 0, else the HIP error code.
int launch_prepass(const KArgs& a, void* stream);
int launch_attn(const KArgs& a, void* stream);
// the attention kernel with the tile dump of KArgs::dbg_* (a.o may be null: no output is written)
int launch_attn_dump(const KArgs& a, void* stream);

}  // namespace sage2
