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

// The correction table of one sequence (q_len queries, kv_len keys) is one row per 128-query block.
// Without a causal mask every row holds all kv_len keys rounded up to 128 (kvpad). With one, row qb
// holds only the keys [0, V(qb)), V(qb) = the block's last visible key + 1 rounded up to 128 (0 if
// it sees none): the attention kernel visits no other key tile, and the table shrinks to about half.
// In units of 128 keys, every block but the last has V(qb)/128 = clamp(qb + 1 + c, 0, K), with
// K = kvpad / 128 and c = ceil128(kv_len - q_len) / 128; the last block sees every key. So the row
// offset of block qb is G(qb + c) - G(c) units, G(n) = sum over v = 1..n of min(v, K) (0 for n <= 0).
// I is the integer type of the arithmetic: int64_t on the host (before any size is validated), int in
// the kernels (the host refuses workspaces whose per-head table passes 2^31 - 1 entries, so every
// offset and every G value, at most 2^24 units, fits).
template <typename I>
struct DeltaRowsT {
  I kvpad, K, c, g0;
  int causal;
  SAGE2_HD static I G(I n, I K) {
    const I np = n > 0 ? n : 0;
    const I t = np < K ? np : K;
    return t * (t + 1) / 2 + (np - t) * K;
  }
  SAGE2_HD DeltaRowsT(int causal_, I q_len, I kv_len) {
    causal = causal_;
    kvpad = (I)ceil128(kv_len);
    K = kvpad / 128;
    c = (I)(ceil128(kv_len - q_len) / 128);
    g0 = G(c, K);
  }
  // offset of row qb within the sequence's table, for 0 <= qb < number of Q blocks
  SAGE2_HD I offset(I qb) const { return causal ? 128 * (G(qb + c, K) - g0) : qb * kvpad; }
  // entries of the sequence's whole table (the last block holds every key)
  SAGE2_HD I total(I q_len) const {
    const I nqb = (q_len + 127) / 128;
    return nqb == 0 ? 0 : offset(nqb - 1) + kvpad;
  }
};
using DeltaRows = DeltaRowsT<int>;

// Entries of one sequence's whole table (host arithmetic).
inline int64_t delta_seq_len(int causal, int64_t q_len, int64_t kv_len) {
  return DeltaRowsT<int64_t>(causal, q_len, kv_len).total(q_len);
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
