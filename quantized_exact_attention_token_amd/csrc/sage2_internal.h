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
