// Host side of the C ABI: argument checks, workspace layout, launch dispatch.
// Pure C++ (no HIP headers): every check here runs before any device call.
#include <cmath>
#include <cstdint>
#include <climits>
#include <cstring>

#include "sage2_internal.h"

namespace sage2 {
namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int elem_size(int dt) { return dt == SAGE2_F32 ? 4 : 2; }

bool varlen_of(const sage2_params* p) {
  return p->cu_seqlens_q || p->cu_seqlens_kv || p->cu_seqlens_q_host || p->cu_seqlens_kv_host;
}

// Length of sequence b (host view).
void seq_lengths(const sage2_params* p, int b, int64_t* lq, int64_t* lkv) {
  if (varlen_of(p)) {
    *lq = p->cu_seqlens_q_host[b + 1] - p->cu_seqlens_q_host[b];
    *lkv = p->cu_seqlens_kv_host[b + 1] - p->cu_seqlens_kv_host[b];
  } else {
    *lq = p->N_q;
    *lkv = p->N_kv;
  }
}

sage2_status check_strides(const int64_t* s, int esize, bool varlen) {
  for (int i = varlen ? 1 : 0; i < 3; ++i) {
    if (s[i] < 0) return SAGE2_ERR_SHAPE;
    if ((s[i] * esize) % 16) return SAGE2_ERR_ALIGN;
  }
  return SAGE2_OK;
}

void compute_layout(const sage2_params* p, sage2_ws_layout* L);

// Checks everything that does not involve a data pointer.
sage2_status validate(const sage2_params* p) {
  if (!p) return SAGE2_ERR_NULL;
  if (p->d < 8 || p->d > 128 || p->d % 8) return SAGE2_ERR_UNSUPPORTED;
  if (p->flags & ~(SAGE2_NO_K_SMOOTH | SAGE2_NO_Q_SMOOTH | SAGE2_PER_BLOCK_SCALES | SAGE2_NO_FP32_FOLD))
    return SAGE2_ERR_UNSUPPORTED;
  if (p->in_dtype != SAGE2_F16 && p->in_dtype != SAGE2_BF16) return SAGE2_ERR_UNSUPPORTED;
  if (p->out_dtype != SAGE2_F16 && p->out_dtype != SAGE2_BF16 && p->out_dtype != SAGE2_F32)
    return SAGE2_ERR_UNSUPPORTED;
  if (!std::isfinite(p->sm_scale)) return SAGE2_ERR_UNSUPPORTED;
  if (p->causal != 0 && p->causal != 1) return SAGE2_ERR_UNSUPPORTED;
  if (p->B <= 0 || p->H_q <= 0 || p->H_kv <= 0 || p->N_q <= 0 || p->N_kv <= 0) return SAGE2_ERR_SHAPE;
  if (p->H_q % p->H_kv) return SAGE2_ERR_SHAPE;
  const bool vl = varlen_of(p);
  if (vl) {
    if (!p->cu_seqlens_q || !p->cu_seqlens_kv || !p->cu_seqlens_q_host || !p->cu_seqlens_kv_host)
      return SAGE2_ERR_NULL;
    if (p->cu_seqlens_q_host[0] != 0 || p->cu_seqlens_kv_host[0] != 0) return SAGE2_ERR_SHAPE;
    for (int b = 0; b < p->B; ++b) {
      int64_t lq, lkv;
      seq_lengths(p, b, &lq, &lkv);
      if (lq < 0 || lkv < 0 || lq > p->N_q || lkv > p->N_kv) return SAGE2_ERR_SHAPE;
    }
  }
  // the device's sequence table holds per-head workspace offsets as int32
  {
    sage2_ws_layout L;
    compute_layout(p, &L);
    const int64_t lim = INT32_MAX;
    if (L.q_rows > lim || L.kv_rows > lim || L.q_blocks > lim || L.delta_len > lim) return SAGE2_ERR_SHAPE;
  }
  const int ei = elem_size(p->in_dtype), eo = elem_size(p->out_dtype);
  sage2_status st;
  if ((st = check_strides(p->q_stride, ei, vl)) != SAGE2_OK) return st;
  if ((st = check_strides(p->k_stride, ei, vl)) != SAGE2_OK) return st;
  if ((st = check_strides(p->v_stride, ei, vl)) != SAGE2_OK) return st;
  if ((st = check_strides(p->o_stride, eo, vl)) != SAGE2_OK) return st;
  return SAGE2_OK;
}

// Head dim inside the workspace: the caller's d padded to 64 or 128.
int padded_d(int d) { return d <= 64 ? 64 : 128; }

void compute_layout(const sage2_params* p, sage2_ws_layout* L) {
  std::memset(L, 0, sizeof(*L));
  const int64_t d = padded_d(p->d);
  for (int b = 0; b < p->B; ++b) {
    int64_t lq, lkv;
    seq_lengths(p, b, &lq, &lkv);
    const int64_t nqb = ceil_div(lq, kQBlock);
    const int64_t kvpad = align_up(lkv, kKVPad);
    L->q_rows += nqb * kQBlock;
    L->q_blocks += nqb;
    L->kv_rows += kvpad;
    L->delta_len += delta_seq_len(p->causal, lq, lkv);
  }
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L->seq_table = take((int64_t)p->B * kSeqCols * 4);
  L->k_partial = take(p->H_kv * (L->kv_rows / kKVPad) * d * 8);
  L->v_partial = take(p->H_kv * (L->kv_rows / kKVPad) * d * 4);
  L->kbar = take((int64_t)p->B * p->H_kv * d * 4);
  L->sv = take((int64_t)p->B * p->H_kv * d * 4);
  L->sv_inv = take((int64_t)p->B * p->H_kv * d * 4);
  L->qbar = take(p->H_q * L->q_blocks * d * 4);
  L->qcode = take(p->H_q * L->q_rows * d * 3 / 4);
  L->sq = take(p->H_q * L->q_rows * 4);
  L->kcode = take(p->H_kv * L->kv_rows * d * 3 / 4);
  L->sk = take(p->H_kv * (L->kv_rows / 16) * 4);
  L->v8 = take(p->H_kv * L->kv_rows * d);
  L->delta = take(p->H_q * L->delta_len * 4);
  L->total_bytes = off;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

void fill_args(const sage2_params* p, KArgs* a) {
  std::memset(a, 0, sizeof(*a));
  a->B = p->B; a->Hq = p->H_q; a->Hkv = p->H_kv; a->Nq = p->N_q; a->Nkv = p->N_kv;
  a->d = padded_d(p->d);
  a->dt = p->d;
  a->flags = p->flags;
  a->causal = p->causal; a->in_dtype = p->in_dtype; a->out_dtype = p->out_dtype;
  a->varlen = varlen_of(p) ? 1 : 0;
  const float scale = p->sm_scale != 0.0f ? p->sm_scale : 1.0f / std::sqrt((float)p->d);
  a->L = scale * 1.44269504088896340736f;
  for (int i = 0; i < 3; ++i) {
    a->qs[i] = p->q_stride[i]; a->ks[i] = p->k_stride[i];
    a->vs[i] = p->v_stride[i]; a->os[i] = p->o_stride[i];
  }
  if (a->varlen) a->qs[0] = a->ks[0] = a->vs[0] = a->os[0] = 0;
  a->cu_q = p->cu_seqlens_q;
  a->cu_kv = p->cu_seqlens_kv;
  compute_layout(p, &a->lay);
}

sage2_status check_ws(const sage2_params* p, const void* ws, size_t ws_bytes) {
  if (!ws) return SAGE2_ERR_NULL;
  if ((uintptr_t)ws & 255) return SAGE2_ERR_ALIGN;
  sage2_ws_layout L;
  compute_layout(p, &L);
  if (ws_bytes < (size_t)L.total_bytes) return SAGE2_ERR_WORKSPACE;
  return SAGE2_OK;
}

}  // namespace
}  // namespace sage2

using namespace sage2;

extern "C" {

const char* sage2_status_string(sage2_status s) {
  switch (s) {
    case SAGE2_OK: return "ok";
    case SAGE2_ERR_NULL: return "a required pointer is NULL";
    case SAGE2_ERR_SHAPE: return "invalid sizes or sequence offsets";
    case SAGE2_ERR_UNSUPPORTED: return "unsupported head dim, dtype, flag, causal flag or scale";
    case SAGE2_ERR_ALIGN: return "pointer or stride not aligned (16 bytes; workspace 256 bytes)";
    case SAGE2_ERR_WORKSPACE: return "workspace too small";
    case SAGE2_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

sage2_status sage2_workspace_layout(const sage2_params* p, sage2_ws_layout* out) {
  if (!out) return SAGE2_ERR_NULL;
  const sage2_status st = validate(p);
  if (st != SAGE2_OK) return st;
  compute_layout(p, out);
  return SAGE2_OK;
}

sage2_status sage2_workspace_size(const sage2_params* p, size_t* bytes) {
  if (!bytes) return SAGE2_ERR_NULL;
  sage2_ws_layout L;
  const sage2_status st = sage2_workspace_layout(p, &L);
  if (st != SAGE2_OK) return st;
  *bytes = (size_t)L.total_bytes;
  return SAGE2_OK;
}

sage2_status sage2_quantize_smooth(const sage2_params* p, const void* q, const void* k,
                                   const void* v, void* ws, size_t ws_bytes, void* stream) {
  sage2_status st = validate(p);
  if (st != SAGE2_OK) return st;
  if (!q || !k || !v) return SAGE2_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return SAGE2_ERR_ALIGN;
  if ((st = check_ws(p, ws, ws_bytes)) != SAGE2_OK) return st;
  KArgs a;
  fill_args(p, &a);
  a.q = q; a.k = k; a.v = v; a.ws = (char*)ws;
  return launch_prepass(a, stream) == 0 ? SAGE2_OK : SAGE2_ERR_HIP;
}

sage2_status sage2_attn_fwd(const sage2_params* p, const void* ws, size_t ws_bytes, void* o,
                            void* stream) {
  sage2_status st = validate(p);
  if (st != SAGE2_OK) return st;
  if (!o) return SAGE2_ERR_NULL;
  if (!aligned16(o)) return SAGE2_ERR_ALIGN;
  if ((st = check_ws(p, ws, ws_bytes)) != SAGE2_OK) return st;
  KArgs a;
  fill_args(p, &a);
  a.o = o; a.ws = (char*)ws;
  return launch_attn(a, stream) == 0 ? SAGE2_OK : SAGE2_ERR_HIP;
}

sage2_status sage2_debug_attn_tiles(const sage2_params* p, const void* ws, size_t ws_bytes,
                                    int32_t q_begin, int32_t q_count, int32_t* s_out,
                                    uint8_t* p8_out, void* o, void* stream) {
  sage2_status st = validate(p);
  if (st != SAGE2_OK) return st;
  if (!s_out && !p8_out) return SAGE2_ERR_NULL;
  if (p->flags & SAGE2_NO_FP32_FOLD) return SAGE2_ERR_UNSUPPORTED;
  if (q_begin < 0 || q_count <= 0 || (int64_t)q_begin + q_count > p->N_q) return SAGE2_ERR_SHAPE;
  if (o && !aligned16(o)) return SAGE2_ERR_ALIGN;
  if ((st = check_ws(p, ws, ws_bytes)) != SAGE2_OK) return st;
  KArgs a;
  fill_args(p, &a);
  a.ws = (char*)ws;
  a.o = o;
  a.dbg_q0 = q_begin; a.dbg_qn = q_count; a.dbg_s = s_out; a.dbg_p8 = p8_out;
  return launch_attn_dump(a, stream) == 0 ? SAGE2_OK : SAGE2_ERR_HIP;
}

}  // extern "C"
