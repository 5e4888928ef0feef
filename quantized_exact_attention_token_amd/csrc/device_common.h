// Device helpers shared by the pre-pass and attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sage2_internal.h"

namespace sage2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_huge_valf();

struct Seq {
  int32_t q_start, q_len, kv_start, kv_len, q_row0, kv_row0, qblk0, delta0;
};

// Sequence b's extents and workspace offsets. Without cu_seqlens every sequence has the full
// lengths and the offsets follow from b (the same values the plan kernel writes, with no memory
// read ahead of a workgroup's first loads); with them, the plan kernel's table.
__device__ inline Seq load_seq(const KArgs& a, int b) {
  if (!a.varlen) {
    const int nqb = (a.Nq + kQBlock - 1) / kQBlock;
    const int kvpad = (a.Nkv + kKVPad - 1) / kKVPad * kKVPad;
    return Seq{0, a.Nq, 0, a.Nkv, b * nqb * kQBlock, b * kvpad, b * nqb,
               b * DeltaRows(a.causal, a.Nq, a.Nkv).total(a.Nq)};
  }
  const int32_t* t = reinterpret_cast<const int32_t*>(a.ws + a.lay.seq_table) + b * kSeqCols;
  Seq s;
  s.q_start = t[kQStart]; s.q_len = t[kQLen]; s.kv_start = t[kKVStart]; s.kv_len = t[kKVLen];
  s.q_row0 = t[kQRow0]; s.kv_row0 = t[kKVRow0]; s.qblk0 = t[kQBlk0]; s.delta0 = t[kDelta0];
  return s;
}

template <typename T>
__device__ inline T* ws_ptr(const KArgs& a, int64_t off) {
  return reinterpret_cast<T*>(a.ws + off);
}

// Element index of (token, head, channel 0) of sequence b in a strided input.
__device__ inline int64_t row_index(const int64_t* s, int b, int64_t token, int head) {
  return (int64_t)b * s[0] + token * s[1] + (int64_t)head * s[2];
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Two f32 -> two OCP e4m3 bytes (round to nearest even), into bytes 0-1 (hi = false) or 2-3
// (hi = true) of `old`.
__device__ inline int cvt_fp8x2(float a, float b, int old, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

}  // namespace sage2
