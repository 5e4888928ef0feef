/* sage2.h — C ABI of the MI355X (gfx950) SageAttention2 forward pass.
 *
 * What is computed (PMLR vol. 267 page "SageAttention2: Efficient Attention with Thorough Outlier
 * Smoothing and Per-thread INT4 Quantization", Abstract; research record of the same title,
 * "Three components"): dense softmax attention O = softmax(sm_scale * Q K^T) V, evaluated with
 *   - K smoothing: K minus its per-channel token mean (visual companion "SageAttention2 and Fast
 *     Exact INT4 Attention", section "Channel Outlier Smoothing");
 *   - Q smoothing: Q minus the mean of each 128-token block, with the block mean's exact
 *     contribution (mean . smoothed key) added back into the logits;
 *   - INT4 Q and K at thread granularity: one scale per query token and one per 16-key group, the
 *     keys that one half of a 64-lane wave owns in a 32x32 MFMA output tile (section "Per-Thread
 *     INT4 Geometry" gives thread-owned scale groups; this is their gfx950 form);
 *   - INT32-exact QK^T, dequantization and an online softmax;
 *   - P~ and V in FP8 (OCP e4m3), P~V on FP8 MFMA with a two-level accumulation: each short MFMA
 *     run is folded into an FP32 buffer (section "Numerical Repair Stack": periodic FP32 foldback).
 * The interface envelope (variable lengths, grouped-query heads, q/kv lengths that differ, head dims
 * up to 128 padded to 64 or 128, larger rejected) follows section "Implementation envelope" of the
 * visual companion. Here a head dim d is any multiple of 8 in [8, 128]; it is padded with zero
 * channels to 64 (d <= 64) or 128 inside the workspace, which changes no code, scale, mean or
 * correction value, and the default softmax scale uses the true d.
 *
 * Two calls do the work: sage2_quantize_smooth (the pre-pass: smoothing statistics, INT4/FP8 codes,
 * scales, correction table, written into a caller-provided workspace) and sage2_attn_fwd (the
 * attention kernel, reading only the workspace). A workspace may serve any number of attn_fwd calls
 * made with the same parameters.
 *
 * Conventions for every call:
 *   - Pointers named "device" are HIP device addresses; "host" pointers are CPU memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). All device work is
 *     enqueued on it; no call synchronizes, allocates or frees memory, or keeps a pointer after it
 *     returns. There are no host callbacks, so calls may be captured in a HIP graph.
 *   - Arguments are checked on the host before anything is enqueued; on an error nothing is
 *     enqueued. A failed launch returns SAGE2_ERR_HIP. Faults during execution surface at the
 *     caller's next synchronization.
 *   - NaN or Inf inputs give unspecified outputs (but no out-of-bounds access).
 *   - The library has no mutable global state and may be called from several threads.
 */
#ifndef SAGE2_H
#define SAGE2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE2_OK = 0,
  SAGE2_ERR_NULL = 1,         /* a required pointer is NULL */
  SAGE2_ERR_SHAPE = 2,        /* bad sizes: B/H/N <= 0, H_q % H_kv != 0, bad cu_seqlens, a workspace
                               * whose per-head extents pass 2^31 - 1 rows or correction entries, ... */
  SAGE2_ERR_UNSUPPORTED = 3,  /* head dim not a multiple of 8 in [8, 128], unknown dtype or flag, ... */
  SAGE2_ERR_ALIGN = 4,        /* pointer or stride not 16-byte aligned; workspace not 256-byte aligned */
  SAGE2_ERR_WORKSPACE = 5,    /* ws_bytes smaller than sage2_workspace_size() */
  SAGE2_ERR_HIP = 6           /* a kernel launch failed */
} sage2_status;

typedef enum { SAGE2_F16 = 0, SAGE2_BF16 = 1, SAGE2_F32 = 2 } sage2_dtype;

/* Ablations of the method's smoothing and scale granularity (research record, "Three components";
 * visual companion, "Channel Outlier Smoothing" and "Per-Thread INT4 Geometry"), for measuring what
 * each one buys. 0 is the full method. */
typedef enum {
  SAGE2_NO_K_SMOOTH = 1,      /* quantize K without subtracting its channel means (k-bar = 0) */
  SAGE2_NO_Q_SMOOTH = 2,      /* quantize Q without its block means (q-bar = 0, so the correction is 0) */
  SAGE2_PER_BLOCK_SCALES = 4, /* one INT4 scale per 128-token Q block and per 64-key K block instead of
                               * the per-thread groups (section "Per-Thread INT4 Geometry" contrasts
                               * the two); the attention kernel is unchanged */
  SAGE2_NO_FP32_FOLD = 8      /* single-level P~V accumulation: the output accumulates across key tiles
                               * inside the FP8 MFMA instead of being folded into FP32 once per tile
                               * (research record, "Three components": FP8 accumulation loses
                               * accuracy). Its result depends on the MFMA's inexact accumulation and
                               * is not reproduced by the CPU oracle */
} sage2_flag;

typedef struct {
  /* Sizes. Dense batch: B sequences of N_q queries and N_kv keys each.
   * Variable length (cu_seqlens set): B sequences packed along the token axis; N_q / N_kv are upper
   * bounds on the per-sequence lengths (used only to size the launch grids). */
  int32_t B, H_q, H_kv, N_q, N_kv, d;
  /* 0 or 1. Causal masks are aligned bottom-right: key j is visible from query i when
   * j <= i + (L_kv - L_q) within a sequence; a row that sees no key outputs zeros. */
  int32_t causal;
  int32_t in_dtype;   /* sage2_dtype of q, k, v: SAGE2_F16 or SAGE2_BF16 */
  int32_t out_dtype;  /* sage2_dtype of o: SAGE2_F16, SAGE2_BF16 or SAGE2_F32 */
  float sm_scale;     /* softmax scale; 0 selects 1/sqrt(d) */
  /* Variable-length batches: cumulative token offsets, B+1 entries, first 0, non-decreasing.
   * Set all four or none. The device copies are read by the kernels, the host copies size the
   * workspace and are validated; both must hold the same values. Sequences may be empty. */
  const int32_t* cu_seqlens_q;        /* device */
  const int32_t* cu_seqlens_kv;       /* device */
  const int32_t* cu_seqlens_q_host;   /* host */
  const int32_t* cu_seqlens_kv_host;  /* host */
  /* Element strides of q, k, v, o: [0] batch, [1] token, [2] head; the channel stride is 1.
   * Dense [B, N, H, d] and [B, H, N, d] layouts are both expressed this way. In variable-length
   * mode the tensors are packed [total_tokens, H, d] and the batch stride is ignored.
   * Strides times the element size must be multiples of 16 bytes. */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  int32_t flags;  /* OR of sage2_flag values; 0 = the full method */
} sage2_params;

/* Byte offsets (from the workspace base) and byte sizes of the workspace buffers, for tests that
 * decode the pre-pass outputs. Row counts are padded per sequence: Q rows to a multiple of 128,
 * K/V rows to a multiple of 128. Layouts (head-major; "row" = padded token slot):
 *   seq_table  int32 [B][8]: q_start, q_len, kv_start, kv_len, q_row0, kv_row0, qblk0, delta0;
 *                                             written for variable-length batches only (without
 *                                             cu_seqlens sequence b has q_len N_q, kv_len N_kv,
 *                                             starts 0 and the offsets of b full sequences)
 *   k_partial  f64   [H_kv][kv_rows/128][d]   per-128-token fp64 sums of K
 *   v_partial  f32   [H_kv][kv_rows/128][d]   per-128-token max |V|
 *   kbar       f32   [B][H_kv][d]             K channel means
 *   sv, sv_inv f32   [B][H_kv][d]             V channel scale amax/448 and its inverse 448/amax
 *   qbar       f32   [H_q][q_blocks][d]       Q block means; within each 8-channel group channel
 *                                             c sits at 4*(c%2) + (c%8)/2 (the order in which the
 *                                             correction MFMA consumes them)
 *   qcode      u8    [H_q][q_rows][3d/4]      INT4 codes in 6-bit e2m3 fields (the gfx950 fp6
 *                                             MFMA operand format, exact for -7..7): channel c at
 *                                             bits [6c, 6c+6) of the row, little-endian
 *   sq         f32   [H_q][q_rows]            per-token Q scale
 *   kcode      u8    [H_kv][kv_rows][3d/4]    INT4 codes, same encoding
 *   sk         f32   [H_kv][kv_rows/16]       K scale of group 2*(j/32) + bit 2 of j
 *   v8         u8    [H_kv][kv_rows/64][d][2][32]  FP8 e4m3 codes of V*sv_inv; within a 64-key
 *                                             tile, channel c, half h, slot s holds key
 *                                             32*(s/16) + 8*((s%16)/4) + 4*h + s%4
 *   delta      f32   [H_q][delta_len]         correction (qbar . smoothed k_j) * sm_scale * log2(e),
 *                                             per sequence one row per Q block from delta0: all
 *                                             kv_rows keys without a causal mask; with one, row qb
 *                                             holds keys [0, V(qb)), V(qb) = the block's last
 *                                             visible key + 1 rounded up to 128 (the last block:
 *                                             all kv_rows), rows back to back; entries of keys the
 *                                             mask hides from every row of the block are unspecified
 */
typedef struct {
  int64_t total_bytes;
  int64_t q_rows, kv_rows, q_blocks, delta_len;  /* per head, summed over sequences */
  int64_t seq_table, k_partial, v_partial, kbar, sv, sv_inv, qbar, qcode, sq, kcode, sk, v8,
      delta;
} sage2_ws_layout;

/* Workspace bytes needed for `p` (validates p first; the same checks as every call below).
 * `bytes` is host memory. The workspace holds what the pre-pass produces (see sage2_ws_layout);
 * its size follows from the envelope of visual companion "SageAttention2 and Fast Exact INT4
 * Attention", section "Implementation envelope" (variable lengths, grouped heads, padded head
 * dims). Errors: SAGE2_ERR_NULL for a null p or bytes, otherwise as the parameter checks. */
sage2_status sage2_workspace_size(const sage2_params* p, size_t* bytes);

/* Pre-pass (PMLR vol. 267 page "SageAttention2: Efficient Attention with Thorough Outlier
 * Smoothing and Per-thread INT4 Quantization", Abstract: Q and K to INT4 at thread granularity, P~
 * and V to FP8, Q smoothed; research record of the same title, "Three components" (1) and (2);
 * visual companion, "Channel Outlier Smoothing"): K channel means over the sequence, Q means per
 * 128-token block, INT4 codes of K - mean (one scale per 16-key group) and Q - block mean (one
 * scale per token), FP8 codes of V with one scale per channel, and the correction table
 * (block mean . smoothed key) in base-2 logit units.
 * q, k, v: device, in_dtype, layout per the strides; read only. ws: device, 256-byte aligned,
 * ws_bytes >= sage2_workspace_size(p); every buffer of the layout in use is overwritten (nothing
 * in it needs to be initialised). Errors: SAGE2_ERR_NULL (p, q, k, v or ws null), SAGE2_ERR_ALIGN,
 * SAGE2_ERR_WORKSPACE, the parameter checks, SAGE2_ERR_HIP if a launch fails; on an error before
 * the launches nothing is enqueued. */
sage2_status sage2_quantize_smooth(const sage2_params* p, const void* q, const void* k,
                                   const void* v, void* ws, size_t ws_bytes, void* stream);

/* Attention (PMLR vol. 267 page, Abstract: INT4 QK^T, FP8 P~V, two-level accumulation; research
 * record, "Three components" (3); visual companion, "Numerical Repair Stack": exact INT4
 * fragments, FP8 value mixing, periodic FP32 foldback): exact INT32 QK^T of the INT4 codes,
 * dequantization with the per-token and per-group scales plus the correction term, online softmax
 * in base 2 over 128-key tiles, P~ = e4m3 of the weights scaled so the row max maps to 448, P~V
 * on the FP8 MFMA accumulated per tile and folded into FP32, division by the row sum and the V
 * channel scale. ws: a workspace filled by sage2_quantize_smooth with the same p (read only; it
 * may serve any number of calls). o: device, out_dtype, layout per o_stride; every valid
 * (token, head) row is written, rows that see no key as zeros. Errors: SAGE2_ERR_NULL (p, ws or
 * o null), SAGE2_ERR_ALIGN, SAGE2_ERR_WORKSPACE, the parameter checks, SAGE2_ERR_HIP if the
 * launch fails. */
sage2_status sage2_attn_fwd(const sage2_params* p, const void* ws, size_t ws_bytes, void* o,
                            void* stream);

/* Static English text for a status code (never NULL). */
const char* sage2_status_string(sage2_status s);

/* ---- test-only exports ------------------------------------------------------------------------ */

/* Workspace layout of p (host struct `out`), for tests that decode the pre-pass outputs into the
 * canonical arrays of the method's steps. Errors: SAGE2_ERR_NULL, the parameter checks. */
sage2_status sage2_workspace_layout(const sage2_params* p, sage2_ws_layout* out);

/* The attention kernel itself (sage2_attn_fwd's kernel, two-level form), additionally writing for
 * query rows [q_begin, q_begin + q_count) of every sequence and q head what its tiles compute:
 *   s_out  (device, may be NULL) int32 [B][H_q][q_count][N_kv]: the exact INT32 Q K^T of the INT4
 *          codes, taken from the same LDS-staged operands and MFMAs that feed the softmax (abstract:
 *          INT4 Q K^T; visual companion, "Numerical Repair Stack": exact INT4 fragments);
 *   p8_out (device, may be NULL) uint8 [B][H_q][q_count][N_kv]: the e4m3 code of P~ that the kernel
 *          feeds to its P~V MFMA for each key (abstract: P~ to FP8); 0 for masked keys.
 * Only the key tiles a row's wave visits are written (under a causal mask, tiles past the wave's last
 * visible key are skipped); other entries, and entries past a sequence's lengths, are left as they
 * were. o (device, may be NULL): the output as sage2_attn_fwd writes it, or nothing when NULL.
 * At least one of s_out and p8_out must be given; SAGE2_NO_FP32_FOLD is rejected. */
sage2_status sage2_debug_attn_tiles(const sage2_params* p, const void* ws, size_t ws_bytes,
                                    int32_t q_begin, int32_t q_count, int32_t* s_out,
                                    uint8_t* p8_out, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE2_H */
