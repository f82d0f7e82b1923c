/*
 * attn.h - fused scaled-dot-product attention forward for AMD Instinct MI355X
 * (gfx950, CDNA4). C ABI: plain pointers and sizes, no framework types.
 *
 * The operation is the one the onecalc.app page "Attention memory" defines in
 * its sections "The quadratic term" and "What this memory is": for every batch
 * item b and head h, each query row is compared with every key row (scores),
 * a softmax over each row of scores gives weights, and the output row is the
 * weighted sum of the value rows:
 *
 *     O[b,h,i,:] = sum_j softmax_j( scale * q[b,h,i,:].k[b,h,j,:] + mask[b,i,j] ) v[b,h,j,:]
 *
 * It is computed the way the page's "FlashAttention" section and the
 * news.hamidun.com glossary entry "Flash attention" (second paragraph)
 * describe: keys and values are visited block by block with a running row max
 * and row sum, so the s_q x s_k score matrix (B*H*s^2*e bytes, section "The
 * formula") is never written to device memory. The result equals the
 * materialising definition up to floating-point rounding (the glossary entry's
 * first paragraph).
 */
#ifndef EXACT_ATTENTION_44_AMD_ATTN_H
#define EXACT_ATTENTION_44_AMD_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Every code except ATTN_ERR_LAUNCH is decided on the host,
 * before any HIP runtime call, so a rejected call has no device side effects. */
typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,     /* a required pointer is NULL                              */
  ATTN_ERR_SHAPE = 2,    /* a size is negative or too large for the kernel's grid   */
  ATTN_ERR_HEAD_DIM = 3, /* d is not 64 or 128                                      */
  ATTN_ERR_ALIGN = 4,    /* q, k, v, out not 16-byte aligned, or lse not 4-byte     */
  ATTN_ERR_ALIAS = 5,    /* out or lse overlaps an input, or out overlaps lse       */
  ATTN_ERR_SCALE = 6,    /* scale is NaN or infinite                                */
  ATTN_ERR_LAUNCH = 7    /* the HIP runtime refused the kernel launch               */
} attn_status;

/*
 * attn_fwd - enqueue the attention forward pass on `stream`.
 *
 * Arguments (all tensors are caller-owned DEVICE memory, dense row-major):
 *   q    bf16 [B, H, s_q, d]   queries
 *   k    bf16 [B, H, s_k, d]   keys
 *   v    bf16 [B, H, s_k, d]   values (value width equals d)
 *   out  bf16 [B, H, s_q, d]   written: the attention output, rounded to bf16
 *   lse  f32  [B, H, s_q]      written: natural-log log-sum-exp of row i's
 *                              scaled, masked scores, lse = max + ln(sum exp(s - max))
 *   B, H, s_q, s_k             sizes; any may be 0 (nothing is computed when
 *                              B*H*s_q == 0; with s_k == 0 every row is empty)
 *   d                          head dimension, 64 or 128
 *   scale                      multiplies q.k before the softmax (callers
 *                              usually pass 1/sqrt(d)); any finite value,
 *                              including 0 and negative values
 *   causal                     nonzero: key j is hidden from query i when j > i
 *                              (top-left alignment, also when s_q != s_k)
 *   key_padding_mask           NULL, or device uint8 [B, s_k]: a nonzero byte
 *                              hides key j of batch item b from every query
 *                              and head; combines with `causal` by union
 *   stream                     a hipStream_t (NULL = the default stream)
 *
 * A row with no visible key (all padded, or s_k == 0) gets out = 0 and
 * lse = -inf. Results are finite whenever |scale * q.k| and the value rows
 * are well inside the float32 range.
 *
 * Ownership and synchrony: the library allocates no device or host memory,
 * keeps no pointer after returning, and holds no state; calls may be made from
 * any thread. The call only enqueues work: results are valid once `stream`
 * has been synchronised. Faults inside the kernel surface through the HIP
 * runtime at synchronisation, not through this return value.
 *
 * Returns ATTN_OK or one of the attn_status codes above.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d,
             float scale, int causal, const uint8_t* key_padding_mask, void* stream);

/*
 * attn_fwd_validate - the host-side checks of attn_fwd (same arguments,
 * no stream), without launching anything and without calling the HIP runtime.
 * Returns the status attn_fwd would return before its launch step.
 */
int attn_fwd_validate(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, int64_t B, int64_t H, int64_t s_q, int64_t s_k,
                      int64_t d, float scale, int causal, const uint8_t* key_padding_mask);

/* attn_status_str - a static, human-readable name for a status code. */
const char* attn_status_str(int status);

/* attn_last_hip_error - the hipError_t value behind the calling thread's last
 * ATTN_ERR_LAUNCH (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_44_AMD_ATTN_H */
