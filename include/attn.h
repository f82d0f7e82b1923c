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
  ATTN_ERR_LAUNCH = 7,   /* the HIP runtime refused the launch or the device query */
  ATTN_ERR_WORKSPACE = 8 /* attn_fwd_split: workspace smaller than required         */
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
 * keeps no pointer after returning, and holds no state between calls (at
 * d = 64 the launch reads the current device's compute-unit count, which it
 * caches); calls may be made from any thread, and calls on different streams
 * may overlap. The call only enqueues work: results are valid once `stream`
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

/*
 * attn_fwd_split - the same result as attn_fwd, computed over n_splits
 * contiguous chunks of the keys (each a multiple of 64 keys; at most one chunk
 * per 64 keys is used) that run as independent workgroups, followed by a merge
 * of the chunks' partial results.
 *
 * Why: the news.hamidun.com glossary entry "Flash attention" (fourth
 * paragraph) names inference frameworks and Ring Attention, which partitions
 * the method's work over keys; with few query rows per (b, h) the plain launch
 * has fewer workgroups than the device has compute units, and splitting the
 * keys fills it. The merge follows from the softmax definition (onecalc.app
 * "Attention memory", section "What this memory is"): for chunk results O_z
 * with log-sum-exps lse_z, lse = ln sum_z exp(lse_z) and
 * O = sum_z exp(lse_z - lse) O_z.
 *
 * Arguments: as attn_fwd, plus
 *   n_splits         requested number of key chunks, 1 .. 65535 (1, or a
 *                    problem with a single 64-key tile, runs attn_fwd and
 *                    needs no workspace)
 *   workspace        caller-owned device memory, 256-byte aligned, of at least
 *                    attn_fwd_split_workspace_bytes(B, H, s_q, d, chunks)
 *                    bytes, chunks = min(n_splits, ceil(s_k / 64)); it holds
 *                    the float32 partial outputs [chunk][B*H][s_q][d] and
 *                    log-sum-exps [chunk][B*H][s_q]; its contents on entry are
 *                    ignored and on return are unspecified
 *   workspace_bytes  its size in bytes
 *
 * The library allocates nothing; two kernels are enqueued on `stream`, and
 * concurrent calls must not share a workspace. Additional statuses:
 * ATTN_ERR_SHAPE for n_splits out of range, ATTN_ERR_NULL for a missing
 * workspace, ATTN_ERR_ALIGN for a misaligned one, ATTN_ERR_WORKSPACE when it
 * is too small, ATTN_ERR_ALIAS when it overlaps a tensor argument.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* out, float* lse,
                   int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d,
                   float scale, int causal, const uint8_t* key_padding_mask,
                   int64_t n_splits, void* workspace, int64_t workspace_bytes, void* stream);

/* Size of the fixed device array attn_fwd_split_noalloc keeps its partial
 * results in (64 MiB; one copy per device). */
#define ATTN_SPLIT_SCRATCH_BYTES (64ll << 20)

/*
 * attn_fwd_split_noalloc - attn_fwd_split for callers that cannot allocate
 * device memory or hold a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the chunks' partial
 * results go to a fixed device array of ATTN_SPLIT_SCRATCH_BYTES bytes that
 * the library holds on each device it runs on until the process ends.
 *
 * Arguments: as attn_fwd_split without the workspace. The result is that of
 * attn_fwd_split with the same arguments (the same kernels run).
 *
 * Limit: attn_fwd_split_workspace_bytes(B, H, s_q, d, chunks) must not exceed
 * ATTN_SPLIT_SCRATCH_BYTES, chunks = min(n_splits, ceil(s_k / 64));
 * larger problems get ATTN_ERR_WORKSPACE before any HIP call (attn_fwd_split
 * with a workspace serves them). A call that uses one chunk runs attn_fwd and
 * does not touch the array.
 *
 * The library allocates nothing here. On the first call on a device it looks
 * up that device's copy of the array (hipGetSymbolAddress, with the device
 * current; ATTN_ERR_LAUNCH if that fails). Every call on a device shares its
 * array, and nothing in it needs clearing between calls (each call writes all
 * it reads). Calls that may run at the same time on one device (on different
 * streams, or from different threads) race on the array and give undefined
 * results: serialise them, or use attn_fwd_split with separate workspaces.
 * Other statuses as attn_fwd_split.
 */
int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                           int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d,
                           float scale, int causal, const uint8_t* key_padding_mask,
                           int64_t n_splits, void* stream);

/*
 * attn_fwd_split_workspace_bytes - workspace bytes attn_fwd_split needs for
 * `n_splits` chunks (0 when n_splits == 1); -1 for invalid sizes (negative
 * sizes, d not 64 or 128, n_splits outside 1 .. 65535). Host-only.
 */
int64_t attn_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t s_q, int64_t d,
                                       int64_t n_splits);

/*
 * attn_bwd - enqueue the backward pass of attn_fwd on `stream`: the gradients
 * of O with respect to q, k and v for a given gradient dO of the output.
 *
 * The onecalc.app page "Attention memory" (section "What this memory is")
 * notes that training frameworks keep the materialised score matrix for the
 * backward pass unless a fused kernel does without it; this one does: the
 * weights are rebuilt tile by tile from the forward pass's log-sum-exp,
 * P = exp(scale q.k - lse), and nothing of size s_q x s_k is stored. The
 * gradients are the chain rule through the definition (the pages give no
 * formulas): dV = P^T dO, dP = dO V^T, D_i = dO_i . O_i,
 * dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 *
 * Arguments (caller-owned DEVICE memory, dense row-major):
 *   q, k, v, causal, key_padding_mask, scale, B, H, s_q, s_k, d
 *                     as given to attn_fwd
 *   out    bf16 [B, H, s_q, d]  attn_fwd's output for these inputs
 *   dout   bf16 [B, H, s_q, d]  gradient of the loss with respect to out
 *   lse    f32  [B, H, s_q]     attn_fwd's log-sum-exp for these inputs
 *                               (-inf marks a row with no visible key)
 *   dq     bf16 [B, H, s_q, d]  written
 *   dk, dv bf16 [B, H, s_k, d]  written (zero for keys no query sees)
 *   workspace        caller-owned device memory, 256-byte aligned, of at
 *                    least attn_bwd_workspace_bytes(B, H, s_q) bytes (it
 *                    holds D = rowsum(dO * O) and lse * log2(e), float32,
 *                    each [B, H, s_q rounded up to 128]); contents on entry
 *                    are ignored and on return unspecified
 *   workspace_bytes  its size
 *   stream           a hipStream_t (NULL = the default stream)
 *
 * Two kernels run in order on `stream` (dq and D, then dk and dv); the library
 * allocates nothing, and concurrent calls must not share a workspace.
 * Returns ATTN_OK or: ATTN_ERR_NULL (a required pointer is NULL),
 * ATTN_ERR_SHAPE, ATTN_ERR_HEAD_DIM, ATTN_ERR_SCALE (as attn_fwd),
 * ATTN_ERR_ALIGN (a bf16 tensor not 16-byte aligned, lse not 4-byte, the
 * workspace not 256-byte), ATTN_ERR_WORKSPACE (workspace too small),
 * ATTN_ERR_ALIAS (an output overlaps an input or another output),
 * ATTN_ERR_LAUNCH.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d,
             float scale, int causal, const uint8_t* key_padding_mask,
             void* workspace, int64_t workspace_bytes, void* stream);

/* attn_bwd_workspace_bytes - workspace bytes attn_bwd needs:
 * 2 * B * H * (s_q rounded up to 128) * 4, rounded up to 256 (-1 for negative
 * sizes). Host-only. */
int64_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t s_q);

/*
 * attn_fwd_fp8 - enqueue the attention forward pass over 8-bit floating-point
 * inputs on `stream`.
 *
 * The news.hamidun.com glossary entry "Flash attention" (second paragraph)
 * names FP8 precision as the method's third version's addition. The inputs
 * are OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * largest finite magnitude 448, NaN = 0x7F / 0xFF), one code per byte; the
 * real value of a code is descale[b*H + h] times its E4M3 value. The result
 * is the attention operation of attn_fwd on those real values:
 *
 *     O[b,h,i,:] = sum_j softmax_j( scale * dq * dk * q8[b,h,i,:].k8[b,h,j,:] + mask ) dv * v8[b,h,j,:]
 *
 * with dq = descale_q[b*H + h] and so on. Both products run on the 8-bit
 * matrix cores with float32 accumulation; the softmax weights, each at most
 * 256 against a running reference max, are rounded to E4M3 (relative error
 * at most 2^-4, or 2^-10 absolute below 2^-6) before the value product; the
 * row max, row sums and the output accumulator are float32.
 *
 * Arguments: as attn_fwd, except
 *   q, k, v    uint8 E4M3 codes [B, H, s, d], 16-byte aligned
 *   descale_q, descale_k, descale_v
 *              NULL (every factor 1) or device float32 [B*H], 4-byte
 *              aligned, finite; any sign (a negative scale * dq * dk is
 *              handled like a negative scale in attn_fwd)
 *   out        bf16 [B, H, s_q, d]; lse float32 [B, H, s_q]:
 *              lse = ln sum_j exp(scale * dq * dk * q8.k8_j) over visible keys
 *
 * Statuses, ownership and synchrony as attn_fwd (ATTN_ERR_ALIGN also covers
 * the descale arrays, ATTN_ERR_ALIAS an out or lse overlapping them). Input
 * codes 0x7F / 0xFF (NaN) give NaN results.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, const float* descale_q,
                 const float* descale_k, const float* descale_v, void* out, float* lse,
                 int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale,
                 int causal, const uint8_t* key_padding_mask, void* stream);

/* attn_fwd_fp8_validate - the host-side checks of attn_fwd_fp8 (same
 * arguments, no stream); no launch, no HIP runtime call. */
int attn_fwd_fp8_validate(const void* q, const void* k, const void* v, const float* descale_q,
                          const float* descale_k, const float* descale_v, const void* out,
                          const float* lse, int64_t B, int64_t H, int64_t s_q, int64_t s_k,
                          int64_t d, float scale, int causal, const uint8_t* key_padding_mask);

/*
 * attn_fwd_unfused - the same operation as attn_fwd, computed the
 * materialising way the fused kernel avoids: the score matrix of every
 * (batch item, head) is written to device memory, turned into weights in
 * place, and multiplied by the values. It exists to measure that path.
 *
 * The onecalc.app page "Attention memory" sizes the matrix ("The formula",
 * "Worked example"): B * H * s_q * s_k elements of e = 2 bytes (16-bit
 * scores), 1.07 GB at B = 1, H = 32, s = 4096 and 4.29 GB at s = 8192. The
 * hyper.ai story on PyTorch's attention backends reports the plain backend
 * that stores it as several times slower than the fused ones.
 *
 * Three kernels run in order on `stream`:
 *   1. scores[b,h,i,j] = bf16(scale * q[b,h,i,:].k[b,h,j,:]) (no masks);
 *   2. in place, per row: hidden keys (causal j > i, padded keys) get weight
 *      0, the others softmax of the stored scores, rounded to bf16;
 *      lse[b,h,i] = max + ln(sum exp(s - max)) over the visible stored scores
 *      (-inf and an all-zero row when no key is visible);
 *   3. out[b,h,i,:] = bf16(sum_j scores[b,h,i,j] * v[b,h,j,:]) (float32 sums).
 * The rounding of the scores to bf16 makes the result differ from attn_fwd's
 * by more than rounding of the output: each weight may move by a factor up
 * to exp(+-2^-7 max|score|).
 *
 * Arguments: as attn_fwd, plus
 *   scores        caller-owned device memory, 16-byte aligned, of at least
 *                 attn_fwd_unfused_workspace_bytes(B, H, s_q, s_k) bytes; on
 *                 return it holds the weights, bf16 [B, H, s_q, s_k]
 *                 (row-major); may be NULL when that size is 0
 *   scores_bytes  its size
 * Statuses as attn_fwd, and ATTN_ERR_NULL / ATTN_ERR_ALIGN /
 * ATTN_ERR_WORKSPACE / ATTN_ERR_ALIAS for a missing, misaligned, short or
 * overlapping scores buffer, ATTN_ERR_SHAPE when its size overflows 64 bits
 * or a grid does not fit. The library allocates nothing.
 */
int attn_fwd_unfused(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale,
                     int causal, const uint8_t* key_padding_mask, void* scores,
                     int64_t scores_bytes, void* stream);

/* attn_fwd_unfused_workspace_bytes - bytes of the score matrix attn_fwd_unfused
 * needs: B * H * s_q * s_k * 2 (0 when any size is 0; -1 for negative sizes
 * or a product beyond 64 bits). Host-only. */
int64_t attn_fwd_unfused_workspace_bytes(int64_t B, int64_t H, int64_t s_q, int64_t s_k);

/* attn_status_str - a static, human-readable name for a status code. */
const char* attn_status_str(int status);

/* attn_last_hip_error - the hipError_t value behind the calling thread's last
 * ATTN_ERR_LAUNCH (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_44_AMD_ATTN_H */
