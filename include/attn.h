/*
 * attn.h -- C ABI of the fused exact-attention forward for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes, in one kernel launch,
 *
 *     O   = softmax(scale * Q K^T + M) V
 *     LSE = log of the softmax denominator (natural log, scaled scores)
 *
 * without writing the score matrix to device memory.  The formula with a mask
 * matrix M is the one in "MiniPaged-Qwen: Qwen3 prefill FlashAttention",
 * section 1; the tiled evaluation with a running max, a running denominator
 * and an unnormalised accumulator is that page's section 4 (online softmax) and
 * the "Online Softmax" section of "FlashAttention personal implementation
 * notes".
 *
 * Conventions
 *   Layout    q, o: (B, Sq, Hq, d); k, v: (B, Sk, Hkv, d); dense, d contiguous,
 *             the (batch, seq, heads, d_head) layout of the personal-notes
 *             page's opening section.  lse: fp32, (B, Hq, Sq), contiguous.
 *   GQA       query head h reads kv head h / (Hq / Hkv) (Qwen3-prefill page,
 *             section 6).
 *   Causal    bottom-right aligned: query i sees key j iff j <= i + (Sk - Sq)
 *             (Qwen3-prefill page, section 13).  Rows that see no key
 *             (i < Sq - Sk) get O = 0 and LSE = -inf.
 *   Precision q, k, v, o are all fp16 or all bf16; products accumulate in
 *             fp32; the probabilities are rounded to the input type before the
 *             P V product, as on every page; O is rounded to nearest even.
 *
 * Ownership and synchronisation
 *   The caller owns every buffer.  The library allocates nothing, keeps no
 *   state between calls and never synchronises: the work is queued on
 *   `stream` and the call returns.  It does not read o or lse; on success
 *   every element of o (and of lse if given) is written.
 *
 * Errors
 *   A nonzero status means nothing was launched and nothing was written,
 *   except ATTN_ERR_LAUNCH, which reports a failure that HIP signalled at or
 *   after the launch.
 */
#ifndef EXACT_ATTENTION_19_AMD_ATTN_H
#define EXACT_ATTENTION_19_AMD_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, size < 1, Hq % Hkv != 0, bad
                               scale, causal not 0/1, misaligned pointer,
                               index space too large */
  ATTN_ERR_UNSUPPORTED = 2, /* d or dtype outside the built set */
  ATTN_ERR_LAUNCH = 3       /* HIP reported an error for the launch */
} attn_status;

typedef enum { ATTN_DTYPE_F16 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype;

#define ATTN_ABI_VERSION 1

/*
 * attn_fwd -- fused attention forward.
 *
 *   q      device pointer, (B, Sq, Hq, d) elements of `dtype`, 16-byte aligned
 *   k, v   device pointers, (B, Sk, Hkv, d), 16-byte aligned
 *   o      device pointer, (B, Sq, Hq, d), 16-byte aligned; written
 *   lse    device pointer to B*Hq*Sq floats, 4-byte aligned, or NULL to skip
 *   B, Sq, Sk, Hq, Hkv, d   sizes, all >= 1; Hq must be a multiple of Hkv;
 *          d must be 64 or 128
 *   scale  multiplier of the scores, finite and > 0 (1/sqrt(d) is usual)
 *   causal 0 = no mask, 1 = bottom-right causal mask
 *   dtype  an attn_dtype value
 *   stream hipStream_t to launch on (NULL = the default stream), passed as a
 *          plain pointer
 *
 * Returns ATTN_OK when the kernel was queued.  Size limits: Sq + Sk < 2^30,
 * B * Sq * Hq < 2^31 and B * Sk * Hkv < 2^31 (rows of each tensor); larger
 * problems are rejected with ATTN_ERR_INVALID_ARG rather than risking index
 * overflow.  attn_fwd_check reports the same status without a device call.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int d,
                     float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd_check -- the argument validation of attn_fwd without any device
 * call: returns the status attn_fwd would return before launching.  Safe on a
 * machine without a GPU.
 */
attn_status attn_fwd_check(const void* q, const void* k, const void* v,
                           void* o, float* lse, int B, int Sq, int Sk, int Hq,
                           int Hkv, int d, float scale, int causal, int dtype);

/*
 * attn_fwd_plan -- describe the launch attn_fwd would make for these sizes,
 * without any device call.  Writes up to n (at most 9) ints into `out`:
 *   [0] workgroups in the grid   [1] threads per workgroup
 *   [2] query rows per workgroup [3] keys per K/V tile
 *   [4] query heads per workgroup (GQA packing)
 *   [5] query rows per wave      [6] LDS bytes per workgroup
 *   [7] 1 if the grid is ordered per XCD, else 0
 *   [8] 1 if the software-pipelined kernel (the softmax of one K/V tile
 *       overlapping the matrix products of the previous and next tiles) is
 *       used
 * Returns the status attn_fwd_check would return.
 */
attn_status attn_fwd_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d,
                          int causal, int dtype, int* out, int n);

/* Human-readable name of a status code (static string). */
const char* attn_status_str(int status);

/* ATTN_ABI_VERSION of the library that was loaded. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_19_AMD_ATTN_H */
