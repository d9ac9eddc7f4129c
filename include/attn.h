/*
 * attn.h -- C ABI of the fused exact-attention forward for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes (attn_fwd: in one kernel launch)
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
 *   The caller owns every buffer (attn_fwd_split's workspace included).  The
 *   library allocates nothing, keeps no state between calls and never
 *   synchronises: the work is queued on `stream` and the call returns.  It
 *   does not read o or lse; on success every element of o (and of lse if
 *   given) is written.
 *
 * Errors
 *   A nonzero status means nothing was launched and nothing was written,
 *   except ATTN_ERR_LAUNCH, which reports a failure that HIP signalled at or
 *   after the launch.
 */
#ifndef EXACT_ATTENTION_19_AMD_ATTN_H
#define EXACT_ATTENTION_19_AMD_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, size < 1, Hq % Hkv != 0, bad
                               scale, causal not 0/1, misaligned pointer,
                               index space too large */
  ATTN_ERR_UNSUPPORTED = 2, /* d, dtype or (paged decode) shape outside the
                               built set */
  ATTN_ERR_LAUNCH = 3,      /* HIP reported an error for the launch */
  ATTN_ERR_SCRATCH = 4      /* attn_fwd_split_noalloc: the key split would
                               need more than ATTN_SCRATCH_BYTES */
} attn_status;

/* F32 is accepted only for the partial outputs passed to attn_merge. */
typedef enum { ATTN_DTYPE_F16 = 0, ATTN_DTYPE_BF16 = 1, ATTN_DTYPE_F32 = 2 } attn_dtype;

#define ATTN_ABI_VERSION 5

/*
 * attn_fwd -- fused attention forward.
 *
 *   q      device pointer, (B, Sq, Hq, d) elements of `dtype`, 16-byte aligned
 *   k, v   device pointers, (B, Sk, Hkv, d), 16-byte aligned
 *   o      device pointer, (B, Sq, Hq, d), 16-byte aligned; written
 *   lse    device pointer to B*Hq*Sq floats, 4-byte aligned, or NULL to skip
 *   B, Sq, Sk, Hq, Hkv, d   sizes, all >= 1; Hq must be a multiple of Hkv;
 *          d must be a multiple of 8 from 8 to 256; sizes other than 32,
 *          64, 96, 128, 192 and 256 run on the kernel of the next of these
 *          (the CuTe DSL Ampere FlashAttention-2 example's head-size
 *          padding, "__init__" and "can_implement"): the columns past d are
 *          loaded as zeros and never written
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
 *
 * Value range: the bf16 kernels up to d = 128 move the running row max only
 * when a tile's probabilities against it overshoot 2^40 (the personal-notes
 * page's online softmax, section "Online Softmax", with a stale max), so
 * their unnormalised sums reach 2^35 * Sk * max|V|: inputs with
 * Sk * max|V| >= 2^93 are outside the domain.  NaN or Inf inputs give
 * undefined results.
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
 * without any device call.  Writes up to n (at most 11) ints into `out`:
 *   [0] workgroups in the grid   [1] threads per workgroup
 *   [2] query rows per workgroup [3] keys per K/V tile
 *   [4] query heads per workgroup (GQA packing)
 *   [5] query rows per wave      [6] LDS bytes per workgroup
 *   [7] 1 if the grid is ordered per XCD, else 0
 *   [8] 1 if the software-pipelined kernel (the softmax of one K/V tile
 *       overlapping the matrix products of the previous and next tiles) is
 *       used
 *   [9] 1 if the decode kernel is used: when the query rows of a kv head
 *       (Hq / Hkv * Sq) number at most 32 (or 128 with Sq <= 8), each group
 *       of up to 32 of them shares one wave and the 4 waves of a workgroup
 *       split the keys (then [0] counts a workgroup per (batch, kv head,
 *       32-row group), [2] is Sq and [4] the GQA group size)
 *   [10] 1 if the waves take key halves: two waves take the same 32 query
 *       rows, one the first and one the second 32 keys of every tile, and
 *       their two partial states are merged in the workgroup.  With 4 waves
 *       (rows per workgroup halve, workgroups double) when the plain grid
 *       would leave most CUs with one workgroup, and always for fp16 at
 *       padded head size 256; with 8 waves ([1] = 512, the plain grid) at
 *       padded head size 192, whose tile buffers leave one workgroup per CU
 * Returns the status attn_fwd_check would return.
 */
attn_status attn_fwd_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d,
                          int causal, int dtype, int* out, int n);

/*
 * attn_fwd_split -- attn_fwd for problems whose query blocks are too few to
 * fill the GPU (short sequences, few heads): the keys of each long query
 * block are cut into ranges ("pieces") that separate workgroups process, and
 * the pieces are merged.
 *
 * Each piece produces, per query row, the state of the online softmax over
 * its keys alone ("FlashAttention personal implementation notes", section
 * "Online Softmax": running max, denominator and unnormalised output), kept
 * as an fp32 output normalised over those keys plus their log-sum-exp.  A
 * second kernel combines the pieces of a row with that section's rescale
 * (factor e^(m_i - m_new) on each state), as attn_merge does.  The result is
 * the same attention as attn_fwd's, to within rounding.
 *
 *   q ... dtype  as for attn_fwd (same validation, same status codes)
 *   kv_split     0 = the library's choice: split only when there are fewer
 *                query blocks than the 256 CUs of the device, into the
 *                shortest pieces that still number at most 256 (for decode
 *                shapes, see attn_fwd_plan [9]: only below 128 (batch, kv
 *                head) pairs, into about 128 workgroups of at least 32
 *                32-key tiles);
 *                1 = never split (exactly attn_fwd);
 *                k > 1 = cut the longest query block into at most k pieces
 *                (pieces hold a whole, even number of 64-key tiles)
 *   workspace    device pointer, 256-byte aligned, of at least the size
 *                attn_fwd_split_workspace reports for the same arguments; may
 *                be NULL when that size is 0 (no split).  Owned by the
 *                caller; its contents on entry do not matter and on return
 *                are scratch.  Two calls in flight must not share one.
 *   workspace_bytes  its size in bytes
 *   stream       as for attn_fwd; up to two kernels are queued on it
 *
 * Returns ATTN_ERR_INVALID_ARG for kv_split < 0 or a missing, misaligned or
 * too small workspace, else as attn_fwd.
 */
attn_status attn_fwd_split(const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int Sq, int Sk, int Hq, int Hkv,
                           int d, float scale, int causal, int dtype,
                           int kv_split, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * attn_fwd_split_noalloc -- attn_fwd_split without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory
 * during the call: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * The key split's partial states go to a static device array of
 * ATTN_SCRATCH_BYTES that the library holds on each GPU it runs on, until
 * the process ends.  Its address on a device is looked up (not allocated)
 * at the first call that runs on that device.  The call allocates nothing
 * and calls no hipMalloc or hipFree.
 *
 *   q ... dtype, kv_split, stream  as for attn_fwd_split; the kernels run on
 *          the device of `stream` (the current device for NULL)
 *
 * Every call on one GPU shares that GPU's array: two calls whose kernels
 * overlap on one GPU (different streams with no ordering between them)
 * race and give wrong results.  Calls on one stream are ordered and safe.
 * Nothing in the array needs clearing: each call's merge reads only what
 * the same call wrote.
 *
 * Returns ATTN_ERR_SCRATCH, before any device call, when the split would
 * need more than ATTN_SCRATCH_BYTES (attn_fwd_split_workspace gives the
 * need; kv_split = 1, or a coarser split, needs less or none); else as
 * attn_fwd_split.
 */
#define ATTN_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_fwd_split_noalloc(const void* q, const void* k, const void* v,
                                   void* o, float* lse, int B, int Sq, int Sk,
                                   int Hq, int Hkv, int d, float scale,
                                   int causal, int dtype, int kv_split,
                                   void* stream);

/*
 * attn_fwd_strided -- attn_fwd_split on tensors with arbitrary row strides:
 * any (batch, seq, head) layout with d contiguous, e.g. the (B, H, S, d)
 * layout of the personal-notes and cuTile pages, or q, k, v sliced out of
 * one packed projection output.
 *
 *   strides  12 element strides (not bytes), in the order
 *            q: batch, seq, head;  k: batch, seq, head;
 *            v: batch, seq, head;  o: batch, seq, head.
 *            Element (b, s, h, c) of q is at q + b*qs_b + s*qs_s + h*qs_h + c.
 *            Each stride must be >= 0 and a multiple of 8 (16-byte aligned
 *            rows), and 64 * (k and v seq stride) * 2 < 2^31.  q, k and v
 *            are only read: any strides (0 broadcasts one row).  The rows of
 *            o must not overlap each other: a layout in which they might
 *            (checked by taking the dimensions by increasing stride, each
 *            reaching past all the smaller ones span) is rejected with
 *            ATTN_ERR_INVALID_ARG.  o must not overlap the inputs (not
 *            checked).
 *   lse      as for attn_fwd: contiguous fp32 (B, Hq, Sq) or NULL
 *   kv_split, workspace, workspace_bytes  as for attn_fwd_split (the
 *            workspace size does not depend on the strides)
 *
 * Dense (B, S, H, d) strides give exactly attn_fwd_split's launches.
 */
attn_status attn_fwd_strided(const void* q, const void* k, const void* v,
                             void* o, float* lse, int B, int Sq, int Sk,
                             int Hq, int Hkv, int d, float scale, int causal,
                             int dtype, const long long* strides,
                             int kv_split, void* workspace,
                             size_t workspace_bytes, void* stream);

/* attn_fwd_strided's validation without any device call. */
attn_status attn_fwd_strided_check(const void* q, const void* k, const void* v,
                                   void* o, float* lse, int B, int Sq, int Sk,
                                   int Hq, int Hkv, int d, float scale,
                                   int causal, int dtype,
                                   const long long* strides);

/*
 * attn_fwd_causal_offset -- causal attention with the mask's offset given
 * explicitly: query i sees key j iff j <= i + causal_offset (attn_fwd's
 * causal mode is causal_offset = Sk - Sq).  This is what a shard of the keys
 * of a longer causal problem needs (context parallelism): for keys
 * [k0, k0 + Sk) of a problem with Sk_total keys, causal_offset =
 * Sk_total - Sq - k0, and the shards' outputs and LSEs merge into the full
 * attention with attn_merge (the pages' online-softmax rescale applied to
 * whole parts; "FlashAttention personal implementation notes", section
 * "Online Softmax").  Rows that see no key of the shard get O = 0 and
 * LSE = -inf, which the merge weighs 0.
 *
 *   causal_offset  -2^30 < causal_offset < 2^30
 *   strides        NULL (dense (B, S, H, d)) or as for attn_fwd_strided
 *   the rest       as for attn_fwd_split; the workspace size is
 *                  attn_fwd_causal_offset_workspace's
 */
attn_status attn_fwd_causal_offset(const void* q, const void* k, const void* v,
                                   void* o, float* lse, int B, int Sq, int Sk,
                                   int Hq, int Hkv, int d, float scale,
                                   long long causal_offset, int dtype,
                                   const long long* strides, int kv_split,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

attn_status attn_fwd_causal_offset_check(const void* q, const void* k,
                                         const void* v, void* o, float* lse,
                                         int B, int Sq, int Sk, int Hq, int Hkv,
                                         int d, float scale,
                                         long long causal_offset, int dtype,
                                         const long long* strides);

attn_status attn_fwd_causal_offset_workspace(int B, int Sq, int Sk, int Hq,
                                             int Hkv, int d,
                                             long long causal_offset,
                                             int dtype, int kv_split,
                                             size_t* bytes);

/*
 * attn_fwd_split_workspace -- bytes of workspace attn_fwd_split needs for
 * these arguments (0 when it would not split), without any device call.
 * Returns the status attn_fwd_split's validation of the sizes would return.
 */
attn_status attn_fwd_split_workspace(int B, int Sq, int Sk, int Hq, int Hkv,
                                     int d, int causal, int dtype,
                                     int kv_split, size_t* bytes);

/*
 * attn_fwd_split_plan -- the launches attn_fwd_split would make, without any
 * device call.  Writes up to n (at most 7) ints into `out`:
 *   [0] attention workgroups     [1] pieces of the longest query block
 *   [2] keys per piece (0 = no split)
 *   [3] first query row of a split block (Sq when nothing is split)
 *   [4] merge workgroups (0 when nothing is split)
 *   [5] threads per attention workgroup (512: two 4-wave groups that take
 *       alternate key tiles of the same rows, or 8 waves of key halves at
 *       padded head size 192, as attn_fwd_plan [1])
 *   [6] 1 if the waves take key halves (as attn_fwd_plan [10]; then nothing
 *       is split, except for fp16 above head size 128, whose pieces of a
 *       split also run key halves)
 */
attn_status attn_fwd_split_plan(int B, int Sq, int Sk, int Hq, int Hkv, int d,
                                int causal, int dtype, int kv_split, int* out,
                                int n);

/*
 * attn_merge -- combine partial attention states over disjoint key subsets
 * into the state of their union (e.g. the key shards of one sequence computed
 * by separate attention calls or on separate devices):
 *
 *     M = max_p lse_p,  w_p = e^(lse_p - M),
 *     O = sum_p w_p O_p / sum_p w_p,   LSE = M + ln sum_p w_p
 *
 * the online-softmax update of the personal-notes page (section "Online
 * Softmax") applied to whole parts.  A part with lse = -inf saw no key and
 * has weight 0; a row that no part saw gets O = 0 and LSE = -inf.
 *
 *   o_parts     device pointer, n_parts blocks of (B, Sq, Hq, d) elements of
 *               parts_dtype (ATTN_DTYPE_F32, F16 or BF16), part p at element
 *               offset p * B * Sq * Hq * d; each normalised over its own
 *               keys (as attn_fwd's O is); 16-byte aligned for F32, 8-byte
 *               aligned otherwise
 *   lse_parts   device pointer, n_parts blocks of (B, Hq, Sq) floats: the
 *               natural-log LSE of each part, as attn_fwd returns it; 4-byte
 *               aligned
 *   n_parts     >= 1
 *   B, Sq, Hq, d  sizes (d a multiple of 8 from 8 to 256)
 *   o           device pointer, (B, Sq, Hq, d) of dtype (F16 or BF16),
 *               8-byte aligned; written (must not overlap the inputs)
 *   lse         B * Hq * Sq floats, or NULL to skip
 *   stream      as for attn_fwd
 *
 * Size limit: B * Sq * Hq < 2^31.  attn_merge_check reports the status
 * without a device call.
 */
attn_status attn_merge(const void* o_parts, const float* lse_parts,
                       int n_parts, int parts_dtype, int B, int Sq, int Hq,
                       int d, void* o, float* lse, int dtype, void* stream);

/* attn_merge's validation without any device call (safe without a GPU). */
attn_status attn_merge_check(const void* o_parts, const float* lse_parts,
                             int n_parts, int parts_dtype, int B, int Sq,
                             int Hq, int d, void* o, float* lse, int dtype);

/*
 * attn_bwd -- gradients of L = sum(dO * O) with respect to q, k and v, for
 * O = attn_fwd(q, k, v) and its LSE (the reason the forward returns the LSE:
 * "CuTe DSL example", docstring).  The pages name FlashAttention 1 and 2 for
 * the backward algorithm; this is that recomputation: P is rebuilt tile by
 * tile from the scores and the LSE and never stored, with
 *     D_i = dO_i . O_i,  dS_ij = P_ij (dO_i . v_j - D_i),
 *     dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q.
 * GQA gradients of a kv head sum over its query heads.  Rows that see no key
 * (LSE = -inf) get dq = 0 and add nothing to dk, dv.
 *
 *   q, k, v, o, lse   the forward's inputs, output and LSE (as attn_fwd
 *                     writes them; dense (B, S, H, d) layouts, lse
 *                     (B, Hq, Sq) fp32)
 *   dout              dO, (B, Sq, Hq, d), the dtype of q
 *   dq                (B, Sq, Hq, d); written
 *   dk, dv            (B, Sk, Hkv, d); written
 *   B ... dtype       as for attn_fwd; d a multiple of 8 up to 256 (padded
 *                     to 32, 64, 96, 128, 192 or 256 inside the loads, as
 *                     the forward)
 *   workspace         device pointer, 256-byte aligned, of at least
 *                     attn_bwd_workspace bytes (two fp32 values per query row)
 *   stream            as for attn_fwd; three kernels are queued on it
 *
 * Every pointer but lse must be 16-byte aligned (lse 4-byte).  Each gradient
 * element is written once (no atomics): results are deterministic.
 * Returns ATTN_ERR_INVALID_ARG for a missing or short workspace and as
 * attn_fwd otherwise; attn_bwd_check validates without a device call.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, int B, int Sq, int Sk,
                     int Hq, int Hkv, int d, float scale, int causal,
                     int dtype, void* workspace, size_t workspace_bytes,
                     void* stream);

attn_status attn_bwd_check(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, int B, int Sq, int Sk,
                           int Hq, int Hkv, int d, float scale, int causal,
                           int dtype);

/*
 * attn_bwd_causal_offset -- attn_bwd for causal attention with an explicit
 * mask offset (query i sees key j iff j <= i + causal_offset), as
 * attn_fwd_causal_offset computes it: the backward of one key shard of a
 * longer causal problem.  Given the full problem's O and LSE (the merged
 * forward) and dO, it returns exactly the shard's dK and dV, and its part
 * of dQ (the sum over the shard's keys; the parts of all shards add up to
 * dQ, which the caller sums, in fp32 for accuracy).  This holds because the
 * recomputation above needs, besides the shard's keys, only the row
 * quantities LSE_i and D_i = dO_i . O_i of the full problem (the same reason
 * the forward returns the LSE: "CuTe DSL example", docstring).
 *
 *   o, lse           the full problem's output and LSE (not the shard's)
 *   causal_offset    -2^30 < causal_offset < 2^30
 *   the rest         as for attn_bwd (dk, dv: the shard's Sk keys)
 */
attn_status attn_bwd_causal_offset(const void* q, const void* k, const void* v,
                                   const void* o, const float* lse,
                                   const void* dout, void* dq, void* dk,
                                   void* dv, int B, int Sq, int Sk, int Hq,
                                   int Hkv, int d, float scale,
                                   long long causal_offset, int dtype,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

attn_status attn_bwd_causal_offset_check(const void* q, const void* k,
                                         const void* v, const void* o,
                                         const float* lse, const void* dout,
                                         void* dq, void* dk, void* dv, int B,
                                         int Sq, int Sk, int Hq, int Hkv, int d,
                                         float scale, long long causal_offset,
                                         int dtype);

/* Workspace bytes attn_bwd needs for B * Hq * Sq query rows (no device call). */
attn_status attn_bwd_workspace(int B, int Sq, int Hq, size_t* bytes);

/*
 * attn_decode_paged -- decode attention over a paged K/V cache: each of B
 * sequences has Sq new query tokens (its last Sq positions) and a history of
 * seqlens[b] keys kept in fixed-size blocks of a shared pool, listed by a
 * block table.  The MiniPaged-Qwen page (section 19, prefill vs. decode) has
 * decode read the K/V cache through Paged Attention; it gives no layout, and
 * this is the plainest one: an address translation in front of attn_fwd, so
 * the result is attn_fwd's on the gathered keys of each sequence (same
 * rounding, same masking; causal is bottom-right aligned to seqlens[b]).
 *
 *   q            (B, Sq, Hq, d), dense; query i of sequence b is position
 *                seqlens[b] - Sq + i
 *   k_cache, v_cache  the pools, (num_blocks, block_size, Hkv, d) each,
 *                dense: token t of sequence b is at block
 *                block_table[b * max_blocks + t / block_size], slot
 *                t % block_size
 *   block_table  device int32, (B, max_blocks), row-major; only the entries
 *                of blocks that hold one of the sequence's first
 *                min(seqlens[b], max_seqlen) tokens are read, and an entry
 *                outside [0, num_blocks) is clamped into it (wrong values, no
 *                out-of-range read)
 *   seqlens      device int32, (B): keys of each sequence; a length <= 0
 *                gives its rows O = 0 and LSE = -inf, and one above
 *                max_seqlen is taken as max_seqlen
 *   o, lse       as for attn_fwd: (B, Sq, Hq, d); lse (B, Hq, Sq) fp32 or NULL
 *   num_blocks   >= 1 blocks in each pool
 *   block_size   tokens per block, a multiple of 16
 *   max_blocks   >= 1 columns of the block table
 *   max_seqlen   the longest length to cover, 1 .. max_blocks * block_size;
 *                it sizes the key split (no device read of seqlens is made)
 *   B ... dtype  as for attn_fwd, restricted to the decode kernel's shapes:
 *                (Hq / Hkv) * Sq <= 32 (or <= 128 with Sq <= 8), else
 *                ATTN_ERR_UNSUPPORTED
 *   kv_split, workspace, workspace_bytes  as for attn_fwd_split, with the
 *                decode rule for kv_split = 0; the workspace size is
 *                attn_decode_paged_workspace's
 *   stream       as for attn_fwd; up to two kernels are queued on it
 *
 * Pointers: q, the pools and o 16-byte aligned; block_table, seqlens and lse
 * 4-byte aligned.  attn_decode_paged_check validates without a device call.
 */
attn_status attn_decode_paged(const void* q, const void* k_cache,
                              const void* v_cache, const int* block_table,
                              const int* seqlens, void* o, float* lse, int B,
                              int Sq, int Hq, int Hkv, int d, int num_blocks,
                              int block_size, int max_blocks, int max_seqlen,
                              float scale, int causal, int dtype,
                              int kv_split, void* workspace,
                              size_t workspace_bytes, void* stream);

attn_status attn_decode_paged_check(const void* q, const void* k_cache,
                                    const void* v_cache, const int* block_table,
                                    const int* seqlens, void* o, float* lse,
                                    int B, int Sq, int Hq, int Hkv, int d,
                                    int num_blocks, int block_size,
                                    int max_blocks, int max_seqlen, float scale,
                                    int causal, int dtype);

/* Workspace bytes attn_decode_paged needs (0 when it does not split). */
attn_status attn_decode_paged_workspace(int B, int Sq, int Hq, int Hkv, int d,
                                        int max_seqlen, int kv_split,
                                        size_t* bytes);

/* Human-readable name of a status code (static string). */
const char* attn_status_str(int status);

/* ATTN_ABI_VERSION of the library that was loaded. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_19_AMD_ATTN_H */
