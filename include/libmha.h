/*
 * libmha.h -- C ABI of a multi-head scaled dot-product attention forward
 * pass for AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every batch b, head t and query row i:
 *
 *     O[b,t,i,:] = sum_j softmax_j( scale * <Q[b,t,i,:], K[b,t,j,:]> + M_bij ) * V[b,t,j,:]
 *
 * the scaled dot-product attention of "Transformer: 详解" §4.1 and
 * "序列建模架构的演进与变革（二）" §4.3 / §4.9, with Q in R^{n x d_k},
 * K in R^{m x d_k}, V in R^{m x d_v} per head (hugogu wiki "Transformer",
 * self-attention steps 1-4), so n queries may attend to m != n keys
 * (cross-attention, "Transformer: 详解" §5.4, "第2章：完整的 Transformer
 * 架构" §7).  The mask M is 0 where the pair is valid and -inf otherwise:
 *
 *     valid(b,i,j) = j < L_b  AND  (causal == 0  OR  j <= i)
 *
 * L_b comes from key_lens: the key-padding mask of "Transformer: 详解" §3.4
 * (tail padding, one keep-flag per key, broadcast over heads and queries),
 * expressed as a length.  causal is the lower-triangular mask of
 * "Transformer: 详解" §5.3 and "第2章：完整的 Transformer 架构" §6 (a query
 * sees itself and earlier keys).  The two combine with AND ("Transformer:
 * 详解" §5.3).  A row with no valid key has output 0 (the pages leave this
 * case open).  Query rows at padded positions are computed like any other
 * row.
 *
 * Layout.  All tensors are dense row-major:
 *     Q [B, H, n, d_k]    K [B, H, m, d_k]    V [B, H, m, d_v]    O [B, H, n, d_v]
 * element type MHA_BF16 (bfloat16) or MHA_F32 (float32), the same for all
 * four.  Accumulation is fp32; bf16 outputs are rounded to nearest even.
 *
 * Ownership.  Every pointer is device memory owned by the caller.  The
 * library allocates nothing, keeps no pointer after returning, holds no
 * mutable global state, and never synchronizes: mha_forward enqueues one
 * kernel on the given stream and returns.  O is fully overwritten; Q, K and
 * V may alias one another (they are only read) but must not overlap O or
 * key_lens.
 *
 * Errors.  mha_validate and the argument check at the top of mha_forward
 * run on the host and make no HIP call; on an error status nothing is
 * enqueued and O is untouched.  key_lens values live on the device and are
 * not validated: each is clamped to [0, m] by the kernel.  A failed launch
 * returns MHA_ERR_HIP.  Device faults surface at the caller's next
 * synchronization, as for any HIP kernel.
 */
#ifndef LIBMHA_H
#define LIBMHA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHA_ABI_VERSION 5

/* Status codes returned by every entry point. */
typedef enum mha_status {
    MHA_OK = 0,
    MHA_ERR_NULL = 1,        /* a required pointer is NULL */
    MHA_ERR_SHAPE = 2,       /* negative size, or causal with n != m */
    MHA_ERR_DTYPE = 3,       /* dtype is not MHA_F32 or MHA_BF16 */
    MHA_ERR_UNSUPPORTED = 4, /* d_k != d_v, d not in {64, 128}, or sizes past the kernel's index range */
    MHA_ERR_SCALE = 5,       /* scale not finite or not > 0 */
    MHA_ERR_ALIAS = 6,       /* O overlaps Q, K, V or key_lens */
    MHA_ERR_HIP = 7,         /* the HIP runtime refused the launch */
    MHA_ERR_ALIGN = 8,       /* a tensor pointer is not 16-byte aligned (lse, slopes: 4) */
    MHA_ERR_MODE = 9,        /* mask_mode is not one of the MHA_MASK_* values */
    MHA_ERR_WORKSPACE = 10   /* decode workspace missing, too small, misaligned or overlapping */
} mha_status;

/* Mask modes of the extended entry points (key padding always applies). */
enum {
    MHA_MASK_NONE = 0,               /* no causal mask */
    MHA_MASK_CAUSAL = 1,             /* top-left: key j visible to query i when j <= i */
    MHA_MASK_CAUSAL_BOTTOM_RIGHT = 2 /* query i is the token at position i + L_b - n */
};

/* Element type of every tensor argument of one call. */
typedef enum mha_dtype { MHA_F32 = 0, MHA_BF16 = 1 } mha_dtype;

/* MHA_ABI_VERSION of the loaded library. */
int mha_abi_version(void);

/* A static, human-readable string for a status code (never NULL). */
const char *mha_status_string(mha_status status);

/*
 * Host-side argument check of mha_forward, without any HIP call.
 *
 *   Q, K, V, O   device pointers, 16-byte aligned; may be NULL only when the
 *                tensor has no element.
 *   key_lens     device int32[B] of valid key counts, or NULL for "all m
 *                keys valid".
 *   causal       0 or non-zero; non-zero requires n == m.
 *   scale        the factor applied to q.k; finite and > 0.  Callers pass
 *                1/sqrt(d_k) for the attention of the pages.
 *   B, H, n, m   batch, heads, query rows, key rows (>= 0).
 *   d_k, d_v     head widths; the GPU kernels support d_k == d_v in {64, 128}.
 *   dtype        MHA_F32 or MHA_BF16.
 *
 * Returns MHA_OK or the first error found.
 */
mha_status mha_validate(const void *Q, const void *K, const void *V,
                        const int32_t *key_lens, int causal, float scale,
                        const void *O, int64_t B, int64_t H, int64_t n, int64_t m,
                        int64_t d_k, int64_t d_v, mha_dtype dtype);

/*
 * Enqueue the attention forward pass on `stream` (a hipStream_t; NULL is the
 * default stream of the current device).  Arguments as in mha_validate.
 * When B, H or n is 0 there is nothing to write and nothing is enqueued;
 * m == 0 writes zeros to O.  Returns MHA_OK once the kernel is enqueued.
 */
mha_status mha_forward(const void *Q, const void *K, const void *V,
                       const int32_t *key_lens, int causal, float scale, void *O,
                       int64_t B, int64_t H, int64_t n, int64_t m,
                       int64_t d_k, int64_t d_v, mha_dtype dtype, void *stream);

/*
 * ---- Extended forward pass -------------------------------------------------
 *
 * The same operation with the variants that sit next to it on the pages:
 *
 *     O[b,t,i,:] = sum_j softmax_j( scale * <Q[b,t,i,:], K[b,g,j,:]>
 *                                   - slope_t * |p_i - j| + M_bij ) * V[b,g,j,:]
 *
 *   - Grouped K/V heads (GQA; MQA when H_kv = 1; hugogu wiki "Transformer",
 *     attention-optimisation table; "序列建模架构的演进与变革（二）" §3.8):
 *     K and V have H_kv heads and query head t reads K/V head
 *     g = t / (H / H_kv).  H_kv = H is plain multi-head attention.
 *   - ALiBi ("第2章：完整的 Transformer 架构" §5.3): a per-head slope times
 *     the query-key distance is subtracted from the scaled score.
 *     alibi_slopes: device fp32[H], or NULL for no bias.
 *   - Causal alignment, mask_mode:
 *       MHA_MASK_NONE                 valid = j < L_b,                p_i = i
 *       MHA_MASK_CAUSAL               valid = j < L_b and j <= i,     p_i = i
 *       MHA_MASK_CAUSAL_BOTTOM_RIGHT  valid = j < L_b and j <= p_i,   p_i = i + L_b - n
 *     Bottom-right places the n queries at the end of a sequence whose first
 *     L_b keys are filled: incremental decoding against a key/value cache
 *     of capacity m (hugogu wiki "Transformer", KV-cache section).  Rows with
 *     no visible key (p_i < 0) have output 0.  Both causal modes accept
 *     n != m.
 *   - lse: device fp32[B, H, n] or NULL.  When given, receives each row's
 *     natural-log log-sum-exp of its valid scaled, biased scores (-inf for a
 *     row with no valid key); mha_attention_weights consumes it.
 *
 * Layout: Q [B, H, n, d_k], K [B, H_kv, m, d_k], V [B, H_kv, m, d_v],
 * O [B, H, n, d_v], row-major.  Ownership and errors as for mha_forward;
 * H % H_kv != 0 or H_kv = 0 with H > 0 is MHA_ERR_SHAPE, a bad mask_mode
 * MHA_ERR_MODE, lse overlapping any other argument MHA_ERR_ALIAS.  Slopes
 * are device data and are not validated.
 */
mha_status mha_validate_ex(const void *Q, const void *K, const void *V,
                           const int32_t *key_lens, int mask_mode,
                           const float *alibi_slopes, float scale, const void *O,
                           const float *lse, int64_t B, int64_t H, int64_t H_kv,
                           int64_t n, int64_t m, int64_t d_k, int64_t d_v, mha_dtype dtype);

mha_status mha_forward_ex(const void *Q, const void *K, const void *V,
                          const int32_t *key_lens, int mask_mode,
                          const float *alibi_slopes, float scale, void *O, float *lse,
                          int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                          int64_t d_k, int64_t d_v, mha_dtype dtype, void *stream);

/*
 * The forward kernel instance that mha_forward / mha_forward_ex launch for
 * these sizes, as profilers name it (e.g.
 * "mha::attn_fwd_kernel<__bf16, 128, 8, 1, true, false>": element type,
 * head width, waves per workgroup, key groups per workgroup, causal, ALiBi),
 * so that a kernel trace can be matched to a call.  mask_mode as for
 * mha_forward_ex (mha_forward's causal flag is MHA_MASK_CAUSAL); alibi: 0
 * or 1.  Pure host arithmetic; returns a static string, or NULL for
 * arguments mha_forward_ex would refuse on their sizes, dtype or mode.
 */
const char *mha_forward_kernel_name(int64_t B, int64_t H, int64_t H_kv,
                                    int64_t n, int64_t m, int64_t d,
                                    mha_dtype dtype, int mask_mode, int alibi);

/*
 * ---- Attention weights --------------------------------------------------------
 *
 * Writes A[b,t,i,j] = exp(scale * <Q[b,t,i,:], K[b,g,j,:]> - slope_t*|p_i - j|
 * - lse[b,t,i]) for valid (i, j) and 0 elsewhere: the softmax weights that
 * the pages' attention function returns beside its output
 * ("序列建模架构的演进与变革（二）" §4.9).  lse must come from mha_forward_ex
 * with the same Q, K, key_lens, mask_mode, alibi_slopes and scale.  A is a
 * dense row-major [B, H, n, m] tensor of the element type `dtype` (16-byte
 * aligned), fully overwritten; it must not overlap any input.  This pass
 * materialises B*H*n*m elements, the n x m memory the fused forward pass
 * avoids; it is for callers that need the weights themselves.  d_k in
 * {64, 128}; one head's A must stay under 2 GiB.  Errors as for
 * mha_forward_ex.
 */
mha_status mha_validate_weights(const void *Q, const void *K, const int32_t *key_lens,
                                int mask_mode, const float *alibi_slopes, float scale,
                                const float *lse, const void *A, int64_t B, int64_t H,
                                int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                                mha_dtype dtype);

mha_status mha_attention_weights(const void *Q, const void *K, const int32_t *key_lens,
                                 int mask_mode, const float *alibi_slopes, float scale,
                                 const float *lse, void *A, int64_t B, int64_t H,
                                 int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                                 mha_dtype dtype, void *stream);

/*
 * ---- Decoding against a key/value cache ---------------------------------------
 *
 * The n new queries of each sequence attend to its cache: K, V [B, H_kv, m, d]
 * hold the keys and values of the sequence's tokens in rows 0..L_b-1 (the
 * new tokens' own rows included), m is the cache capacity, L_b =
 * cache_lens[b] (clamped to [0, m]; NULL means m).  Incremental decoding
 * stores every earlier token's K and V in a cache allocated at the maximum
 * length and computes only the new tokens' (hugogu wiki "Transformer",
 * KV-cache section; "序列建模架构的演进与变革（二）" §3.4).
 *
 * The result is exactly that of mha_forward_ex with mask_mode =
 * MHA_MASK_CAUSAL_BOTTOM_RIGHT and key_lens = cache_lens: query i is the
 * token at position i + L_b - n.  The difference is the schedule, built for
 * small n and long caches: the key axis is cut across workgroups so that
 * the cache streams from HBM at full width even for one sequence.  When it
 * is cut, the partial results go to a caller-provided workspace and a
 * second kernel merges them.
 *
 * mha_decode_workspace_size: *bytes receives the workspace size the call
 * with these sizes needs (0 when it needs none).  Pure host arithmetic.
 *
 * mha_decode: arguments as for mha_forward_ex (no mask_mode), plus
 * workspace (device memory of at least that size, 16-byte aligned, not
 * overlapping any other argument; may be NULL when the size is 0) and its
 * size.  The workspace holds no state between calls; two calls in flight
 * at once need two workspaces.  Errors as for mha_forward_ex, and
 * MHA_ERR_WORKSPACE.
 */
mha_status mha_decode_workspace_size(int64_t B, int64_t H, int64_t H_kv, int64_t n,
                                     int64_t m, int64_t d, mha_dtype dtype, int64_t *bytes);

mha_status mha_validate_decode(const void *Q, const void *K, const void *V,
                               const int32_t *cache_lens, const float *alibi_slopes,
                               float scale, const void *O, const float *lse,
                               const void *workspace, int64_t workspace_bytes,
                               int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                               int64_t d_k, int64_t d_v, mha_dtype dtype);

mha_status mha_decode(const void *Q, const void *K, const void *V,
                      const int32_t *cache_lens, const float *alibi_slopes, float scale,
                      void *O, float *lse, void *workspace, int64_t workspace_bytes,
                      int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                      int64_t d_k, int64_t d_v, mha_dtype dtype, void *stream);

/*
 * mha_decode_noalloc: mha_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments without the workspace: when the key
 * axis is split, the partial results go to a fixed scratch array of 8.5 MiB
 * that the library keeps in device memory, one per GPU, until the process
 * ends; the call allocates nothing.  Every size mha_decode accepts fits it
 * (no split plan needs more); a plan that would not is MHA_ERR_UNSUPPORTED.
 * All calls on one GPU share that GPU's array, and no call reads what an
 * earlier one left there: calls that may overlap on one GPU (other streams
 * or other host threads) race on it, and the caller must serialise them.
 * Errors as for mha_decode; MHA_ERR_HIP also when the array's device
 * address cannot be obtained.
 */
mha_status mha_decode_noalloc(const void *Q, const void *K, const void *V,
                              const int32_t *cache_lens, const float *alibi_slopes,
                              float scale, void *O, float *lse, int64_t B, int64_t H,
                              int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                              int64_t d_v, mha_dtype dtype, void *stream);

/*
 * ---- Multi-head attention with its projections ---------------------------------
 *
 * The layer around the core, as the pages write it ("序列建模架构的演进与变革
 * （二）" §4.9; "Transformer: 详解" §4.2; "第2章：完整的 Transformer 架构"
 * §2.2):
 *
 *     Q = split(Xq Wq^T + bq)    K = split(Xk Wk^T + bk)    V = split(Xv Wv^T + bv)
 *     O = attention(Q, K, V)     per head, with key_lens and mask_mode as in
 *                                mha_forward_ex (no ALiBi, H_kv = H)
 *     Y = concat(O) Wo^T + bo
 *
 * split: [B, L, d_model] -> [B, H, L, d_k], d_k = d_model / H; concat is its
 * inverse.  Self-attention passes the same tensor as Xq, Xk and Xv;
 * cross-attention passes the decoder states as Xq and the encoder output as
 * Xk and Xv.
 *
 *   Xq        [B, n, d_model]; Xk, Xv [B, m, d_model] (may alias each other)
 *   W*        [d_model, d_model] in nn.Linear's [out, in] layout, 16-byte aligned
 *   b*        [d_model] or NULL for no bias
 *   Y         [B, n, d_model] output
 *   A         [B, H, n, m] attention weights (as mha_attention_weights), or NULL
 *   workspace at least mha_multihead_workspace_size bytes, 16-byte aligned,
 *             overlapping nothing else; it holds Q, K, V and O (and the row
 *             log-sum-exp when A is requested) during the call.
 *
 * All tensors share `dtype`; projections accumulate in fp32 and round
 * their results (Q, K, V, O, Y) to dtype.  d_k in {64, 128}.  Errors as for
 * mha_forward_ex, plus MHA_ERR_WORKSPACE; sizes whose tensors pass 2 GiB are
 * MHA_ERR_UNSUPPORTED.  Enqueues four to five kernels on `stream`.
 */
mha_status mha_multihead_workspace_size(int64_t B, int64_t n, int64_t m,
                                        int64_t d_model, int64_t H, mha_dtype dtype,
                                        int need_weights, int64_t *bytes);

/* Host-side argument check of mha_multihead_forward (no HIP call); the
 * arguments are those of the call below without the stream. */
mha_status mha_validate_multihead(const void *Xq, const void *Xk, const void *Xv,
                                  const void *Wq, const void *bq, const void *Wk,
                                  const void *bk, const void *Wv, const void *bv,
                                  const void *Wo, const void *bo,
                                  const int32_t *key_lens, int mask_mode, float scale,
                                  const void *Y, const void *A, const void *workspace,
                                  int64_t workspace_bytes, int64_t B, int64_t n,
                                  int64_t m, int64_t d_model, int64_t H, mha_dtype dtype);

mha_status mha_multihead_forward(const void *Xq, const void *Xk, const void *Xv,
                                 const void *Wq, const void *bq, const void *Wk,
                                 const void *bk, const void *Wv, const void *bv,
                                 const void *Wo, const void *bo,
                                 const int32_t *key_lens, int mask_mode, float scale,
                                 void *Y, void *A, void *workspace,
                                 int64_t workspace_bytes, int64_t B, int64_t n,
                                 int64_t m, int64_t d_model, int64_t H, mha_dtype dtype,
                                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMHA_H */
