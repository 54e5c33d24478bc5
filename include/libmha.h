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

#define MHA_ABI_VERSION 1

/* Status codes returned by every entry point. */
enum {
    MHA_OK = 0,
    MHA_ERR_NULL = 1,        /* a required pointer is NULL */
    MHA_ERR_SHAPE = 2,       /* negative size, or causal with n != m */
    MHA_ERR_DTYPE = 3,       /* dtype is not MHA_F32 or MHA_BF16 */
    MHA_ERR_UNSUPPORTED = 4, /* d_k != d_v, d not in {64, 128}, or sizes past the kernel's index range */
    MHA_ERR_SCALE = 5,       /* scale not finite or not > 0 */
    MHA_ERR_ALIAS = 6,       /* O overlaps Q, K, V or key_lens */
    MHA_ERR_HIP = 7,         /* the HIP runtime refused the launch */
    MHA_ERR_ALIGN = 8        /* a tensor pointer is not 16-byte aligned */
};

/* Element types. */
enum { MHA_F32 = 0, MHA_BF16 = 1 };

/* MHA_ABI_VERSION of the loaded library. */
int mha_abi_version(void);

/* A static, human-readable string for a status code (never NULL). */
const char *mha_status_string(int status);

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
int mha_validate(const void *Q, const void *K, const void *V,
                 const int32_t *key_lens, int causal, float scale,
                 const void *O, int64_t B, int64_t H, int64_t n, int64_t m,
                 int64_t d_k, int64_t d_v, int dtype);

/*
 * Enqueue the attention forward pass on `stream` (a hipStream_t; NULL is the
 * default stream of the current device).  Arguments as in mha_validate.
 * When B, H or n is 0 there is nothing to write and nothing is enqueued;
 * m == 0 writes zeros to O.  Returns MHA_OK once the kernel is enqueued.
 */
int mha_forward(const void *Q, const void *K, const void *V,
                const int32_t *key_lens, int causal, float scale, void *O,
                int64_t B, int64_t H, int64_t n, int64_t m,
                int64_t d_k, int64_t d_v, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMHA_H */
