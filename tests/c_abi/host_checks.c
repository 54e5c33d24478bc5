/*
 * host_checks.c -- drives every host-side entry point of libmha (the
 * argument checks, workspace sizes, status strings and kernel names) from
 * plain C with fake, never-dereferenced device addresses, and checks the
 * status each call returns.  Linked against the host-only translation unit
 * (mha_host.cpp) built with address and undefined-behaviour sanitizers, so
 * that an overflow, an out-of-bounds access or a bad conversion anywhere in
 * the checks aborts the program, including on the extreme sizes below.
 *
 * Exit status 0 and the line "host checks: N passed" when every case holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "libmha.h"

static int failures = 0, passed = 0;

#define EXPECT(expr, want)                                                         \
    do {                                                                           \
        long long got_ = (long long)(expr);                                        \
        if (got_ != (long long)(want)) {                                           \
            fprintf(stderr, "%s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__,   \
                    #expr, got_, (long long)(want));                               \
            ++failures;                                                            \
        } else {                                                                   \
            ++passed;                                                              \
        }                                                                          \
    } while (0)

/* Fake, 16-byte aligned, far-apart device addresses. */
#define P(x) ((void *)(uintptr_t)(x))
static const uintptr_t Q = 1ull << 40, K = 2ull << 40, V = 3ull << 40, O = 4ull << 40,
                       KL = 5ull << 40, LSE = 6ull << 40, SL = 7ull << 40, A = 8ull << 40,
                       WSP = 9ull << 40;

static mha_status val(uintptr_t q, uintptr_t k, uintptr_t v, uintptr_t kl, int causal,
                      float scale, uintptr_t o, int64_t B, int64_t H, int64_t n, int64_t m,
                      int64_t dk, int64_t dv, int dtype) {
    return mha_validate(P(q), P(k), P(v), (const int32_t *)P(kl), causal, scale, P(o), B, H, n,
                        m, dk, dv, (mha_dtype)dtype);
}

static mha_status val_ex(uintptr_t lse, uintptr_t sl, int mode, int64_t B, int64_t H,
                         int64_t Hkv, int64_t n, int64_t m, int64_t d) {
    return mha_validate_ex(P(Q), P(K), P(V), NULL, mode, (const float *)P(sl), 0.125f, P(O),
                           (const float *)P(lse), B, H, Hkv, n, m, d, d, MHA_BF16);
}

static void forward_checks(void) {
    const int64_t big = (int64_t)1 << 62, lim = ((int64_t)1 << 23) - 1;
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_OK);
    EXPECT(val(Q, K, V, KL, 1, 0.125f, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_OK);
    EXPECT(val(0, K, V, 0, 0, 0.125f, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_NULL);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, -1, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_SHAPE);
    EXPECT(val(Q, K, V, 0, 1, 0.125f, O, 2, 8, 128, 129, 64, 64, MHA_BF16), MHA_ERR_SHAPE);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, 2, 8, 128, 128, 64, 64, 2), MHA_ERR_DTYPE);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, 2, 8, 128, 128, 96, 96, MHA_BF16), MHA_ERR_UNSUPPORTED);
    EXPECT(val(Q, K, V, 0, 0, 0.0f, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_SCALE);
    EXPECT(val(Q, K, V, 0, 0, NAN, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_SCALE);
    EXPECT(val(Q, K, V, 0, 0, INFINITY, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_SCALE);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, Q + 64, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_ALIAS);
    EXPECT(val(Q, K, V, O + 16, 0, 0.125f, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_ALIAS);
    EXPECT(val(Q + 8, K, V, 0, 0, 0.125f, O, 2, 8, 128, 128, 64, 64, MHA_BF16), MHA_ERR_ALIGN);
    /* size limits: 2 GiB per head, 2^32 work-items per grid, saturating extents */
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, 1, 1, lim, 64, 128, 128, MHA_BF16), MHA_OK);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, 1, 1, lim + 1, 64, 128, 128, MHA_BF16),
           MHA_ERR_UNSUPPORTED);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, 1, 1, big, 64, 64, 64, MHA_BF16), MHA_ERR_UNSUPPORTED);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, 1, 1, 64, big, 64, 64, MHA_BF16), MHA_ERR_UNSUPPORTED);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, INT64_MAX, INT64_MAX, 128, 128, 64, 64, MHA_BF16),
           MHA_ERR_UNSUPPORTED);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, ((int64_t)1 << 31) - 1, ((int64_t)1 << 31) - 1, 0, lim,
               128, 128, MHA_BF16),
           MHA_OK);
    EXPECT(val(Q, K, V, 0, 0, 0.125f, O, ((int64_t)1 << 31) - 1, ((int64_t)1 << 31) - 1, 1, lim,
               128, 128, MHA_BF16),
           MHA_ERR_UNSUPPORTED);
    /* extended forward */
    EXPECT(val_ex(0, 0, 0, 2, 8, 8, 128, 128, 64), MHA_OK);
    EXPECT(val_ex(LSE, SL, 2, 2, 8, 1, 1, 4096, 128), MHA_OK);
    EXPECT(val_ex(0, 0, 0, 2, 8, 3, 128, 128, 64), MHA_ERR_SHAPE);
    EXPECT(val_ex(0, 0, 0, 2, 8, 0, 128, 128, 64), MHA_ERR_SHAPE);
    EXPECT(val_ex(0, 0, 3, 2, 8, 8, 128, 128, 64), MHA_ERR_MODE);
    EXPECT(val_ex(O + 64, 0, 0, 2, 8, 8, 128, 128, 64), MHA_ERR_ALIAS);
    EXPECT(val_ex(LSE + 2, 0, 0, 2, 8, 8, 128, 128, 64), MHA_ERR_ALIGN);
    EXPECT(val_ex(0, SL + 1, 0, 2, 8, 8, 128, 128, 64), MHA_ERR_ALIGN);
    EXPECT(val_ex(LSE, 0, 1, INT64_MAX, INT64_MAX, 1, big, big, 64), MHA_ERR_UNSUPPORTED);
    EXPECT(val_ex(LSE, 0, 1, INT64_MAX, INT64_MAX, INT64_MAX, 0, 0, 64), MHA_ERR_UNSUPPORTED);
    EXPECT(val_ex(LSE, 0, 1, ((int64_t)1 << 31) - 1, ((int64_t)1 << 31) - 1,
                  ((int64_t)1 << 31) - 1, 0, lim, 128),
           MHA_OK);
}

static void weights_checks(void) {
#define VW(a, lse, B, H, Hkv, n, m, dk)                                                     \
    mha_validate_weights(P(Q), P(K), NULL, 0, NULL, 0.125f, (const float *)P(lse), P(a), B, \
                         H, Hkv, n, m, dk, MHA_BF16)
    EXPECT(VW(A, LSE, 2, 8, 8, 128, 128, 64), MHA_OK);
    EXPECT(VW(A, LSE, 2, 8, 3, 128, 128, 64), MHA_ERR_SHAPE);
    EXPECT(VW(A, 0, 2, 8, 8, 128, 128, 64), MHA_ERR_NULL);
    EXPECT(VW(Q, LSE, 2, 8, 8, 128, 128, 64), MHA_ERR_ALIAS);
    EXPECT(VW(A + 8, LSE, 2, 8, 8, 128, 128, 64), MHA_ERR_ALIGN);
    EXPECT(VW(A, LSE, 2, 8, 8, 1 << 16, 1 << 16, 64), MHA_ERR_UNSUPPORTED);
    EXPECT(VW(A, LSE, INT64_MAX, INT64_MAX, 1, INT64_MAX, INT64_MAX, 128), MHA_ERR_UNSUPPORTED);
    EXPECT(VW(A, LSE, INT64_MAX, INT64_MAX, INT64_MAX, 0, INT64_MAX, 128), MHA_ERR_UNSUPPORTED);
#undef VW
}

static void decode_checks(void) {
    int64_t bytes = -1, need = 0;
    EXPECT(mha_decode_workspace_size(8, 32, 8, 1, 16384, 128, MHA_BF16, &need), MHA_OK);
    EXPECT(need > 0, 1);
    EXPECT(mha_decode_workspace_size(8, 32, 8, 1, 16384, 128, MHA_BF16, NULL), MHA_ERR_NULL);
    EXPECT(mha_decode_workspace_size(8, 32, 3, 1, 16384, 128, MHA_BF16, &bytes), MHA_ERR_SHAPE);
    EXPECT(mha_decode_workspace_size(8, 32, 8, 1, 16384, 96, MHA_BF16, &bytes),
           MHA_ERR_UNSUPPORTED);
    EXPECT(mha_decode_workspace_size(0, 32, 8, 1, 16384, 128, MHA_BF16, &bytes), MHA_OK);
    EXPECT(bytes, 0);
    /* sizes far past anything a launch accepts: refused, never wrapped */
    EXPECT(mha_decode_workspace_size(INT64_MAX, INT64_MAX, 1, INT64_MAX, INT64_MAX, 128,
                                     MHA_BF16, &bytes),
           MHA_ERR_UNSUPPORTED);
    EXPECT(mha_decode_workspace_size(1, 1, 1, 1, INT64_MAX, 128, MHA_BF16, &bytes),
           MHA_ERR_UNSUPPORTED);
#define VD(ws, wsb, B, H, Hkv, n, m)                                                          \
    mha_validate_decode(P(Q), P(K), P(V), NULL, NULL, 0.125f, P(O), NULL, P(ws), wsb, B, H,   \
                        Hkv, n, m, 128, 128, MHA_BF16)
    EXPECT(VD(WSP, need, 8, 32, 8, 1, 16384), MHA_OK);
    EXPECT(VD(WSP, need - 1, 8, 32, 8, 1, 16384), MHA_ERR_WORKSPACE);
    EXPECT(VD(0, need, 8, 32, 8, 1, 16384), MHA_ERR_WORKSPACE);
    EXPECT(VD(WSP + 8, need, 8, 32, 8, 1, 16384), MHA_ERR_WORKSPACE);
    EXPECT(VD(O, need, 8, 32, 8, 1, 16384), MHA_ERR_WORKSPACE);
    EXPECT(VD(WSP, need, 8, 32, 5, 1, 16384), MHA_ERR_SHAPE);
    EXPECT(VD(WSP, INT64_MAX, INT64_MAX, INT64_MAX, 1, INT64_MAX, INT64_MAX),
           MHA_ERR_UNSUPPORTED);
#undef VD
}

static void multihead_checks(void) {
    int64_t b = -1, bw = -1;
    EXPECT(mha_multihead_workspace_size(4, 128, 128, 512, 8, MHA_BF16, 0, &b), MHA_OK);
    EXPECT(mha_multihead_workspace_size(4, 128, 128, 512, 8, MHA_BF16, 1, &bw), MHA_OK);
    EXPECT(bw > b, 1);
    EXPECT(mha_multihead_workspace_size(4, 128, 128, 500, 8, MHA_BF16, 0, &b), MHA_ERR_SHAPE);
    EXPECT(mha_multihead_workspace_size(4, 128, 128, 256, 8, MHA_BF16, 0, &b),
           MHA_ERR_UNSUPPORTED);
    EXPECT(mha_multihead_workspace_size(4, 128, 128, 512, 8, 3, 0, &b), MHA_ERR_DTYPE);
    EXPECT(mha_multihead_workspace_size(INT64_MAX, INT64_MAX, INT64_MAX, 512, 8, MHA_BF16, 1,
                                        &b),
           MHA_ERR_UNSUPPORTED);
    EXPECT(mha_multihead_workspace_size(4, 128, 128, 512, 0, MHA_BF16, 0, &b), MHA_ERR_SHAPE);
    int64_t need = 0;
    mha_multihead_workspace_size(4, 128, 128, 512, 8, MHA_BF16, 0, &need);
    const uintptr_t X = 10ull << 40, W = 11ull << 40, Y = 12ull << 40;
#define MH(ws, wsb, y, a, mode, scale, B, n, m, dm, H)                                          \
    mha_validate_multihead(P(X), P(X), P(X), P(W), NULL, P(W + (1 << 24)), NULL,                \
                           P(W + (2 << 24)), NULL, P(W + (3 << 24)), NULL, NULL, mode, scale,   \
                           P(y), P(a), P(ws), wsb, B, n, m, dm, H, MHA_BF16)
    EXPECT(MH(WSP, need - 1, Y, 0, 0, 0.125f, 4, 128, 128, 512, 8), MHA_ERR_WORKSPACE);
    EXPECT(MH(0, need, Y, 0, 0, 0.125f, 4, 128, 128, 512, 8), MHA_ERR_WORKSPACE);
    EXPECT(MH(W, need, Y, 0, 0, 0.125f, 4, 128, 128, 512, 8), MHA_ERR_WORKSPACE);
    EXPECT(MH(WSP, need, X, 0, 0, 0.125f, 4, 128, 128, 512, 8), MHA_ERR_ALIAS);
    EXPECT(MH(WSP, need, Y + 4, 0, 0, 0.125f, 4, 128, 128, 512, 8), MHA_ERR_ALIGN);
    EXPECT(MH(WSP, need, Y, 0, 7, 0.125f, 4, 128, 128, 512, 8), MHA_ERR_MODE);
    EXPECT(MH(WSP, need, Y, 0, 0, -1.0f, 4, 128, 128, 512, 8), MHA_ERR_SCALE);
    EXPECT(MH(WSP, need, Y, 0, 0, 0.125f, 4, 128, 128, 512, 5), MHA_ERR_SHAPE);
    EXPECT(MH(WSP, need, Y, 0, 0, 0.125f, 0, 128, 128, 512, 8), MHA_OK);
    EXPECT(MH(WSP, INT64_MAX, Y, A, 0, 0.125f, 4, 1 << 20, 1 << 20, 512, 8), MHA_ERR_UNSUPPORTED);
    EXPECT(MH(WSP, INT64_MAX, Y, 0, 0, 0.125f, INT64_MAX, INT64_MAX, 1, 512, 8),
           MHA_ERR_UNSUPPORTED);
#undef MH
}

static void name_checks(void) {
    const char *s = mha_forward_kernel_name(1, 16, 16, 16384, 16384, 128, MHA_BF16, 1, 0);
    EXPECT(s != NULL && strcmp(s, "mha::attn_fwd_kernel<__bf16, 128, 8, 1, true, false>") == 0,
           1);
    s = mha_forward_kernel_name(32, 8, 8, 128, 128, 64, MHA_BF16, 0, 0);
    EXPECT(s != NULL && strcmp(s, "mha::attn_fwd_kernel<__bf16, 64, 4, 1, false, false>") == 0,
           1);
    EXPECT(mha_forward_kernel_name(1, 8, 8, 16, 16, 96, MHA_BF16, 0, 0) == NULL, 1);
    EXPECT(mha_forward_kernel_name(INT64_MAX, INT64_MAX, 1, INT64_MAX, INT64_MAX, 128, MHA_BF16,
                                   1, 1) != NULL,
           1);
    for (int st = -2; st < 14; ++st) EXPECT(mha_status_string((mha_status)st) != NULL, 1);
    EXPECT(strcmp(mha_status_string((mha_status)99), "unknown status"), 0);
    EXPECT(mha_abi_version(), MHA_ABI_VERSION);
}

int main(void) {
    forward_checks();
    weights_checks();
    decode_checks();
    multihead_checks();
    name_checks();
    if (failures) {
        fprintf(stderr, "host checks: %d failed, %d passed\n", failures, passed);
        return 1;
    }
    printf("host checks: %d passed\n", passed);
    return 0;
}
