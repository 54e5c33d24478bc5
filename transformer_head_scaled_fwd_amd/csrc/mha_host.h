// mha_host.h -- host-side pieces of the library that involve no HIP call:
// the argument checks of every entry point, the decode and multi-head
// plans, and the choice of forward-kernel variant.  They live in a
// translation unit of plain C++ (mha_host.cpp) so that the same code can be
// built for the host alone, e.g. with sanitizers.
#pragma once

#include <stdint.h>

#include "libmha.h"

namespace mha {

// Checks shared by the forward entry points.  H_kv: K/V heads; mode 0/1/2
// (none, causal top-left, causal bottom-right).  Returns a status code.
mha_status check_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens, int mode,
                  const float* alibi, float scale, const void* O, const float* lse, int64_t B,
                  int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k, int64_t d_v,
                  mha_dtype dtype);

// How the decode kernel cuts the key axis: row sets of 32 query rows,
// splits of split_blocks key blocks of 64, and the workspace the splits
// need (0 when one split covers the whole axis): every split's partial
// output, running max and row sum in fp32, which a second kernel merges.
struct DecodePlan {
  int64_t nrs, nsplit, split_blocks, workspace_bytes;
};
DecodePlan plan_decode(int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m, int d,
                       bool bf16);

// Size of the library's own decode scratch (mha_decode_noalloc).  The key
// axis is split only while fewer than 256 (batch, K/V head, row set) units
// exist, each unit holds at most 32 query rows, and a unit gets at most
// ceil(256 / units) splits, so every split plan needs at most
// 32 * 510 * (128 + 2) * 4 = 8486400 bytes; 8.5 MiB covers it.
constexpr int64_t kDecodeScratchBytes = (int64_t)17 << 19;

// Argument check of mha_decode_noalloc: that of mha_decode without the
// workspace, and the split plan must fit kDecodeScratchBytes.
mha_status check_decode_noalloc(const void* Q, const void* K, const void* V,
                                const int32_t* cache_lens, const float* alibi_slopes,
                                float scale, const void* O, const float* lse, int64_t B,
                                int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                                int64_t d_v, mha_dtype dtype);

// Workspace of the multi-head forward: Q, K, V, O in [B, H, L, d_k], then
// the row log-sum-exp when the weights are requested; each part 256-byte
// aligned.
struct MhLayout {
  int64_t q, k, v, o, lse, total;
};
MhLayout mh_layout(int64_t B, int64_t n, int64_t m, int64_t d_model, int64_t H, int64_t es,
                   bool weights);
mha_status check_multihead_sizes(int64_t B, int64_t n, int64_t m, int64_t d_model, int64_t H,
                          mha_dtype dtype);

// The full argument check of mha_multihead_forward (sizes, pointers,
// alignment, overlaps, workspace).
mha_status check_multihead(const void* Xq, const void* Xk, const void* Xv, const void* Wq,
                    const void* bq, const void* Wk, const void* bk, const void* Wv,
                    const void* bv, const void* Wo, const void* bo, const int32_t* key_lens,
                    int mask_mode, float scale, const void* Y, const void* A,
                    const void* workspace, int64_t workspace_bytes, int64_t B, int64_t n,
                    int64_t m, int64_t d_model, int64_t H, mha_dtype dtype);

// Division by a divisor d in [1, 2^31) fixed at launch, for indices n in
// [0, 2^31): n / d = (n + mulhi(n, mul)) >> shift, where shift = ceil(log2 d)
// and 2^32 + mul = ceil(2^(32 + shift) / d) (the round-up multiplier of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  With 2^shift >= d the multiplier exceeds
// 2^(32 + shift) / d by less than 1 / d of a unit, and n d < 2^(32 + shift),
// so the product never carries n / d past the next integer.  Kernels decode
// their block index with it instead of a run-time division.
struct FastDiv {
  uint32_t d, mul, shift;
};
FastDiv fast_div(uint32_t d);

// Workgroup shape of the forward kernel for a problem: NW waves per
// workgroup, KS key groups (see the kernel).  mode: 0 no causal mask, 1
// causal top-left, 2 causal bottom-right.
struct FwdVariant {
  int nw, ks;
};
FwdVariant forward_variant(bool bf16, int d, int64_t B, int64_t H, int64_t n, int64_t m,
                           int mode);

}  // namespace mha
