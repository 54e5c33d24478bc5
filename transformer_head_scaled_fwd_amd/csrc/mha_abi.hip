// mha_abi.hip -- the launching entry points of the C ABI declared in
// include/libmha.h.  Each runs the host-side argument check of mha_host.cpp
// first (no HIP call before it passes) and then enqueues the kernels.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "libmha.h"
#include "mha_host.h"
#include "mha_launch.h"

namespace {

mha_status launch_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                   int mode, const float* alibi, float scale, void* O, float* lse, int64_t B,
                   int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k, mha_dtype dtype,
                   void* stream) {
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  mha::LaunchArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.key_lens = key_lens;
  a.O = O;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.n = n;
  a.m = m;
  a.d = (int)d_k;
  a.bf16 = dtype == MHA_BF16;
  a.mode = mode;
  a.alibi_slopes = alibi;
  a.lse = lse;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.stream = stream;
  return mha::launch_attention(a) == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

}  // namespace

extern "C" {

mha_status mha_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                int causal, float scale, void* O, int64_t B, int64_t H, int64_t n, int64_t m,
                int64_t d_k, int64_t d_v, mha_dtype dtype, void* stream) {
  const mha_status st = mha_validate(Q, K, V, key_lens, causal, scale, O, B, H, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  return launch_forward(Q, K, V, key_lens, causal ? MHA_MASK_CAUSAL : MHA_MASK_NONE, nullptr,
                        scale, O, nullptr, B, H, H, n, m, d_k, dtype, stream);
}

mha_status mha_forward_ex(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                   int mask_mode, const float* alibi_slopes, float scale, void* O, float* lse,
                   int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                   int64_t d_v, mha_dtype dtype, void* stream) {
  const mha_status st = mha::check_forward(Q, K, V, key_lens, mask_mode, alibi_slopes, scale, O, lse, B, H,
                               H_kv, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  return launch_forward(Q, K, V, key_lens, mask_mode, alibi_slopes, scale, O, lse, B, H, H_kv, n,
                        m, d_k, dtype, stream);
}

mha_status mha_attention_weights(const void* Q, const void* K, const int32_t* key_lens, int mask_mode,
                          const float* alibi_slopes, float scale, const float* lse, void* A,
                          int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                          int64_t d_k, mha_dtype dtype, void* stream) {
  const mha_status st = mha_validate_weights(Q, K, key_lens, mask_mode, alibi_slopes, scale, lse, A, B,
                                      H, H_kv, n, m, d_k, dtype);
  if (st != MHA_OK) return st;
  if (B == 0 || H == 0 || n == 0 || m == 0) return MHA_OK;
  mha::WeightsArgs a;
  a.Q = Q;
  a.K = K;
  a.key_lens = key_lens;
  a.alibi_slopes = alibi_slopes;
  a.lse = lse;
  a.A = A;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.n = n;
  a.m = m;
  a.d = (int)d_k;
  a.bf16 = dtype == MHA_BF16;
  a.mode = mask_mode;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.stream = stream;
  return mha::launch_weights(a) == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

}  // extern "C"

namespace {

// The decode launch once the arguments have passed their check;
// `workspace` is the caller's or the library's scratch.
mha_status launch_decode_checked(const void* Q, const void* K, const void* V,
                                 const int32_t* cache_lens, const float* alibi_slopes,
                                 float scale, void* O, float* lse, void* workspace, int64_t B,
                                 int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                                 mha_dtype dtype, const mha::DecodePlan& p, void* stream) {
  mha::DecodeArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.cache_lens = cache_lens;
  a.alibi_slopes = alibi_slopes;
  a.O = O;
  a.lse = lse;
  a.workspace = workspace;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.n = n;
  a.m = m;
  a.d = (int)d_k;
  a.bf16 = dtype == MHA_BF16;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.stream = stream;
  return mha::launch_decode(a, p) == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

}  // namespace

extern "C" {

mha_status mha_decode(const void* Q, const void* K, const void* V, const int32_t* cache_lens,
                      const float* alibi_slopes, float scale, void* O, float* lse,
                      void* workspace, int64_t workspace_bytes, int64_t B, int64_t H,
                      int64_t H_kv, int64_t n, int64_t m, int64_t d_k, int64_t d_v,
                      mha_dtype dtype, void* stream) {
  const mha_status st = mha_validate_decode(Q, K, V, cache_lens, alibi_slopes, scale, O, lse,
                                            workspace, workspace_bytes, B, H, H_kv, n, m, d_k,
                                            d_v, dtype);
  if (st != MHA_OK) return st;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  const mha::DecodePlan p = mha::plan_decode(B, H, H_kv, n, m, (int)d_k, dtype == MHA_BF16);
  return launch_decode_checked(Q, K, V, cache_lens, alibi_slopes, scale, O, lse, workspace, B, H,
                               H_kv, n, m, d_k, dtype, p, stream);
}

mha_status mha_decode_noalloc(const void* Q, const void* K, const void* V,
                              const int32_t* cache_lens, const float* alibi_slopes, float scale,
                              void* O, float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t n,
                              int64_t m, int64_t d_k, int64_t d_v, mha_dtype dtype,
                              void* stream) {
  const mha_status st = mha::check_decode_noalloc(Q, K, V, cache_lens, alibi_slopes, scale, O,
                                                  lse, B, H, H_kv, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  const mha::DecodePlan p = mha::plan_decode(B, H, H_kv, n, m, (int)d_k, dtype == MHA_BF16);
  void* scratch = nullptr;
  if (p.workspace_bytes > 0 && mha::decode_scratch_address(&scratch) != hipSuccess)
    return MHA_ERR_HIP;
  return launch_decode_checked(Q, K, V, cache_lens, alibi_slopes, scale, O, lse, scratch, B, H,
                               H_kv, n, m, d_k, dtype, p, stream);
}

mha_status mha_multihead_forward(const void* Xq, const void* Xk, const void* Xv, const void* Wq,
                          const void* bq, const void* Wk, const void* bk, const void* Wv,
                          const void* bv, const void* Wo, const void* bo,
                          const int32_t* key_lens, int mask_mode, float scale, void* Y, void* A,
                          void* workspace, int64_t workspace_bytes, int64_t B, int64_t n,
                          int64_t m, int64_t d_model, int64_t H, mha_dtype dtype, void* stream) {
  mha_status st = mha_validate_multihead(Xq, Xk, Xv, Wq, bq, Wk, bk, Wv, bv, Wo, bo, key_lens,
                                         mask_mode, scale, Y, A, workspace, workspace_bytes, B,
                                         n, m, d_model, H, dtype);
  if (st != MHA_OK || B == 0 || n == 0) return st;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  const int64_t dk = d_model / H;
  const mha::MhLayout lay = mha::mh_layout(B, n, m, d_model, H, es, A != nullptr);
  char* ws = static_cast<char*>(workspace);
  void* Q = ws + lay.q;
  void* K = ws + lay.k;
  void* V = ws + lay.v;
  void* O = ws + lay.o;
  float* lse = A ? reinterpret_cast<float*>(ws + lay.lse) : nullptr;
  const bool bf16 = dtype == MHA_BF16;

  // 1. Q, K, V projections, written head-split.
  mha::ProjBatch in;
  const void* xs[3] = {Xq, Xk, Xv};
  const void* ws_[3] = {Wq, Wk, Wv};
  const void* bs[3] = {bq, bk, bv};
  void* outs[3] = {Q, K, V};
  const int64_t Ls[3] = {n, m, m};
  for (int j = 0; j < 3; ++j) {
    mha::ProjProblem& p = in.p[j];
    p.A = xs[j];
    p.W = ws_[j];
    p.bias = bs[j];
    p.C = outs[j];
    p.M = (int)(B * Ls[j]);
    p.N = (int)d_model;
    p.K = (int)d_model;
    p.L = (int)(Ls[j] > 0 ? Ls[j] : 1);
    p.H = (int)H;
    p.dk = (int)dk;
    p.a_bytes = B * Ls[j] * d_model * es;
  }
  if (mha::launch_proj(in, 3, bf16, false, true, stream) != hipSuccess) return MHA_ERR_HIP;
  // 2. attention per head (and the row log-sum-exp when weights are asked for).
  st = launch_forward(Q, K, V, key_lens, mask_mode, nullptr, scale, O, lse, B, H, H, n, m, dk,
                      dtype, stream);
  if (st != MHA_OK) return st;
  // 3. the weights.
  if (A && m > 0) {
    st = mha_attention_weights(Q, K, key_lens, mask_mode, nullptr, scale, lse, A, B, H, H, n, m,
                               dk, dtype, stream);
    if (st != MHA_OK) return st;
  }
  // 4. concatenate the heads and project.
  mha::ProjBatch out;
  mha::ProjProblem& p = out.p[0];
  p.A = O;
  p.W = Wo;
  p.bias = bo;
  p.C = Y;
  p.M = (int)(B * n);
  p.N = (int)d_model;
  p.K = (int)d_model;
  p.L = (int)n;
  p.H = (int)H;
  p.dk = (int)dk;
  p.a_bytes = B * n * d_model * es;
  out.p[1] = out.p[0];
  out.p[2] = out.p[0];
  return mha::launch_proj(out, 1, bf16, true, false, stream) == hipSuccess ? MHA_OK
                                                                          : MHA_ERR_HIP;
}

}  // extern "C"
