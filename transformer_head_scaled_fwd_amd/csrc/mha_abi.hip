// mha_abi.hip -- the C ABI declared in include/libmha.h: host-side argument
// checks (no HIP call before they pass) and dispatch to the kernels.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "libmha.h"
#include "mha_launch.h"

namespace {

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (a == nullptr || b == nullptr || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest byte extent one head's tensor may have: the kernels address a
// head with 32-bit buffer offsets.
constexpr int64_t kMaxHeadBytes = (int64_t)1 << 31;

// a * b for non-negative sizes, saturating at INT64_MAX instead of wrapping.
int64_t mul_sat(int64_t a, int64_t b) {
  if (a == 0 || b == 0) return 0;
  return a > INT64_MAX / b ? INT64_MAX : a * b;
}

// Byte extent a * b * c * d of a tensor, saturating: with an empty query
// axis nothing else bounds the batch and head counts.
int64_t extent(int64_t a, int64_t b, int64_t c, int64_t d) {
  return mul_sat(mul_sat(mul_sat(a, b), c), d);
}

// Whether `count` elements of `bytes_each` bytes stay under kMaxHeadBytes.
bool head_fits(int64_t count, int64_t bytes_each) {
  return count <= (kMaxHeadBytes - 1) / bytes_each;
}

// A dispatch counts its grid in work-items, in 32 bits: `blocks` workgroups
// of `threads` work-items each must stay within that.
bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= (int64_t)UINT32_MAX / threads;
}

// Shared checks of the forward entry points.  H_kv: K/V heads; mode 0/1/2.
int check_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens, int mode,
                  const float* alibi, float scale, const void* O, const float* lse, int64_t B,
                  int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k, int64_t d_v,
                  int dtype) {
  if (B < 0 || H < 0 || H_kv < 0 || n < 0 || m < 0 || d_k < 0 || d_v < 0) return MHA_ERR_SHAPE;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (dtype != MHA_F32 && dtype != MHA_BF16) return MHA_ERR_DTYPE;
  if (mode < MHA_MASK_NONE || mode > MHA_MASK_CAUSAL_BOTTOM_RIGHT) return MHA_ERR_MODE;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return MHA_ERR_SCALE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return MHA_ERR_UNSUPPORTED;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (!head_fits(n, d_k * es) || !head_fits(m, d_k * es)) return MHA_ERR_UNSUPPORTED;
  // Grid: workgroups of 4 waves over 128 query rows (the launcher takes 8
  // waves over 256 rows only where that grid fits as well).
  if (B > INT32_MAX || H > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  if (!grid_fits(mul_sat(mul_sat((n + 127) / 128, B), H), 256)) return MHA_ERR_UNSUPPORTED;
  const int64_t q_bytes = extent(B, H, n, d_k * es);
  const int64_t kv_bytes = extent(B, H_kv, m, d_k * es);
  const int64_t o_bytes = extent(B, H, n, d_v * es);
  const int64_t lse_bytes = lse ? extent(B, H, n, 4) : 0;
  const int64_t alibi_bytes = alibi ? H * 4 : 0;
  const int64_t lens_bytes = mul_sat(B, 4);
  if ((q_bytes > 0 && Q == nullptr) || (kv_bytes > 0 && (K == nullptr || V == nullptr)) ||
      (o_bytes > 0 && O == nullptr))
    return MHA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return MHA_ERR_ALIGN;
  if (((uintptr_t)lse & 3u) || ((uintptr_t)alibi & 3u)) return MHA_ERR_ALIGN;
  if (overlaps(O, o_bytes, Q, q_bytes) || overlaps(O, o_bytes, K, kv_bytes) ||
      overlaps(O, o_bytes, V, kv_bytes) || overlaps(O, o_bytes, key_lens, lens_bytes) ||
      overlaps(O, o_bytes, alibi, alibi_bytes) || overlaps(O, o_bytes, lse, lse_bytes))
    return MHA_ERR_ALIAS;
  if (overlaps(lse, lse_bytes, Q, q_bytes) || overlaps(lse, lse_bytes, K, kv_bytes) ||
      overlaps(lse, lse_bytes, V, kv_bytes) || overlaps(lse, lse_bytes, key_lens, lens_bytes) ||
      overlaps(lse, lse_bytes, alibi, alibi_bytes))
    return MHA_ERR_ALIAS;
  return MHA_OK;
}

int launch_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                   int mode, const float* alibi, float scale, void* O, float* lse, int64_t B,
                   int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k, int dtype,
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

int mha_abi_version(void) { return MHA_ABI_VERSION; }

const char* mha_status_string(int s) {
  switch (s) {
    case MHA_OK: return "ok";
    case MHA_ERR_NULL: return "a required pointer is NULL";
    case MHA_ERR_SHAPE:
      return "bad shape: negative size, H not a multiple of H_kv, or causal with n != m";
    case MHA_ERR_DTYPE: return "dtype must be MHA_F32 or MHA_BF16";
    case MHA_ERR_UNSUPPORTED:
      return "unsupported: needs d_k == d_v in {64, 128} and per-head tensors under 2 GiB";
    case MHA_ERR_SCALE: return "scale must be finite and > 0";
    case MHA_ERR_ALIAS: return "an output (O, lse or A) overlaps another argument";
    case MHA_ERR_HIP: return "the HIP runtime refused the kernel launch";
    case MHA_ERR_ALIGN:
      return "Q, K, V, O (and A) must be 16-byte aligned; lse and alibi_slopes 4-byte aligned";
    case MHA_ERR_MODE: return "mask_mode must be MHA_MASK_NONE, _CAUSAL or _CAUSAL_BOTTOM_RIGHT";
    case MHA_ERR_WORKSPACE: return "workspace missing, too small, misaligned or overlapping";
    default: return "unknown status";
  }
}

int mha_validate(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                 int causal, float scale, const void* O, int64_t B, int64_t H, int64_t n,
                 int64_t m, int64_t d_k, int64_t d_v, int dtype) {
  if (causal && n != m && n >= 0 && m >= 0) return MHA_ERR_SHAPE;
  return check_forward(Q, K, V, key_lens, causal ? MHA_MASK_CAUSAL : MHA_MASK_NONE, nullptr,
                       scale, O, nullptr, B, H, H, n, m, d_k, d_v, dtype);
}

int mha_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                int causal, float scale, void* O, int64_t B, int64_t H, int64_t n, int64_t m,
                int64_t d_k, int64_t d_v, int dtype, void* stream) {
  const int st = mha_validate(Q, K, V, key_lens, causal, scale, O, B, H, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  return launch_forward(Q, K, V, key_lens, causal ? MHA_MASK_CAUSAL : MHA_MASK_NONE, nullptr,
                        scale, O, nullptr, B, H, H, n, m, d_k, dtype, stream);
}

int mha_validate_ex(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                    int mask_mode, const float* alibi_slopes, float scale, const void* O,
                    const float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                    int64_t d_k, int64_t d_v, int dtype) {
  return check_forward(Q, K, V, key_lens, mask_mode, alibi_slopes, scale, O, lse, B, H, H_kv, n,
                       m, d_k, d_v, dtype);
}

int mha_forward_ex(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                   int mask_mode, const float* alibi_slopes, float scale, void* O, float* lse,
                   int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                   int64_t d_v, int dtype, void* stream) {
  const int st = check_forward(Q, K, V, key_lens, mask_mode, alibi_slopes, scale, O, lse, B, H,
                               H_kv, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  return launch_forward(Q, K, V, key_lens, mask_mode, alibi_slopes, scale, O, lse, B, H, H_kv, n,
                        m, d_k, dtype, stream);
}

int mha_validate_weights(const void* Q, const void* K, const int32_t* key_lens, int mask_mode,
                         const float* alibi_slopes, float scale, const float* lse,
                         const void* A, int64_t B, int64_t H, int64_t H_kv, int64_t n,
                         int64_t m, int64_t d_k, int dtype) {
  if (B < 0 || H < 0 || H_kv < 0 || n < 0 || m < 0 || d_k < 0) return MHA_ERR_SHAPE;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (dtype != MHA_F32 && dtype != MHA_BF16) return MHA_ERR_DTYPE;
  if (mask_mode < MHA_MASK_NONE || mask_mode > MHA_MASK_CAUSAL_BOTTOM_RIGHT) return MHA_ERR_MODE;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return MHA_ERR_SCALE;
  if (d_k != 64 && d_k != 128) return MHA_ERR_UNSUPPORTED;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (!head_fits(n, d_k * es) || !head_fits(m, d_k * es)) return MHA_ERR_UNSUPPORTED;
  if (n > 0 && m > 0 && !head_fits(mul_sat(n, m), es)) return MHA_ERR_UNSUPPORTED;
  if (B > INT32_MAX || H > INT32_MAX || !grid_fits(mul_sat(mul_sat((n + 127) / 128, B), H), 256))
    return MHA_ERR_UNSUPPORTED;
  const int64_t q_bytes = extent(B, H, n, d_k * es);
  const int64_t k_bytes = extent(B, H_kv, m, d_k * es);
  const int64_t a_bytes = extent(B, H, mul_sat(n, m), es);
  const int64_t lse_bytes = extent(B, H, n, 4);
  const int64_t alibi_bytes = alibi_slopes ? H * 4 : 0;
  if (a_bytes > 0 && (Q == nullptr || K == nullptr || lse == nullptr || A == nullptr))
    return MHA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(A)) return MHA_ERR_ALIGN;
  if (((uintptr_t)lse & 3u) || ((uintptr_t)alibi_slopes & 3u)) return MHA_ERR_ALIGN;
  if (overlaps(A, a_bytes, Q, q_bytes) || overlaps(A, a_bytes, K, k_bytes) ||
      overlaps(A, a_bytes, key_lens, mul_sat(B, 4)) ||
      overlaps(A, a_bytes, alibi_slopes, alibi_bytes) ||
      overlaps(A, a_bytes, lse, lse_bytes))
    return MHA_ERR_ALIAS;
  return MHA_OK;
}

int mha_attention_weights(const void* Q, const void* K, const int32_t* key_lens, int mask_mode,
                          const float* alibi_slopes, float scale, const float* lse, void* A,
                          int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                          int64_t d_k, int dtype, void* stream) {
  const int st = mha_validate_weights(Q, K, key_lens, mask_mode, alibi_slopes, scale, lse, A, B,
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

int mha_decode_workspace_size(int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                              int64_t d, int dtype, int64_t* bytes) {
  if (bytes == nullptr) return MHA_ERR_NULL;
  *bytes = 0;
  if (B < 0 || H < 0 || H_kv < 0 || n < 0 || m < 0 || d < 0) return MHA_ERR_SHAPE;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (dtype != MHA_F32 && dtype != MHA_BF16) return MHA_ERR_DTYPE;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  *bytes = mha::plan_decode(B, H, H_kv, n, m, (int)d, dtype == MHA_BF16).workspace_bytes;
  return MHA_OK;
}

int mha_validate_decode(const void* Q, const void* K, const void* V, const int32_t* cache_lens,
                        const float* alibi_slopes, float scale, const void* O, const float* lse,
                        const void* workspace, int64_t workspace_bytes, int64_t B, int64_t H,
                        int64_t H_kv, int64_t n, int64_t m, int64_t d_k, int64_t d_v,
                        int dtype) {
  int st = check_forward(Q, K, V, cache_lens, MHA_MASK_CAUSAL_BOTTOM_RIGHT, alibi_slopes, scale,
                         O, lse, B, H, H_kv, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (!head_fits(mul_sat(H, n), d_k * es)) return MHA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  const mha::DecodePlan p = mha::plan_decode(B, H, H_kv, n, m, (int)d_k, dtype == MHA_BF16);
  // Grids: the decode kernel (at most 4 waves per workgroup) and the merge
  // of the splits (4 rows per 256 work-items).
  const int64_t rows = mul_sat(mul_sat(B, H), n);
  if (rows > INT32_MAX || !grid_fits(mul_sat(mul_sat(mul_sat(B, H_kv), p.nrs), p.nsplit), 256) ||
      !grid_fits((rows + 3) / 4, 256))
    return MHA_ERR_UNSUPPORTED;
  if (p.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < p.workspace_bytes || !aligned16(workspace))
      return MHA_ERR_WORKSPACE;
    const int64_t wb = p.workspace_bytes;
    const int64_t q_bytes = extent(B, H, n, d_k * es);
    const int64_t kv_bytes = extent(B, H_kv, m, d_k * es);
    if (overlaps(workspace, wb, Q, q_bytes) || overlaps(workspace, wb, K, kv_bytes) ||
        overlaps(workspace, wb, V, kv_bytes) || overlaps(workspace, wb, O, q_bytes) ||
        overlaps(workspace, wb, cache_lens, mul_sat(B, 4)) ||
        overlaps(workspace, wb, alibi_slopes, alibi_slopes ? 4 * H : 0) ||
        overlaps(workspace, wb, lse, lse ? extent(B, H, n, 4) : 0))
      return MHA_ERR_WORKSPACE;
  }
  return MHA_OK;
}

int mha_decode(const void* Q, const void* K, const void* V, const int32_t* cache_lens,
               const float* alibi_slopes, float scale, void* O, float* lse, void* workspace,
               int64_t workspace_bytes, int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
               int64_t d_k, int64_t d_v, int dtype, void* stream) {
  const int st = mha_validate_decode(Q, K, V, cache_lens, alibi_slopes, scale, O, lse, workspace,
                                     workspace_bytes, B, H, H_kv, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  const mha::DecodePlan p = mha::plan_decode(B, H, H_kv, n, m, (int)d_k, dtype == MHA_BF16);
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

namespace {

// Workspace of the multi-head forward: Q, K, V, O in [B, H, L, d_k], then
// the row log-sum-exp when the weights are requested; each part 256-byte
// aligned.
struct MhLayout {
  int64_t q, k, v, o, lse, total;
};

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

MhLayout mh_layout(int64_t B, int64_t n, int64_t m, int64_t d_model, int64_t H, int64_t es,
                   bool weights) {
  MhLayout l;
  l.q = 0;
  l.k = l.q + round256(B * n * d_model * es);
  l.v = l.k + round256(B * m * d_model * es);
  l.o = l.v + round256(B * m * d_model * es);
  l.lse = l.o + round256(B * n * d_model * es);
  l.total = l.lse + (weights ? round256(B * H * n * 4) : 0);
  return l;
}

int check_multihead_sizes(int64_t B, int64_t n, int64_t m, int64_t d_model, int64_t H,
                          int dtype) {
  if (B < 0 || n < 0 || m < 0 || d_model < 0 || H < 0) return MHA_ERR_SHAPE;
  if (dtype != MHA_F32 && dtype != MHA_BF16) return MHA_ERR_DTYPE;
  if (H == 0 || d_model % H != 0) return MHA_ERR_SHAPE;
  const int64_t dk = d_model / H;
  if (dk != 64 && dk != 128) return MHA_ERR_UNSUPPORTED;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (!head_fits(mul_sat(mul_sat(B, n), d_model), es) ||
      !head_fits(mul_sat(mul_sat(B, m), d_model), es) || !head_fits(mul_sat(d_model, d_model), es))
    return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

}  // namespace

int mha_multihead_workspace_size(int64_t B, int64_t n, int64_t m, int64_t d_model, int64_t H,
                                 int dtype, int need_weights, int64_t* bytes) {
  if (bytes == nullptr) return MHA_ERR_NULL;
  *bytes = 0;
  const int st = check_multihead_sizes(B, n, m, d_model, H, dtype);
  if (st != MHA_OK) return st;
  *bytes = mh_layout(B, n, m, d_model, H, dtype == MHA_BF16 ? 2 : 4, need_weights != 0).total;
  return MHA_OK;
}

int mha_multihead_forward(const void* Xq, const void* Xk, const void* Xv, const void* Wq,
                          const void* bq, const void* Wk, const void* bk, const void* Wv,
                          const void* bv, const void* Wo, const void* bo,
                          const int32_t* key_lens, int mask_mode, float scale, void* Y, void* A,
                          void* workspace, int64_t workspace_bytes, int64_t B, int64_t n,
                          int64_t m, int64_t d_model, int64_t H, int dtype, void* stream) {
  int st = check_multihead_sizes(B, n, m, d_model, H, dtype);
  if (st != MHA_OK) return st;
  if (mask_mode < MHA_MASK_NONE || mask_mode > MHA_MASK_CAUSAL_BOTTOM_RIGHT) return MHA_ERR_MODE;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return MHA_ERR_SCALE;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  const int64_t dk = d_model / H;
  const int64_t xq_b = B * n * d_model * es, xkv_b = B * m * d_model * es;
  const int64_t w_b = d_model * d_model * es, b_b = d_model * es;
  const int64_t a_b = A ? B * H * n * m * es : 0;
  if (B == 0 || n == 0) return MHA_OK;
  if (Xq == nullptr || Y == nullptr || Wq == nullptr || Wo == nullptr) return MHA_ERR_NULL;
  if (m > 0 && (Xk == nullptr || Xv == nullptr || Wk == nullptr || Wv == nullptr))
    return MHA_ERR_NULL;
  const void* t16[] = {Xq, Xk, Xv, Wq, Wk, Wv, Wo, Y, A, workspace};
  for (const void* p : t16)
    if (!aligned16(p)) return MHA_ERR_ALIGN;
  const void* bias[] = {bq, bk, bv, bo};
  for (const void* p : bias)
    if ((uintptr_t)p % es) return MHA_ERR_ALIGN;
  if (A && !head_fits(mul_sat(n, m), es)) return MHA_ERR_UNSUPPORTED;
  // Outputs must not overlap any input or each other.
  struct R { const void* p; int64_t b; } ins[] = {
      {Xq, xq_b}, {Xk, xkv_b}, {Xv, xkv_b}, {Wq, w_b}, {Wk, w_b}, {Wv, w_b}, {Wo, w_b},
      {bq, bq ? b_b : 0}, {bk, bk ? b_b : 0}, {bv, bv ? b_b : 0}, {bo, bo ? b_b : 0},
      {key_lens, key_lens ? 4 * B : 0}};
  const MhLayout lay = mh_layout(B, n, m, d_model, H, es, A != nullptr);
  if (workspace == nullptr || workspace_bytes < lay.total) return MHA_ERR_WORKSPACE;
  for (const R& r : ins) {
    if (overlaps(Y, xq_b, r.p, r.b) || overlaps(A, a_b, r.p, r.b)) return MHA_ERR_ALIAS;
    if (overlaps(workspace, lay.total, r.p, r.b)) return MHA_ERR_WORKSPACE;
  }
  if (overlaps(Y, xq_b, A, a_b)) return MHA_ERR_ALIAS;
  if (overlaps(workspace, lay.total, Y, xq_b) || overlaps(workspace, lay.total, A, a_b))
    return MHA_ERR_WORKSPACE;

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
