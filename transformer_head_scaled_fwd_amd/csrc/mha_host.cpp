// mha_host.cpp -- the host-only half of the C ABI declared in
// include/libmha.h: every argument check (no HIP call is made before one
// passes), the workspace sizes, the status strings, and the plans and
// kernel choices the launchers follow.  Plain C++; it includes no HIP
// header, so it also builds for the host alone (the tests build it with
// address and undefined-behaviour sanitizers).

#include <cmath>
#include <cstdint>

#include "libmha.h"
#include "mha_host.h"

namespace {

// Query rows per wave and keys per block of the kernels (their tile sizes).
constexpr int64_t kRowsPerWave = 32;
constexpr int64_t kKeysPerBlock = 64;

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

bool bad_dtype(mha_dtype dtype) { return dtype != MHA_F32 && dtype != MHA_BF16; }
bool bad_mode(int mode) { return mode < MHA_MASK_NONE || mode > MHA_MASK_CAUSAL_BOTTOM_RIGHT; }
bool bad_scale(float scale) { return !std::isfinite(scale) || !(scale > 0.0f); }

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1.
int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0); }

// Sizes the decode kernels can index (shapes already valid): every head
// and the queries of one K/V head's group under 2 GiB, B * H * n rows in
// 32 bits, and the grids of the decode kernel (at most 4 waves per
// workgroup) and of the merge of the splits (4 rows per 256 work-items).
// The row bounds come first: with them the plan's products stay far inside
// 64 bits.
mha_status check_decode_sizes(int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d,
                              bool bf16) {
  const int64_t es = bf16 ? 2 : 4;
  if (B > INT32_MAX || H > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  if (!head_fits(n, d * es) || !head_fits(m, d * es) || !head_fits(mul_sat(H, n), d * es))
    return MHA_ERR_UNSUPPORTED;
  const int64_t rows = mul_sat(mul_sat(B, H), n);
  if (rows > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  const mha::DecodePlan p = mha::plan_decode(B, H, H_kv, n, m, (int)d, bf16);
  if (!grid_fits(mul_sat(mul_sat(mul_sat(B, H_kv), p.nrs), p.nsplit), 256))
    return MHA_ERR_UNSUPPORTED;
  // the split merge: one 256-thread workgroup per query row
  if (p.nsplit > 1 && !grid_fits(rows, 256)) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

}  // namespace

namespace mha {

mha_status check_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens, int mode,
                  const float* alibi, float scale, const void* O, const float* lse, int64_t B,
                  int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k, int64_t d_v,
                  mha_dtype dtype) {
  if (B < 0 || H < 0 || H_kv < 0 || n < 0 || m < 0 || d_k < 0 || d_v < 0) return MHA_ERR_SHAPE;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (bad_dtype(dtype)) return MHA_ERR_DTYPE;
  if (bad_mode(mode)) return MHA_ERR_MODE;
  if (bad_scale(scale)) return MHA_ERR_SCALE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return MHA_ERR_UNSUPPORTED;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (!head_fits(n, d_k * es) || !head_fits(m, d_k * es)) return MHA_ERR_UNSUPPORTED;
  // Grid: workgroups of 4 waves over 128 query rows (the launcher takes 8
  // waves over 256 rows only where that grid fits as well).
  if (B > INT32_MAX || H > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  if (!grid_fits(mul_sat(mul_sat(cdiv(n, 128), B), H), 256)) return MHA_ERR_UNSUPPORTED;
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

DecodePlan plan_decode(int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m, int d,
                       bool bf16) {
  DecodePlan p;
  const int nw = (!bf16 && d == 128) ? 2 : 4;
  const int64_t R = (H / H_kv) * n;
  p.nrs = (R + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t nkb = (m + kKeysPerBlock - 1) / kKeysPerBlock;
  const int64_t units = B * H_kv * p.nrs;
  // About one workgroup per CU of a 256-CU device (a workgroup's four K/V
  // tile pairs take 128 KiB of the CU's 160 KiB of LDS, so one is resident at
  // a time): each wave then streams several key blocks, the next block's
  // loads overlapping the current block's compute, instead of one block per
  // wave and several rounds of workgroups.  At least one key block per wave
  // in every split.
  const int64_t target = 256;
  int64_t nsplit = units >= target ? 1 : (target + units - 1) / units;
  const int64_t max_split = (nkb + nw - 1) / nw;
  if (nsplit > max_split) nsplit = max_split;
  if (nsplit < 1) nsplit = 1;
  int64_t sb = (nkb + nsplit - 1) / nsplit;
  sb = ((sb + nw - 1) / nw) * nw;
  if (sb < nw) sb = nw;
  p.split_blocks = sb;
  p.nsplit = nkb > 0 ? (nkb + sb - 1) / sb : 1;
  p.workspace_bytes = p.nsplit > 1 ? B * H * n * p.nsplit * ((int64_t)d + 2) * 4 : 0;
  return p;
}

mha_status check_decode_noalloc(const void* Q, const void* K, const void* V,
                                const int32_t* cache_lens, const float* alibi_slopes,
                                float scale, const void* O, const float* lse, int64_t B,
                                int64_t H, int64_t H_kv, int64_t n, int64_t m, int64_t d_k,
                                int64_t d_v, mha_dtype dtype) {
  mha_status st = check_forward(Q, K, V, cache_lens, MHA_MASK_CAUSAL_BOTTOM_RIGHT, alibi_slopes,
                                scale, O, lse, B, H, H_kv, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  st = check_decode_sizes(B, H, H_kv, n, m, d_k, dtype == MHA_BF16);
  if (st != MHA_OK || B == 0 || H == 0 || n == 0) return st;
  if (plan_decode(B, H, H_kv, n, m, (int)d_k, dtype == MHA_BF16).workspace_bytes >
      kDecodeScratchBytes)
    return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

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

mha_status check_multihead_sizes(int64_t B, int64_t n, int64_t m, int64_t d_model, int64_t H,
                          mha_dtype dtype) {
  if (B < 0 || n < 0 || m < 0 || d_model < 0 || H < 0) return MHA_ERR_SHAPE;
  if (bad_dtype(dtype)) return MHA_ERR_DTYPE;
  if (H == 0 || d_model % H != 0) return MHA_ERR_SHAPE;
  const int64_t dk = d_model / H;
  if (dk != 64 && dk != 128) return MHA_ERR_UNSUPPORTED;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (!head_fits(mul_sat(mul_sat(B, n), d_model), es) ||
      !head_fits(mul_sat(mul_sat(B, m), d_model), es) || !head_fits(mul_sat(d_model, d_model), es))
    return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

mha_status check_multihead(const void* Xq, const void* Xk, const void* Xv, const void* Wq,
                    const void* bq, const void* Wk, const void* bk, const void* Wv,
                    const void* bv, const void* Wo, const void* bo, const int32_t* key_lens,
                    int mask_mode, float scale, const void* Y, const void* A,
                    const void* workspace, int64_t workspace_bytes, int64_t B, int64_t n,
                    int64_t m, int64_t d_model, int64_t H, mha_dtype dtype) {
  const mha_status st = check_multihead_sizes(B, n, m, d_model, H, dtype);
  if (st != MHA_OK) return st;
  if (bad_mode(mask_mode)) return MHA_ERR_MODE;
  if (bad_scale(scale)) return MHA_ERR_SCALE;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  // Each product below is bounded: the size check keeps B*n*d_model and
  // B*m*d_model elements (and d_model^2) under 2 GiB.
  const int64_t xq_b = B * n * d_model * es, xkv_b = B * m * d_model * es;
  const int64_t w_b = d_model * d_model * es, b_b = d_model * es;
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
  if (A && (!head_fits(mul_sat(n, m), es) || H > INT32_MAX)) return MHA_ERR_UNSUPPORTED;
  const int64_t a_b = A ? extent(B, H, mul_sat(n, m), es) : 0;
  // Outputs must not overlap any input or each other.
  struct R {
    const void* p;
    int64_t b;
  } ins[] = {{Xq, xq_b},          {Xk, xkv_b},         {Xv, xkv_b},         {Wq, w_b},
             {Wk, w_b},           {Wv, w_b},           {Wo, w_b},           {bq, bq ? b_b : 0},
             {bk, bk ? b_b : 0},  {bv, bv ? b_b : 0},  {bo, bo ? b_b : 0},
             {key_lens, key_lens ? mul_sat(B, 4) : 0}};
  const MhLayout lay = mh_layout(B, n, m, d_model, H, es, A != nullptr);
  if (workspace == nullptr || workspace_bytes < lay.total) return MHA_ERR_WORKSPACE;
  for (const R& r : ins) {
    if (overlaps(Y, xq_b, r.p, r.b) || overlaps(A, a_b, r.p, r.b)) return MHA_ERR_ALIAS;
    if (overlaps(workspace, lay.total, r.p, r.b)) return MHA_ERR_WORKSPACE;
  }
  if (overlaps(Y, xq_b, A, a_b)) return MHA_ERR_ALIAS;
  if (overlaps(workspace, lay.total, Y, xq_b) || overlaps(workspace, lay.total, A, a_b))
    return MHA_ERR_WORKSPACE;
  return MHA_OK;
}

FastDiv fast_div(uint32_t d) {
  FastDiv f{d, 0, 0};
  if (d == 0) return f;  // not a divisor; callers pass d >= 1
  while (f.shift < 31 && (1u << f.shift) < d) ++f.shift;
  // ceil(2^(32 + shift) / d) - 2^32, below 2^32 for every d >= 1
  const uint64_t num = (uint64_t)1 << (32 + f.shift);
  f.mul = (uint32_t)((num + d - 1) / d - ((uint64_t)1 << 32));
  return f;
}

// Workgroup shape:
//  - 8 waves as 8 row groups (256 query rows, one workgroup per CU) for bf16
//    with d = 128 when the query axis gives every CU several workgroups and
//    the key walks are long (48 or more 64-key blocks on average): 8 waves
//    halve the K/V staging per query row.  On shorter walks 4-wave
//    workgroups, two per CU, win instead: one workgroup's prologue and
//    diagonal blocks overlap the other's steady state, and the causal
//    diagonal is cut at 128 rows.  (Measured, same process, 8 against 4
//    waves: causal n = 16384 -2.5%, 8192 -1.0%, 4096 +1.4..2.0%, 2048 +5.3%;
//    non-causal m = 16384 -3%, 8192 -2.5%, 4096 -0.5%, 2048 equal.)
//  - 8 waves as 4 row groups x 2 key groups (128 rows) for bf16 when 128-row
//    workgroups would leave one wave per SIMD (at most one workgroup per CU)
//    and the key axis is long (m >= 1024): one wave would walk all of it
//    serially, and splitting the walk halves the chain of dependent blocks.
//    The merge at the end costs about as much as three blocks of the walk,
//    so shorter walks keep one key group (measured: m = 256 and 512 lose
//    4-11%, m = 1024, 2048 and 4096 gain 4%, 9% and 12%);
//  - otherwise 4 waves (128 rows, two workgroups per CU).
FwdVariant forward_variant(bool bf16, int d, int64_t B, int64_t H, int64_t n, int64_t m,
                           int mode) {
  if (bf16) {
    if (d == 128) {
      const int64_t big_blocks = mul_sat(mul_sat(cdiv(n, 256), B), H);
      // Average key blocks a 256-row workgroup walks: all of them without a
      // causal mask; for a causal one, the visible keys of a middle row.
      const int64_t nn = n < m ? n : m;
      const int64_t walk = mode == MHA_MASK_NONE ? cdiv(m, 64)
                           : mode == MHA_MASK_CAUSAL
                               ? nn / 128 + 2
                               : (m > n / 2 ? (m - n / 2) / 64 : 0) + 2;
      if (big_blocks >= 4 * 256 && big_blocks <= (int64_t)UINT32_MAX / 512 && walk >= 48)
        return {8, 1};
    }
    const int64_t blocks = mul_sat(mul_sat(cdiv(n, 128), B), H);
    if (blocks <= 256 && m >= 16 * kKeysPerBlock) return {8, 2};
  }
  return {4, 1};
}

}  // namespace mha

extern "C" {

int mha_abi_version(void) { return MHA_ABI_VERSION; }

const char* mha_status_string(mha_status s) {
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

mha_status mha_validate(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                 int causal, float scale, const void* O, int64_t B, int64_t H, int64_t n,
                 int64_t m, int64_t d_k, int64_t d_v, mha_dtype dtype) {
  if (causal && n != m && n >= 0 && m >= 0) return MHA_ERR_SHAPE;
  return mha::check_forward(Q, K, V, key_lens, causal ? MHA_MASK_CAUSAL : MHA_MASK_NONE, nullptr,
                            scale, O, nullptr, B, H, H, n, m, d_k, d_v, dtype);
}

mha_status mha_validate_ex(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                    int mask_mode, const float* alibi_slopes, float scale, const void* O,
                    const float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                    int64_t d_k, int64_t d_v, mha_dtype dtype) {
  return mha::check_forward(Q, K, V, key_lens, mask_mode, alibi_slopes, scale, O, lse, B, H,
                            H_kv, n, m, d_k, d_v, dtype);
}

mha_status mha_validate_weights(const void* Q, const void* K, const int32_t* key_lens, int mask_mode,
                         const float* alibi_slopes, float scale, const float* lse,
                         const void* A, int64_t B, int64_t H, int64_t H_kv, int64_t n,
                         int64_t m, int64_t d_k, mha_dtype dtype) {
  if (B < 0 || H < 0 || H_kv < 0 || n < 0 || m < 0 || d_k < 0) return MHA_ERR_SHAPE;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (bad_dtype(dtype)) return MHA_ERR_DTYPE;
  if (bad_mode(mask_mode)) return MHA_ERR_MODE;
  if (bad_scale(scale)) return MHA_ERR_SCALE;
  if (d_k != 64 && d_k != 128) return MHA_ERR_UNSUPPORTED;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (!head_fits(n, d_k * es) || !head_fits(m, d_k * es)) return MHA_ERR_UNSUPPORTED;
  if (n > 0 && m > 0 && !head_fits(mul_sat(n, m), es)) return MHA_ERR_UNSUPPORTED;
  if (B > INT32_MAX || H > INT32_MAX || !grid_fits(mul_sat(mul_sat(cdiv(n, 128), B), H), 256))
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
      overlaps(A, a_bytes, alibi_slopes, alibi_bytes) || overlaps(A, a_bytes, lse, lse_bytes))
    return MHA_ERR_ALIAS;
  return MHA_OK;
}

mha_status mha_decode_workspace_size(int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                                     int64_t d, mha_dtype dtype, int64_t* bytes) {
  if (bytes == nullptr) return MHA_ERR_NULL;
  *bytes = 0;
  if (B < 0 || H < 0 || H_kv < 0 || n < 0 || m < 0 || d < 0) return MHA_ERR_SHAPE;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (bad_dtype(dtype)) return MHA_ERR_DTYPE;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;
  const mha_status st = check_decode_sizes(B, H, H_kv, n, m, d, dtype == MHA_BF16);
  if (st != MHA_OK) return st;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  *bytes = mha::plan_decode(B, H, H_kv, n, m, (int)d, dtype == MHA_BF16).workspace_bytes;
  return MHA_OK;
}

mha_status mha_validate_decode(const void* Q, const void* K, const void* V, const int32_t* cache_lens,
                        const float* alibi_slopes, float scale, const void* O, const float* lse,
                        const void* workspace, int64_t workspace_bytes, int64_t B, int64_t H,
                        int64_t H_kv, int64_t n, int64_t m, int64_t d_k, int64_t d_v,
                        mha_dtype dtype) {
  mha_status st = mha::check_forward(Q, K, V, cache_lens, MHA_MASK_CAUSAL_BOTTOM_RIGHT, alibi_slopes,
                              scale, O, lse, B, H, H_kv, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  st = check_decode_sizes(B, H, H_kv, n, m, d_k, dtype == MHA_BF16);
  if (st != MHA_OK) return st;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  const mha::DecodePlan p = mha::plan_decode(B, H, H_kv, n, m, (int)d_k, dtype == MHA_BF16);
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

mha_status mha_multihead_workspace_size(int64_t B, int64_t n, int64_t m, int64_t d_model, int64_t H,
                                 mha_dtype dtype, int need_weights, int64_t* bytes) {
  if (bytes == nullptr) return MHA_ERR_NULL;
  *bytes = 0;
  const mha_status st = mha::check_multihead_sizes(B, n, m, d_model, H, dtype);
  if (st != MHA_OK) return st;
  *bytes =
      mha::mh_layout(B, n, m, d_model, H, dtype == MHA_BF16 ? 2 : 4, need_weights != 0).total;
  return MHA_OK;
}

mha_status mha_validate_multihead(const void* Xq, const void* Xk, const void* Xv, const void* Wq,
                                  const void* bq, const void* Wk, const void* bk, const void* Wv,
                                  const void* bv, const void* Wo, const void* bo,
                                  const int32_t* key_lens, int mask_mode, float scale,
                                  const void* Y, const void* A, const void* workspace,
                                  int64_t workspace_bytes, int64_t B, int64_t n, int64_t m,
                                  int64_t d_model, int64_t H, mha_dtype dtype) {
  return mha::check_multihead(Xq, Xk, Xv, Wq, bq, Wk, bk, Wv, bv, Wo, bo, key_lens, mask_mode,
                              scale, Y, A, workspace, workspace_bytes, B, n, m, d_model, H,
                              dtype);
}

// Names of the forward kernel's instances, as the profilers print them:
// [dtype][d][variant (4 waves; 8 waves; 8 waves in two key groups)]
// [causal][alibi].
#define MHA_KN(T, D, NW, KS, C, A) "mha::attn_fwd_kernel<" T ", " #D ", " #NW ", " #KS ", " C ", " A ">"
#define MHA_KN4(T, D, NW, KS)                                                    \
  MHA_KN(T, D, NW, KS, "false", "false"), MHA_KN(T, D, NW, KS, "false", "true"), \
      MHA_KN(T, D, NW, KS, "true", "false"), MHA_KN(T, D, NW, KS, "true", "true")
#define MHA_KN12(T, D) MHA_KN4(T, D, 4, 1), MHA_KN4(T, D, 8, 1), MHA_KN4(T, D, 8, 2)
static const char* const kForwardKernelNames[48] = {MHA_KN12("float", 64), MHA_KN12("float", 128),
                                                    MHA_KN12("__bf16", 64),
                                                    MHA_KN12("__bf16", 128)};
#undef MHA_KN12
#undef MHA_KN4
#undef MHA_KN

const char* mha_forward_kernel_name(int64_t B, int64_t H, int64_t H_kv, int64_t n, int64_t m,
                                    int64_t d, mha_dtype dtype, int mask_mode, int alibi) {
  if (B < 0 || H < 0 || H_kv < 0 || n < 0 || m < 0 || (H > 0 && (H_kv == 0 || H % H_kv != 0)) ||
      bad_dtype(dtype) || bad_mode(mask_mode) || (d != 64 && d != 128))
    return nullptr;
  const bool bf16 = dtype == MHA_BF16;
  const mha::FwdVariant v = mha::forward_variant(bf16, (int)d, B, H, n, m, mask_mode);
  const int vi = v.nw == 4 ? 0 : (v.ks == 1 ? 1 : 2);
  const int causal = mask_mode != MHA_MASK_NONE;
  return kForwardKernelNames[(((bf16 ? 2 : 0) + (d == 128 ? 1 : 0)) * 3 + vi) * 4 + causal * 2 +
                             (alibi != 0)];
}

}  // extern "C"
