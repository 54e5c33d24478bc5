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

}  // namespace

extern "C" {

int mha_abi_version(void) { return MHA_ABI_VERSION; }

const char* mha_status_string(int s) {
  switch (s) {
    case MHA_OK: return "ok";
    case MHA_ERR_NULL: return "a required pointer is NULL";
    case MHA_ERR_SHAPE: return "bad shape: negative size, or causal with n != m";
    case MHA_ERR_DTYPE: return "dtype must be MHA_F32 or MHA_BF16";
    case MHA_ERR_UNSUPPORTED:
      return "unsupported: needs d_k == d_v in {64, 128} and per-head tensors under 2 GiB";
    case MHA_ERR_SCALE: return "scale must be finite and > 0";
    case MHA_ERR_ALIAS: return "O overlaps Q, K, V or key_lens";
    case MHA_ERR_HIP: return "the HIP runtime refused the kernel launch";
    case MHA_ERR_ALIGN: return "Q, K, V and O must be 16-byte aligned";
    default: return "unknown status";
  }
}

int mha_validate(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                 int causal, float scale, const void* O, int64_t B, int64_t H, int64_t n,
                 int64_t m, int64_t d_k, int64_t d_v, int dtype) {
  if (B < 0 || H < 0 || n < 0 || m < 0 || d_k < 0 || d_v < 0) return MHA_ERR_SHAPE;
  if (dtype != MHA_F32 && dtype != MHA_BF16) return MHA_ERR_DTYPE;
  if (causal && n != m) return MHA_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return MHA_ERR_SCALE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return MHA_ERR_UNSUPPORTED;
  const int64_t es = dtype == MHA_BF16 ? 2 : 4;
  if (n * d_k * es >= kMaxHeadBytes || m * d_k * es >= kMaxHeadBytes) return MHA_ERR_UNSUPPORTED;
  const int64_t rows_per_block = 128;
  const int64_t blocks = ((n + rows_per_block - 1) / rows_per_block) * B * H;
  if (B > INT32_MAX || H > INT32_MAX || blocks > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  const int64_t q_bytes = B * H * n * d_k * es;
  const int64_t kv_bytes = B * H * m * d_k * es;
  const int64_t o_bytes = B * H * n * d_v * es;
  if ((q_bytes > 0 && Q == nullptr) || (kv_bytes > 0 && (K == nullptr || V == nullptr)) ||
      (o_bytes > 0 && O == nullptr))
    return MHA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return MHA_ERR_ALIGN;
  if (overlaps(O, o_bytes, Q, q_bytes) || overlaps(O, o_bytes, K, kv_bytes) ||
      overlaps(O, o_bytes, V, kv_bytes) || overlaps(O, o_bytes, key_lens, 4 * B))
    return MHA_ERR_ALIAS;
  return MHA_OK;
}

int mha_forward(const void* Q, const void* K, const void* V, const int32_t* key_lens,
                int causal, float scale, void* O, int64_t B, int64_t H, int64_t n, int64_t m,
                int64_t d_k, int64_t d_v, int dtype, void* stream) {
  const int st = mha_validate(Q, K, V, key_lens, causal, scale, O, B, H, n, m, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  if (B == 0 || H == 0 || n == 0) return MHA_OK;
  mha::LaunchArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.key_lens = key_lens;
  a.O = O;
  a.B = B;
  a.H = H;
  a.n = n;
  a.m = m;
  a.d = (int)d_k;
  a.bf16 = dtype == MHA_BF16;
  a.causal = causal != 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.stream = stream;
  return mha::launch_attention(a) == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

}  // extern "C"
