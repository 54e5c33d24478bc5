// mha_launch.h -- internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mha_host.h"

namespace mha {

// n / f.d for 0 <= n < 2^31 by a launch's divisor (FastDiv, mha_host.h): a
// multiply-high, an add and a shift.
__device__ __forceinline__ uint32_t div_by(uint32_t n, FastDiv f) {
  return (n + __umulhi(n, f.mul)) >> f.shift;
}

// Arguments after host validation; sizes fit the kernels' 32-bit offsets.
struct LaunchArgs {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* key_lens;  // device int32[B] or nullptr
  void* O;
  int64_t B, H, H_kv, n, m;  // H % H_kv == 0
  int d;                    // d_k == d_v, 64 or 128
  bool bf16;                // element type: bf16 (true) or fp32 (false)
  int mode;                 // 0 no causal mask, 1 causal top-left, 2 causal bottom-right
  const float* alibi_slopes;  // device fp32[H] or nullptr
  float* lse;               // device fp32[B, H, n] or nullptr
  float scale;              // scale applied to q.k
  float scale_log2;         // scale * log2(e)
  void* stream;             // hipStream_t
};

hipError_t launch_attention(const LaunchArgs& a);

// Arguments of the weights pass (A = exp(score - lse) over valid pairs).
struct WeightsArgs {
  const void* Q;
  const void* K;
  const int32_t* key_lens;    // device int32[B] or nullptr
  const float* alibi_slopes;  // device fp32[H] or nullptr
  const float* lse;           // device fp32[B, H, n] from the forward pass
  void* A;                    // device [B, H, n, m], element type of Q
  int64_t B, H, H_kv, n, m;
  int d;
  bool bf16;
  int mode;
  float scale, scale_log2;
  void* stream;
};

hipError_t launch_weights(const WeightsArgs& a);

// Arguments of the decode pass (few queries against a key/value cache).
struct DecodeArgs {
  const void* Q;              // [B, H, n, d]
  const void* K;              // [B, H_kv, m, d], m = cache capacity
  const void* V;
  const int32_t* cache_lens;  // device int32[B] or nullptr (= m)
  const float* alibi_slopes;  // device fp32[H] or nullptr
  void* O;                    // [B, H, n, d]
  float* lse;                 // device fp32[B, H, n] or nullptr
  void* workspace;            // DecodePlan::workspace_bytes, or nullptr when 0
  int64_t B, H, H_kv, n, m;
  int d;
  bool bf16;
  float scale, scale_log2;
  void* stream;
};

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p);

// Device address, on the current device, of the decode scratch array of
// kDecodeScratchBytes (looked up once per device).
hipError_t decode_scratch_address(void** ptr);

// One projection C = A W^T + bias: A [M, K] (or, with a_heads, the
// concatenation of [B, H, L, dk] heads), W [N, K], C [M, N] (or, with
// c_heads, split into [B, H, L, dk]); M = B * L.
struct ProjProblem {
  const void* A;
  const void* W;
  const void* bias;  // [N] or nullptr
  void* C;
  int M, N, K;
  int L, H, dk;      // tokens per sequence, heads, head width (head layouts)
  int64_t a_bytes;   // bytes of A (M * K * element size)
};
struct ProjBatch {
  ProjProblem p[3];
  int stream_out;    // C written through to memory (set by launch_proj)
};
hipError_t launch_proj(const ProjBatch& b, int count, bool bf16, bool a_heads, bool c_heads,
                       void* stream);

}  // namespace mha
