// mha_launch.h -- internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

// Arguments after host validation; sizes fit the kernels' 32-bit offsets.
struct LaunchArgs {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* key_lens;  // device int32[B] or nullptr
  void* O;
  int64_t B, H, n, m;
  int d;                    // d_k == d_v, 64 or 128
  bool bf16;                // element type: bf16 (true) or fp32 (false)
  bool causal;
  float scale_log2;         // scale * log2(e)
  void* stream;             // hipStream_t
};

hipError_t launch_attention(const LaunchArgs& a);

}  // namespace mha
