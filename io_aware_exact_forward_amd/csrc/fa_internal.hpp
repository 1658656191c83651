// Internal interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a forward kernel needs, passed by value as one kernel argument.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* key_len;  // device [B] or nullptr
  int B, H, N;
  int n_qtiles;            // ceil(N / query-tile rows)
  float c;                 // |scale| * log2(e): scores enter exp2 in log2 units
  uint32_t q_sign;         // sign bits xor-ed into Q when scale < 0 (0 otherwise)
};

// Parameters of the materialised (three-pass) path's softmax pass.
struct NaiveSoftmaxParams {
  const void* s;           // [B*H, N, N] scores already multiplied by scale
  void* p;                 // [B*H, N, N] probabilities (same dtype as s)
  float* lse;              // [B*H, N]
  const int32_t* key_len;  // device [B] or nullptr
  int B, H, N;
  int causal;
};

// Query rows per workgroup of the fused kernels.
constexpr int kQueryTile = 128;

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_naive_softmax(const NaiveSoftmaxParams& p, bool bf16, hipStream_t stream);

}  // namespace fa
