// Sustained bf16 matrix-core rate of the device, for reading the attention
// kernels' throughput against what the chip delivers under a dense MFMA load
// (the engine clock settles below its 2.4 GHz maximum there).
//
// Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on operands held in
// registers (pseudo-random bf16 values that differ per lane, so that the
// multipliers toggle as they do on real data), rotating over four
// accumulators, and writes one sum per lane at the end so that nothing is
// optimised away.  This library is a measurement helper, separate from the
// attention library and its ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeWaves = 8;
constexpr int kMfmaPerIter = 16;

__global__ __launch_bounds__(64 * kProbeWaves, 1) void mfma_probe_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  bf16x8 a[4], b[4];
  uint32_t x = (uint32_t)(blockIdx.x * 1024 + tid) * 2654435761u + 12345u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // xorshift32: values in [-1, 1)
      x ^= x << 13;
      x ^= x >> 17;
      x ^= x << 5;
      a[j][i] = (__bf16)((float)(int)(x & 0xFFFF) * (1.0f / 32768.f) - 1.0f);
      x ^= x << 13;
      x ^= x >> 17;
      x ^= x << 5;
      b[j][i] = (__bf16)((float)(int)(x & 0xFFFF) * (1.0f / 32768.f) - 1.0f);
    }
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaPerIter; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j >> 2) & 3], b[(j + (j >> 2)) & 3],
                                                          acc[j & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(size_t)blockIdx.x * blockDim.x + tid] = s;
}

}  // namespace

// Launches `blocks` workgroups of 8 waves, each wave issuing 16 * iters MFMAs
// (2 * 32 * 32 * 16 flops each) on `stream`; out (device) receives
// blocks * 512 floats.  Returns 0, -1 for invalid arguments (nothing is
// launched), or -2 when the launch fails.
extern "C" int fa_probe_mfma_bf16(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(64 * kProbeWaves), 0,
                     (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Flops of one launch with these arguments.
extern "C" double fa_probe_mfma_flops(int blocks, int iters) {
  return 2.0 * 32 * 32 * 16 * kMfmaPerIter * (double)iters * kProbeWaves * blocks;
}
