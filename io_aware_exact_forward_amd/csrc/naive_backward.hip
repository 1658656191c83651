// Row passes of the stored-state attention backward: the conventional path
// that keeps the N x N probability matrix in HBM, against which "IO-aware
// exact attention" (section "Measure stored-state and recomputed attention
// backward") measures the recomputing backward.  The products around these
// passes are rocBLAS GEMMs (fa_api.cpp).  Deliberately plain: one workgroup
// per row, full sweeps over the row.
//
//   naive_bwd_p_kernel:  P_ij = exp(S_ij - LSE_i) on visible pairs, else 0,
//                        written over S (S already holds scale * q_i . k_j).
//   naive_bwd_ds_kernel: D_i = sum_j P_ij dP_ij, then dS_ij = P_ij (dP_ij - D_i),
//                        written over dP.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

__device__ __forceinline__ float ld_bf16(const uint16_t* p, int64_t i) {
  return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
}

__device__ float block_sum(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Visible keys of row i are j < jend (0 for padding rows).
__device__ __forceinline__ int row_end(const NaiveBwdParams& p, int64_t row, int* i_out) {
  const int N = p.N;
  const int i = (int)(row % N);
  const int b = (int)(row / N) / p.H;
  int L = N;
  if (p.key_len) {
    const int kl = p.key_len[b];
    L = kl < 0 ? 0 : (kl > N ? N : kl);
  }
  *i_out = i;
  if (i >= L) return 0;
  return p.causal ? min(i + 1, L) : L;
}

__global__ __launch_bounds__(256) void naive_bwd_p_kernel(NaiveBwdParams p) {
  const int64_t row = blockIdx.x;  // (b*H + h)*N + i
  int i;
  const int jend = row_end(p, row, &i);
  uint16_t* s = (uint16_t*)p.sp + row * (int64_t)p.N;
  const float lse = jend > 0 ? p.lse[row] : 0.f;
  for (int j = threadIdx.x; j < p.N; j += 256) {
    const float e = j < jend ? __expf(ld_bf16(s, j) - lse) : 0.f;
    ((__bf16*)s)[j] = (__bf16)e;
  }
}

__global__ __launch_bounds__(256) void naive_bwd_ds_kernel(NaiveBwdParams p) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  int i;
  const int jend = row_end(p, row, &i);
  const uint16_t* pm = (const uint16_t*)p.sp + row * (int64_t)p.N;
  uint16_t* dp = (uint16_t*)p.dpds + row * (int64_t)p.N;
  float part = 0.f;
  for (int j = threadIdx.x; j < jend; j += 256) part += ld_bf16(pm, j) * ld_bf16(dp, j);
  const float dsum = block_sum(part, red);
  for (int j = threadIdx.x; j < p.N; j += 256) {
    const float x = j < jend ? ld_bf16(pm, j) * (ld_bf16(dp, j) - dsum) : 0.f;
    ((__bf16*)dp)[j] = (__bf16)x;
  }
}

}  // namespace

hipError_t launch_naive_bwd_p(const NaiveBwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(naive_bwd_p_kernel, dim3((unsigned)((int64_t)p.B * p.H * p.N)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_naive_bwd_ds(const NaiveBwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(naive_bwd_ds_kernel, dim3((unsigned)((int64_t)p.B * p.H * p.N)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace fa
