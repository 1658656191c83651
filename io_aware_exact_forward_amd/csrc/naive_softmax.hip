// Softmax pass of the materialised three-pass attention ("IO-aware exact
// attention", section "Traffic in the materialized implementation"): reads
// one full row of the stored score matrix S, applies the mask, and writes
// the full probability row P plus the row's log-sum-exp.  Deliberately
// plain: one workgroup per row, three sweeps over the row (max, sum, write).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (BF16) {
    const uint32_t u = ((const uint16_t*)base)[i];
    return __builtin_bit_cast(float, u << 16);
  } else {
    return ((const float*)base)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float x) {
  if constexpr (BF16) {
    ((__bf16*)base)[i] = (__bf16)x;
  } else {
    ((float*)base)[i] = x;
  }
}

template <bool MAX>
__device__ float block_reduce(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red[] may still be read from a previous reduction
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

template <bool BF16>
__global__ __launch_bounds__(256) void naive_softmax_kernel(NaiveSoftmaxParams p) {
  __shared__ float red[4];
  const int N = p.N;
  const int64_t row = blockIdx.x;  // (b*H + h)*N + i
  const int i = (int)(row % N);
  const int bh = (int)(row / N);
  const int b = bh / p.H;
  int L = N;
  if (p.key_len) {
    const int kl = p.key_len[b];
    L = kl < 0 ? 0 : (kl > N ? N : kl);
  }
  int jend = 0;  // visible keys are j < jend
  if (i < L) jend = p.causal ? min(i + 1, L) : L;
  const int64_t off = row * (int64_t)N;

  float mx = kNegInf;
  for (int j = threadIdx.x; j < jend; j += 256) mx = fmaxf(mx, load_elem<BF16>(p.s, off + j));
  mx = block_reduce<true>(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j < jend; j += 256) sum += __expf(load_elem<BF16>(p.s, off + j) - mx);
  sum = block_reduce<false>(sum, red);
  const float inv = jend > 0 ? 1.f / sum : 0.f;
  for (int j = threadIdx.x; j < N; j += 256) {
    const float e = j < jend ? __expf(load_elem<BF16>(p.s, off + j) - mx) * inv : 0.f;
    store_elem<BF16>(p.p, off + j, e);
  }
  if (threadIdx.x == 0) p.lse[row] = jend > 0 ? mx + __logf(sum) : kNegInf;
}

}  // namespace

hipError_t launch_naive_softmax(const NaiveSoftmaxParams& p, bool bf16, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.N));
  if (bf16) hipLaunchKernelGGL((naive_softmax_kernel<true>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((naive_softmax_kernel<false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
