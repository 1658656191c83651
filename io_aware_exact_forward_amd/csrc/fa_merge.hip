// Merge of split-KV partial results.
//
// Each key range s of a query row left a normalised partial output o_s and
// its log-sum-exp L_s (natural log; -inf when the range held no visible
// key).  Disjoint key blocks combine by expressing each block's denominator
// and numerator against a common reference maximum and adding (page
// "FlashAttention", sections "Why a tile can be discarded" and "One row,
// checked two ways"; the rule extends to any number of blocks).  With
// L_s = m_s + ln l_s and o_s = u_s / l_s that is
//   m = max_s L_s,  w_s = exp(L_s - m),  L = m + ln(sum_s w_s),
//   o = sum_s w_s o_s / sum_s w_s.
// The weights w_s carry each range's share of the denominator: normalised
// block outputs cannot simply be averaged (same page, "Practice: can you
// average block outputs?").  A row with every L_s = -inf saw no key at all:
// o = 0, L = -inf.
//
// One thread per four consecutive output elements of a row: the partial
// outputs of a row are read once, as 16-byte loads, and the row's L_s by
// every thread of the row (they are few and cached).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / TPR;
  const int c4 = (int)(gid % TPR);
  if (row >= p.rows) return;

  float m = kNegInf;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.lse_part[(int64_t)s * p.rows + row]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < p.splits; ++s) {
      const float ls = p.lse_part[(int64_t)s * p.rows + row];
      if (ls == kNegInf) continue;  // the range saw no key of this row
      const float w = __expf(ls - m);
      const f32x4 os = *(const f32x4*)(p.o_part + ((int64_t)s * p.rows + row) * D + 4 * c4);
      wsum += w;
      acc += w * os;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const f32x4 y = acc * inv;
  if constexpr (BF16) {
    u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    *(u32x2*)((uint16_t*)p.o + row * D + 4 * c4) = w;
  } else {
    *(f32x4*)((float*)p.o + row * D + 4 * c4) = y;
  }
  if (c4 == 0) p.lse[row] = wsum > 0.f ? m + __logf(wsum) : kNegInf;
}

template <int D, bool BF16>
hipError_t launch(const MergeParams& p, hipStream_t stream) {
  constexpr int TPR = D / 4;
  const int64_t threads = p.rows * TPR;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((merge_kernel<D, BF16>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int d, bool bf16, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  if (d == 128) return bf16 ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return bf16 ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}

}  // namespace fa
