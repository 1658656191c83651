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
// One wave per row.  The lanes read the row's L_s side by side (64 at a
// time) and reduce the maximum and the weight sum across the wave; then the
// wave streams the partial outputs, each lane D/64 dimensions of each, in a
// loop without branches (a partial whose weight is 0 is read and discarded),
// so that the loads of several partials are in flight together.  The
// partials come in two layouts: fixed key ranges (slot s * rows + row for
// range s) and the balanced shares of a decode step (slots 4 (w + row) +
// wave for share w).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kMergeWaves = 4;  // rows per workgroup

// The partials of one row: count K and the slot of the k-th (fixed ranges:
// first + k * stride; balanced shares: first + k).
struct RowParts {
  int64_t first, count, stride;
  __device__ __forceinline__ int64_t slot(int64_t k) const { return first + k * stride; }
};

template <int D, bool BF16, bool BALANCED>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeParams p) {
  constexpr int DPL = D / 64;  // dimensions per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (row >= p.rows) return;

  RowParts rp{};
  bool none = false;  // the row saw no key at all
  if constexpr (BALANCED) {
    // Row bh (sequence b, head h; one query row) holds units [start, start
    // + nb) of the T units laid end to end, start = cum[b] + h nb, nb =
    // ceil(L_b / 64).  Share w covers units [w S, (w + 1) S), S = ceil(T /
    // P), so unit u lies in share u / S, and every share from the first
    // unit's to the last unit's left four partials (one per wave) at slots
    // 4 (w + bh) + 0..3, LSE -inf for a wave with no unit of the row.  A
    // sequence with no visible key has no units.  (The three loads are
    // independent: they are issued together.)
    const int b = (int)(row / p.H), h = (int)(row - (int64_t)b * p.H);
    const int kl = p.key_len ? p.key_len[b] : p.Nk;
    const int64_t cb = p.cum[b], T = p.cum[p.B];
    const int L = kl < 0 ? 0 : (kl > p.Nk ? p.Nk : kl);
    const int64_t nb = (L + 63) >> 6;
    none = nb == 0;
    if (!none) {
      const int64_t S = (T + p.workgroups - 1) / p.workgroups;
      const int64_t start = cb + h * nb, last = start + nb - 1;
      const int64_t w1 = start / S, w2 = last / S;
      rp = RowParts{4 * (w1 + row), 4 * (w2 - w1 + 1), 1};
    }
  } else {
    rp = RowParts{row, p.splits, p.rows};
  }

  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  float m = kNegInf;
  // ---- few partials: their outputs are loaded together with their LSE
  // (the addresses need no LSE), so the row costs one round trip less
  auto few = [&](auto f_tag) __attribute__((always_inline)) {
    constexpr int F = decltype(f_tag)::value;
    float os[F][DPL];
#pragma unroll
    for (int k = 0; k < F; ++k) {
      // past the count: partial 0 again (in bounds), weighted 0 below
      const float* src = p.o_part + rp.slot(k < rp.count ? k : 0) * D + DPL * lane;
      if constexpr (DPL == 2) {
        const f32x2 t = *(const f32x2*)src;
        os[k][0] = t[0];
        os[k][1] = t[1];
      } else {
        os[k][0] = *src;
      }
    }
    const float ls = lane < rp.count ? p.lse_part[rp.slot(lane)] : kNegInf;
    m = ls;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (m == kNegInf) return;
    const float wk = ls == kNegInf ? 0.f : __expf(ls - m);
    wsum = wk;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
#pragma unroll
    for (int k = 0; k < F; ++k) {
      const float wv =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), k));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += wv > 0.f ? wv * os[k][e] : 0.f;
    }
  };
  if (none) {
  } else if (rp.count <= 8) {
    few(std::integral_constant<int, 8>{});
  } else if (rp.count <= 32) {
    few(std::integral_constant<int, 32>{});
  } else if (!none) {
    // ---- maximum and weight sum over the partials' LSE, lane-parallel
    for (int64_t k0 = 0; k0 < rp.count; k0 += 64) {
      const int64_t k = k0 + lane;
      const float ls = k < rp.count ? p.lse_part[rp.slot(k)] : kNegInf;
      m = fmaxf(m, ls);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    for (int64_t k0 = 0; m != kNegInf && k0 < rp.count; k0 += 64) {
      const int64_t k = k0 + lane;
      const float ls = k < rp.count ? p.lse_part[rp.slot(k)] : kNegInf;
      const float wk = ls == kNegInf ? 0.f : __expf(ls - m);  // this lane's partial's weight
      float part = wk;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
      wsum += part;
      // ---- the outputs of these (up to) 64 partials, weighted
      const int n = (int)min<int64_t>(64, rp.count - k0);
      int j = 0;
      for (; j + 4 <= n; j += 4) {
        float wj[4];
        float os[4][DPL];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wj[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), j + i));
          const float* src = p.o_part + rp.slot(k0 + j + i) * D + DPL * lane;
          if constexpr (DPL == 2) {
            const f32x2 t = *(const f32x2*)src;
            os[i][0] = t[0];
            os[i][1] = t[1];
          } else {
            os[i][0] = *src;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] += wj[i] > 0.f ? wj[i] * os[i][e] : 0.f;
      }
      for (; j < n; ++j) {
        const float wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), j));
        const float* src = p.o_part + rp.slot(k0 + j) * D + DPL * lane;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += wv > 0.f ? wv * src[e] : 0.f;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if constexpr (BF16) {
    uint16_t* orow = (uint16_t*)p.o + row * D + DPL * lane;
    if constexpr (DPL == 2) *(uint32_t*)orow = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    else *orow = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xFFFFu);
  } else {
    float* orow = (float*)p.o + row * D + DPL * lane;
#pragma unroll
    for (int e = 0; e < DPL; ++e) orow[e] = acc[e] * inv;
  }
  if (lane == 0) p.lse[row] = wsum > 0.f ? m + __logf(wsum) : kNegInf;
}

template <int D, bool BF16, bool BALANCED>
hipError_t launch(const MergeParams& p, hipStream_t stream) {
  const int64_t blocks = (p.rows + kMergeWaves - 1) / kMergeWaves;
  hipLaunchKernelGGL((merge_kernel<D, BF16, BALANCED>), dim3((unsigned)blocks),
                     dim3(64 * kMergeWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int d, bool bf16, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  if (p.cum) {  // balanced decode shares (bf16)
    return d == 128 ? launch<128, true, true>(p, stream) : launch<64, true, true>(p, stream);
  }
  if (d == 128) return bf16 ? launch<128, true, false>(p, stream) : launch<128, false, false>(p, stream);
  return bf16 ? launch<64, true, false>(p, stream) : launch<64, false, false>(p, stream);
}

}  // namespace fa
