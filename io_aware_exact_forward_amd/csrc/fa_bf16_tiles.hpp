// LDS layout of the bf16 K and V tiles shared by the bf16 kernels: rows are
// keys ([key][dim], d bf16 each) and the 16-byte chunks of a row are permuted
// by an XOR of the row index, which makes the fragment reads free of bank
// conflicts (checked with SQ_LDS_BANK_CONFLICT = 0 on the kernels).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Physical 16-byte chunk of logical chunk c in row `row` of a K tile.  Reads
// of one chunk by 16 consecutive rows then touch 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_chunk(int row, int c) {
  return D == 128 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
}

// Physical 16-byte chunk of logical chunk c in row `row` of a V tile.  A
// transpose read covers 4 consecutive keys x 32 dims per half wave (and 8
// keys x 16 dims per 16-lane pair); this permutation spreads both over all
// banks.
template <int D>
__device__ __forceinline__ int v_chunk(int row, int c) {
  return D == 128 ? (c ^ (4 * (row & 3) + 2 * ((row >> 2) & 1)))
                  : (c ^ (4 * ((row >> 1) & 1) + 2 * ((row >> 2) & 1)));
}

}  // namespace fa
