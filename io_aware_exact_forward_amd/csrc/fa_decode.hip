// Attention for one query row per (batch, head) against a key cache: the
// decode step of "IO-aware exact attention" (section "Common errors" names
// decode as a shape that needs its own schedule).  One workgroup computes one
// key range of one (batch, head); ranges are merged by their log-sum-exp
// ("FlashAttention" glossary, section "Why a tile can be discarded").
//
// With a single query row there is no matrix product to speak of: the work
// is streaming K and V once from HBM.  Each wave takes 64 keys at a time:
//  * D/8 lanes share each K and V row, 16 bytes apiece (coalesced,
//    range-checked buffer loads: keys past the sequence's length read
//    zeros), so each of the wave's 64/(D/8) lane groups holds D/8 of its
//    64 keys;
//  * scores: each lane forms the bf16 dot products of its 8 dimensions of K
//    with its 8 dimensions of q (fp32 accumulation) and DPP additions sum them
//    over the row's lanes;
//  * the wave keeps a running maximum, each group its denominator, each lane
//    a numerator slice of 8 dimensions, rescaled when the maximum rises
//    ("FlashAttention: Exact Attention as an IO-Aware Streaming Computation",
//    section "Mathematical structure"); the weights never leave the lane.
// At the end the wave's slices are summed across its lane groups and the
// four waves' states are merged through LDS.  (One key row per lane would
// need no sum across lanes, but its loads touch 64 rows per instruction and
// ran 1.7x slower.)
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kDecodeWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void fa_decode_kernel(FwdParams p) {
  constexpr int LPR = D / 8;   // lanes per K or V row (16 bytes each)
  constexpr int G = 64 / LPR;  // key groups per wave
  constexpr int IT = 64 / G;   // keys per group and chunk
  static_assert(LPR == 8 || LPR == 16, "d = 64 or 128");
  __shared__ float m_lds[kDecodeWaves], l_lds[kDecodeWaves];
  __shared__ __attribute__((aligned(16))) float o_lds[kDecodeWaves][D];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int x = blockIdx.x;
  const int split = x % p.splits;
  const int bh = x / p.splits;
  const int b = bh / p.H, hq = bh - b * p.H;
  const int hk = hq / (p.H / p.Hkv);
  int L = p.Nk;
  if (p.key_len) {
    const int kl = p.key_len[b];
    L = kl < 0 ? 0 : (kl > p.Nk ? p.Nk : kl);
  }
  L = __builtin_amdgcn_readfirstlane(L);
  // this workgroup's keys: [k0, k1) (the row sits at position L - 1, so
  // under the causal mask it sees every key below L as well)
  const int k0 = split * p.split_keys;
  const int k1 = min(L, k0 + p.split_keys);

  const uint32_t row_bytes = D * 2;
  const void* kbase = (const uint16_t*)p.k + ((int64_t)b * p.Hkv + hk) * p.Nk * D;
  const void* vbase = (const uint16_t*)p.v + ((int64_t)b * p.Hkv + hk) * p.Nk * D;
  const uint32_t valid_bytes = (uint32_t)L * row_bytes;
  const int g = lane / LPR, t = lane % LPR;  // key group, 16-byte column

  float m_run = kNegInf;  // running maximum of c * s (log2 units), wave-uniform
  float l_g = 0.f;        // denominator over group g's keys (the same in its LPR lanes)
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // dims 8t .. 8t+7 over group g's keys
  // this lane's part of q: dimensions 8t .. 8t+7 as bf16 pairs, the sign
  // folded in for a negative scale
  const u32x4 qv = *(const u32x4*)((const uint16_t*)p.q + (int64_t)bh * D + 8 * t);
  uint32_t qt4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = qv[j];
    qt4[j] = w ^ p.q_sign;
  }

  for (int c0 = k0 + 64 * wave; c0 < k1; c0 += 64 * kDecodeWaves) {
    // ---- loads: rows c0 + g IT + i of K and V, 16 bytes (column t) each
    u32x4 kr[IT], vr[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint32_t off = (uint32_t)(c0 + g * IT + i) * row_bytes + 16 * t;
      kr[i] = load_ranged_16(kbase, valid_bytes, off);
      vr[i] = load_ranged_16(vbase, valid_bytes, off);
    }
    // ---- scores of the group's IT keys: partial dot products over this
    // lane's 8 dimensions, summed over the row's LPR lanes by DPP adds
    float sc[IT];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // (through named scalars: a bit cast of a vector element itself
        // compiles to a read of element 0 with this compiler)
        const uint32_t kw = kr[i][j];
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                            __builtin_bit_cast(bf16x2, qt4[j]), a, false);
      }
      a += dpp_f32<0xB1>(a);   // quad_perm [1, 0, 3, 2]
      a += dpp_f32<0x4E>(a);   // quad_perm [2, 3, 0, 1]
      a += dpp_f32<0x141>(a);  // row_half_mirror: the 8-lane sum
      if constexpr (LPR == 16) a += dpp_f32<0x140>(a);  // row_mirror: the 16-lane sum
      sc[i] = c0 + g * IT + i < k1 ? a * p.c : kNegInf;
      mx = fmaxf(mx, sc[i]);
    }
    // ---- running maximum (over the wave's 64 keys) and weights
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float m_new = fmaxf(m_run, mx);  // finite: key c0 < k1 is visible
    const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - m_new);
    m_run = m_new;
    l_g *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
    // ---- values: o += p_i v_i over the group's keys
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const float pw = fast_exp2(sc[i] - m_new);  // 0 for masked keys
      l_g += pw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = vr[i][j];
        o[2 * j] = __builtin_fmaf(pw, __builtin_bit_cast(float, w << 16), o[2 * j]);
        o[2 * j + 1] = __builtin_fmaf(pw, __builtin_bit_cast(float, w & 0xFFFF0000u), o[2 * j + 1]);
      }
    }
  }

  // ---- the wave's state: denominator over all lanes, numerator over the
  // key groups (lanes t, t + LPR, ... hold the same dimensions)
  float l_w = l_g;
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    l_w += __shfl_xor(l_w, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off);
  }
  if (lane == 0) {
    m_lds[wave] = m_run;
    l_lds[wave] = l_w;
  }
  if (g == 0) {
    *(f32x4*)&o_lds[wave][8 * t] = f32x4{o[0], o[1], o[2], o[3]};
    *(f32x4*)&o_lds[wave][8 * t + 4] = f32x4{o[4], o[5], o[6], o[7]};
  }
  __syncthreads();

  // ---- merge of the four waves (each a common-reference summary) and output
  if (tid < D) {
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) m = fmaxf(m, m_lds[w]);
    float l = 0.f, a = 0.f;
    if (m != kNegInf) {
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        if (m_lds[w] == kNegInf) continue;  // the wave saw no key
        const float sc = fast_exp2(m_lds[w] - m);
        l += sc * l_lds[w];
        a += sc * o_lds[w][tid];
      }
    }
    const bool any = l > 0.f;
    const float y = any ? a / l : 0.f;
    const float lse = any ? (m + __log2f(l)) * kLn2 : kNegInf;
    if (p.o_part) {
      const int64_t prow = (int64_t)split * p.B * p.H + bh;  // [split, B, H, 1]
      p.o_part[prow * D + tid] = y;
      if (tid == 0) p.lse_part[prow] = lse;
    } else {
      ((uint16_t*)p.o)[(int64_t)bh * D + tid] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
      if (tid == 0) p.lse[bh] = lse;
    }
  }
}

}  // namespace

hipError_t launch_decode_bf16(const FwdParams& p, int d, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.splits));
  const dim3 block(64 * kDecodeWaves);
  if (d == 128) hipLaunchKernelGGL((fa_decode_kernel<128>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((fa_decode_kernel<64>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
