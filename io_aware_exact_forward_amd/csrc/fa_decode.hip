// Attention for one query row per (batch, head) against a key cache: the
// decode step of "IO-aware exact attention" (section "Common errors" names
// decode as a shape that needs its own schedule).  A workgroup computes key
// ranges of (batch, head) rows; a row split over several workgroups is merged
// by the ranges' log-sum-exp ("FlashAttention" glossary, section "Why a tile
// can be discarded").  Two ways to hand out the work:
//  * fixed ranges: workgroup = (range of split_keys keys, (batch, head));
//  * balanced: the visible keys of all rows, in 64-key units, are cut into
//    equal shares, one per workgroup, whatever the per-sequence lengths.
//    Rows are laid end to end (sequence by sequence, head by head, key
//    order within a row) and workgroup w takes units [w S, (w + 1) S) of
//    the T units, S = ceil(T / P) for P workgroups.  The per-sequence
//    lengths are read on the device, so the host needs none of them.
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
// At the end the wave's slices are summed across its lane groups; with fixed
// ranges the four waves' states are then merged through LDS.  (One key row
// per lane would need no sum across lanes, but its loads touch 64 rows per
// instruction and ran 1.7x slower.)
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kDecodeWaves = 4;

template <int D>
struct DecodeLds {
  float m[kDecodeWaves], l[kDecodeWaves];
  __attribute__((aligned(16))) float o[kDecodeWaves][D];
};

__device__ __forceinline__ int seq_len(const FwdParams& p, int b) {
  if (!p.key_len) return p.Nk;
  const int kl = p.key_len[b];
  return kl < 0 ? 0 : (kl > p.Nk ? p.Nk : kl);
}

// One wave's pass over keys [k0, k1) of row bh (sequence b, key/value head
// hk, L keys visible), 64 keys at a time with a stride of `step` keys (the
// waves that share a range take its 64-key chunks in turn).  On return the
// lanes of group 0 (lane < D/8) hold the wave's numerator for dimensions
// 8 lane .. 8 lane + 7 in o, every lane the wave's running maximum m (log2
// units, -inf if the wave saw no key) and denominator l.
template <int D>
__device__ __forceinline__ void decode_wave(const FwdParams& p, const int bh, const int b,
                                            const int hk, const int L, const int k0, const int k1,
                                            const int step, float (&o)[8], float& m, float& l) {
  constexpr int LPR = D / 8;   // lanes per K or V row (16 bytes each)
  constexpr int G = 64 / LPR;  // key groups per wave
  constexpr int IT = 64 / G;   // keys per group and chunk
  static_assert(LPR == 8 || LPR == 16, "d = 64 or 128");
  const int lane = threadIdx.x & 63;

  const uint32_t row_bytes = D * 2;
  const void* kbase = (const uint16_t*)p.k + ((int64_t)b * p.Hkv + hk) * p.Nk * D;
  const void* vbase = (const uint16_t*)p.v + ((int64_t)b * p.Hkv + hk) * p.Nk * D;
  const uint32_t valid_bytes = (uint32_t)L * row_bytes;
  const int g = lane / LPR, t = lane % LPR;  // key group, 16-byte column

  float m_run = kNegInf;  // running maximum of c * s (log2 units), wave-uniform
  float l_g = 0.f;        // denominator over group g's keys (the same in its LPR lanes)
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;  // dims 8t .. 8t+7 over group g's keys
  // this lane's part of q: dimensions 8t .. 8t+7 as bf16 pairs.  Its first
  // use is in the first chunk, after that chunk's K and V loads are issued,
  // so the q load costs no round trip of its own; a negative scale therefore
  // enters through the sign of c (exactly: negating q negates every fp32
  // product and sum) rather than through q.
  const u32x4 qv = *(const u32x4*)((const uint16_t*)p.q + (int64_t)bh * D + 8 * t);
  uint32_t qt4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qt4[j] = qv[j];
  const float c = p.q_sign ? -p.c : p.c;

  for (int c0 = k0; c0 < k1; c0 += step) {
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
      sc[i] = c0 + g * IT + i < k1 ? a * c : kNegInf;
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
  m = m_run;
  l = l_w;
}

// Keys [k0, k1) of row bh by the four waves of the workgroup, their states
// merged through LDS.  Threads tid < D return element tid of the range's
// normalised output in y and the range's log-sum-exp (natural log) in lse;
// the range holds at least one key.
template <int D>
__device__ __forceinline__ void decode_range(const FwdParams& p, DecodeLds<D>& s, const int bh,
                                             const int b, const int hk, const int L, const int k0,
                                             const int k1, float& y, float& lse) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  float o[8], m_w, l_w;
  decode_wave<D>(p, bh, b, hk, L, k0 + 64 * wave, k1, 64 * kDecodeWaves, o, m_w, l_w);
  if (lane == 0) {
    s.m[wave] = m_w;
    s.l[wave] = l_w;
  }
  if (lane < D / 8) {
    *(f32x4*)&s.o[wave][8 * lane] = f32x4{o[0], o[1], o[2], o[3]};
    *(f32x4*)&s.o[wave][8 * lane + 4] = f32x4{o[4], o[5], o[6], o[7]};
  }
  __syncthreads();

  // ---- merge of the four waves (each a common-reference summary)
  if (tid < D) {
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) m = fmaxf(m, s.m[w]);
    float l = 0.f, a = 0.f;
    if (m != kNegInf) {
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        if (s.m[w] == kNegInf) continue;  // the wave saw no key
        const float sc = fast_exp2(s.m[w] - m);
        l += sc * s.l[w];
        a += sc * s.o[w][tid];
      }
    }
    const bool any = l > 0.f;
    y = any ? a / l : 0.f;
    lse = any ? (m + __log2f(l)) * kLn2 : kNegInf;
  }
}

template <int D>
__device__ __forceinline__ void store_row(const FwdParams& p, int64_t bh, float y, float lse) {
  const int tid = threadIdx.x;
  ((uint16_t*)p.o)[bh * D + tid] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
  if (tid == 0) p.lse[bh] = lse;
}

template <int D>
__device__ __forceinline__ void store_part(const FwdParams& p, int64_t slot, float y, float lse) {
  const int tid = threadIdx.x;
  p.o_part[slot * D + tid] = y;
  if (tid == 0) p.lse_part[slot] = lse;
}

// Fixed ranges.  Key range major: the (batch, head) pairs of one range take
// consecutive ids, so the heads of every sequence are dealt evenly over the
// 8 XCDs (round-robin by id) whichever ranges its length leaves empty.
template <int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void fa_decode_kernel(FwdParams p) {
  __shared__ DecodeLds<D> s;
  const int BH = p.B * p.H;
  const int split = (int)blockIdx.x / BH;
  const int bh = (int)blockIdx.x - split * BH;
  const int b = bh / p.H, hq = bh - b * p.H;
  const int hk = hq / (p.H / p.Hkv);
  const int L = __builtin_amdgcn_readfirstlane(seq_len(p, b));
  // this workgroup's keys: [k0, k1) (the row sits at position L - 1, so
  // under the causal mask it sees every key below L as well)
  const int k0 = split * p.split_keys;
  const int k1 = min(L, k0 + p.split_keys);
  float y = 0.f, lse = kNegInf;
  if (k0 < k1) decode_range<D>(p, s, bh, b, hk, L, k0, k1, y, lse);
  if (threadIdx.x < D) {
    if (p.o_part) store_part<D>(p, (int64_t)split * BH + bh, y, lse);  // [split, B, H, 1]
    else store_row<D>(p, bh, y, lse);
  }
}

// Units (of 64 keys) of one row of sequence b.
__device__ __forceinline__ int64_t row_units(const FwdParams& p, int b) {
  return (seq_len(p, b) + 63) >> 6;
}

// A wave-uniform 64-bit value held in vector registers, moved to scalar ones.
__device__ __forceinline__ int64_t uniform64(const int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t wave_incl_scan(int64_t x, const int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Balanced shares, one per workgroup: share w = blockIdx.x of P = gridDim.x
// takes units [w S, min(T, (w + 1) S)), S = ceil(T / P).  Every wave scans
// the per-sequence unit counts itself (a few wave-wide steps per 64
// sequences); wave 0 of workgroup 0 also stores the exclusive prefix cum[b]
// (units before sequence b) and the total T = cum[B] for the merge.  Unit u of the share goes to wave (u - begin) mod 4, so the four
// waves read adjacent 16 KB (d = 128) chunks of K and V, as with fixed
// ranges.  Each wave walks every row the share touches, one after the other
// with no barrier, and leaves for each a partial result at slot
// 4 (w + bh) + wave of o_part / lse_part (LSE -inf when it had no unit of
// the row).  (Shares are consecutive and rows are consecutive, so w1 < w2
// implies bh1 <= bh2 for any rows bh1 of w1 and bh2 of w2: w + bh never
// repeats across shares, and 4 (P + B*H) slots hold every partial.)  Every
// row is completed by the merge.
template <int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void fa_decode_balanced_kernel(FwdParams p,
                                                                               int64_t* cum) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool store_cum = blockIdx.x == 0 && wave == 0;
  const int B = p.B, H = p.H;
  int64_t T = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int64_t n = b < B ? row_units(p, b) * H : 0;
    const int64_t incl = wave_incl_scan(n, lane);
    if (store_cum && b < B) cum[b] = T + incl - n;
    T += __shfl(incl, 63);
  }
  if (store_cum && lane == 0) cum[B] = T;
  T = uniform64(T);
  // S = ceil(T / P) units per share: only the last shares can be empty
  const int64_t P = gridDim.x, w = blockIdx.x;
  const int64_t S = (T + P - 1) / P;
  const int64_t begin = w * S, end = min(T, begin + S);
  if (begin >= end) return;

  // the sequence holding unit `begin`, and its first unit
  int b = 0;
  int64_t seq_base = 0;
  {
    int64_t run = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int bl = b0 + lane;
      const int64_t n = bl < B ? row_units(p, bl) * H : 0;
      const int64_t incl = wave_incl_scan(n, lane);
      const bool hit = n > 0 && begin >= run + incl - n && begin < run + incl;
      const uint64_t mask = __ballot(hit);
      if (mask) {
        const int l = __builtin_ctzll(mask);
        b = b0 + l;
        seq_base = __shfl(run + incl - n, l);
        break;
      }
      run += __shfl(incl, 63);
    }
  }
  b = __builtin_amdgcn_readfirstlane(b);
  seq_base = uniform64(seq_base);
  int L = __builtin_amdgcn_readfirstlane(seq_len(p, b));
  int64_t nb = (L + 63) >> 6;  // > 0: the sequence holds unit `begin`
  const int group = H / p.Hkv;
  for (int64_t u = begin; u < end;) {
    const int h = (int)((u - seq_base) / nb);
    const int64_t row_start = seq_base + h * nb, row_end = row_start + nb;
    const int64_t seg_end = end < row_end ? end : row_end;
    // this wave's first unit of the segment: the next u' >= u with
    // (u' - begin) mod 4 == wave
    const int64_t first = u + ((wave - (u - begin)) & (kDecodeWaves - 1));
    const int k0 = (int)(first - row_start) * 64;
    const int k1 = min(L, (int)(seg_end - row_start) * 64);
    const int64_t bh = (int64_t)b * H + h;
    float o[8], m, l;
    decode_wave<D>(p, (int)bh, b, h / group, L, k0, k1, 64 * kDecodeWaves, o, m, l);
    const int64_t slot = kDecodeWaves * (w + bh) + wave;
    if (l > 0.f) {
      const float inv = 1.f / l;
      if (lane < D / 8) {
        float* dst = p.o_part + slot * D + 8 * lane;
        *(f32x4*)dst = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        *(f32x4*)(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
      }
      if (lane == 0) p.lse_part[slot] = (m + __log2f(l)) * kLn2;
    } else if (lane == 0) {
      p.lse_part[slot] = kNegInf;  // no unit of this row
    }
    u = seg_end;
    if (u == seq_base + H * nb && u < end) {
      // the next sequence with a visible key (one exists: units remain)
      seq_base = u;
      do {
        ++b;
        L = __builtin_amdgcn_readfirstlane(seq_len(p, b));
      } while (L == 0);
      nb = (L + 63) >> 6;
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

hipError_t launch_decode_balanced_bf16(const FwdParams& p, int d, int shares, int64_t* cum,
                                       hipStream_t stream) {
  const dim3 grid((unsigned)shares);
  const dim3 block(64 * kDecodeWaves);
  if (d == 128) hipLaunchKernelGGL((fa_decode_balanced_kernel<128>), grid, block, 0, stream, p, cum);
  else hipLaunchKernelGGL((fa_decode_balanced_kernel<64>), grid, block, 0, stream, p, cum);
  return hipGetLastError();
}

}  // namespace fa
