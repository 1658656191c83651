// Fused attention forward for bf16 Q/K/V on gfx950 (CDNA4).
//
// One workgroup owns a tile of 128 query rows of one (batch, head) and keeps,
// per row, the running maximum m, denominator l and unnormalised numerator a
// of "FlashAttention: Exact Attention as an IO-Aware Streaming Computation"
// (section "Mathematical structure"), while key/value tiles stream through
// LDS ("IO-aware exact attention", section "One tiled forward-pass
// iteration").  Score tiles live only in registers; only O and the per-row
// log-sum-exp are written.
//
// Work split: 4 waves x 32 query rows.  Each wave computes the transposed
// score tile S^T = K Q^T on 32x32x16 bf16 MFMA so that every lane holds one
// query row's scores (column l % 32 of the accumulator); row maxima and sums
// are then in-lane reductions plus one exchange between the two wave halves.
// The probabilities are packed to bf16 in place and are already in the
// B-operand layout of the second product O^T = V^T P^T, provided V^T is laid
// out in LDS with the key order the accumulator rows use (bits 2 and 3 of
// the key index swapped within each group of 16).  O^T keeps one query row
// per lane as well, so the exp2(m_old - m_new) rescale is one multiply per
// register.
//
// Causal tiles run heaviest first; consecutive workgroups cycle over
// (batch, head) so all tiles of a head land on one XCD when B*H is a
// multiple of 8 (workgroups are dealt round-robin to the 8 XCDs).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int D>
struct Bf16Cfg {
  static constexpr int BQ = kQueryTile;          // query rows per workgroup
  static constexpr int BK = D == 128 ? 64 : 128; // keys per streamed tile
  static constexpr int KS = D + 8;               // K row stride in LDS (elements)
  static constexpr int VS = BK + 8;              // V^T row stride in LDS (elements)
  static constexpr int K_ELEMS = BK * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;  // one K tile + one V^T tile
  static constexpr int DCH = D / 8;              // 16-byte chunks per row
  static constexpr int K_LOADS = BK * DCH / 256; // 16-byte K loads per thread
  static constexpr int NB = BK / 32;             // 32-key blocks per tile
  static constexpr int ND = D / 32;              // 32-wide slices of the head dim
  static_assert(K_LOADS * 256 == BK * DCH, "K tile must split evenly over 256 threads");
  static_assert((BK / 4) * DCH == 256, "one V task (4 keys x 8 dims) per thread");
};

// Position of key kk (0 <= kk < BK) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa_fwd_bf16_kernel(FwdParams p) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- tile assignment ----------------------------------------------------
  const int BH = p.B * p.H;
  const int x = blockIdx.x;
  const int bh = x % BH;
  int qt = x / BH;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest tiles first
  const int b = bh / p.H;
  const int N = p.N;
  const int q0 = qt * C::BQ;
  int kv_lim = N;
  if (p.key_len) {
    const int L = p.key_len[b];
    kv_lim = L < 0 ? 0 : (L > N ? N : L);
  }
  int n_kv = kv_lim;
  if (CAUSAL) n_kv = min(n_kv, q0 + C::BQ);
  if (q0 >= kv_lim) n_kv = 0;  // every row of the tile is padding
  const int ntiles = (n_kv + C::BK - 1) / C::BK;

  const int64_t base = (int64_t)bh * N * D;
  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + base;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + base;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + base;

  const int qw0 = q0 + 32 * wave;  // first query row of this wave
  const int qrow = qw0 + l32;      // the query row this lane owns

  // ---- Q fragments (B operand of S^T = K Q^T) -----------------------------
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < N) w = *(const u32x4*)(qg + (int64_t)qrow * D + 16 * kk + 8 * h);
    w ^= p.q_sign;
    qf[kk] = __builtin_bit_cast(bf16x8, w);
  }

  // ---- K/V tile staging: global -> registers -> LDS -----------------------
  u32x4 kreg[C::K_LOADS];
  u32x4 vreg[4];
  const int vg_g = tid / C::DCH;  // V task: keys 4*vg_g .. +3
  const int vg_ch = tid % C::DCH; //         dims 8*vg_ch .. +7

  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int lin = i * 256 + tid;
      const int row = lin / C::DCH, ch = lin % C::DCH;
      const int key = kv0 + row;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (key < kv_lim) w = *(const u32x4*)(kg + (int64_t)key * D + 8 * ch);
      kreg[i] = w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kv0 + 4 * vg_g + i;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (key < kv_lim) w = *(const u32x4*)(vg + (int64_t)key * D + 8 * vg_ch);
      vreg[i] = w;
    }
  };

  auto store_tile = [&](int stage) {
    uint16_t* ks = lds + stage * C::STAGE;
    uint16_t* vt = ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int lin = i * 256 + tid;
      const int row = lin / C::DCH, ch = lin % C::DCH;
      *(u32x4*)(ks + row * C::KS + 8 * ch) = kreg[i];
    }
    // V^T: for each of the 8 dims, the 4 keys' values form one 8-byte store.
    const int pos = vt_pos(4 * vg_g);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a0 = vreg[0][w], a1 = vreg[1][w], a2 = vreg[2][w], a3 = vreg[3][w];
      u32x2 ev = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
      u32x2 od = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
      *(u32x2*)(vt + (8 * vg_ch + 2 * w) * C::VS + pos) = ev;
      *(u32x2*)(vt + (8 * vg_ch + 2 * w + 1) * C::VS + pos) = od;
    }
  };

  // ---- running state (one query row per lane) -----------------------------
  f32x16 o_acc[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) o_acc[i] = f32x16{};
  float m_run = kNegInf;  // running max of scale*log2(e)*s
  float l_run = 0.f;      // this lane's part of the denominator
  const float c = p.c;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * C::BK;
    if (t + 1 < ntiles) load_tile(kv0 + C::BK);  // prefetch, consumed after compute

    const uint16_t* ks = lds + (t & 1) * C::STAGE;
    const uint16_t* vt = ks + C::K_ELEMS;

    // Waves whose rows see no key of this tile skip it (wave-uniform).
    const bool skip = (CAUSAL && kv0 > qw0 + 31) || (qw0 >= kv_lim);
    if (!skip) {
      // S^T = K Q^T for this tile: NB accumulators of 32 keys x 32 queries.
      f32x16 s[C::NB];
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb) s[bb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int bb = 0; bb < C::NB; ++bb) {
          const bf16x8 kf = *(const bf16x8*)(ks + (32 * bb + l32) * C::KS + 16 * kk + 8 * h);
          s[bb] = mfma_32x32x16_bf16(kf, qf[kk], s[bb]);
        }
      }

      // Element masks only where the tile crosses the diagonal or the
      // sequence end (wave-uniform test).
      const bool masked = (CAUSAL && kv0 + C::BK - 1 > qw0) || (kv0 + C::BK > kv_lim);
      float mx = kNegInf;
      if (masked) {
#pragma unroll
        for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * bb + acc_row(r, h);
            const bool vis = key < kv_lim && (!CAUSAL || key <= qrow);
            s[bb][r] = vis ? s[bb][r] : kNegInf;
            mx = fmaxf(mx, s[bb][r]);
          }
      } else {
#pragma unroll
        for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[bb][r]);
      }
      mx = halves_max(mx);

      // New reference maximum (log2 units); -inf - (-inf) never evaluated.
      const float m_blk = (mx == kNegInf) ? kNegInf : mx * c;
      const float m_new = fmaxf(m_run, m_blk);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      // P = exp2(c*s - m_use); masked entries are exactly 0.
      float lsum = 0.f;
      bf16x8 pf[C::NB][2];
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float e[8];
#pragma unroll
          for (int t8 = 0; t8 < 8; ++t8) {
            const float sv = s[bb][8 * half + t8];
            float pv = fast_exp2(__builtin_fmaf(sv, c, -m_use));
            if (masked) pv = (sv == kNegInf) ? 0.f : pv;
            e[t8] = pv;
            lsum += pv;
          }
          u32x4 w = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                     pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
          pf[bb][half] = __builtin_bit_cast(bf16x8, w);
        }
      }
      l_run = alpha * l_run + lsum;

      // a <- alpha * a, skipped when no row's maximum moved (exact).
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < C::ND; ++i) o_acc[i] *= alpha;
      }

      // O^T += V^T P^T.
#pragma unroll
      for (int db = 0; db < C::ND; ++db) {
#pragma unroll
        for (int bb = 0; bb < C::NB; ++bb) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const bf16x8 vf =
                *(const bf16x8*)(vt + (32 * db + l32) * C::VS + 32 * bb + 16 * half + 8 * h);
            o_acc[db] = mfma_32x32x16_bf16(vf, pf[bb][half], o_acc[db]);
          }
        }
      }
    }

    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: o = a / l, LSE = ln(2) * (m + log2 l) ---------------------
  const float l_tot = halves_sum(l_run);
  const bool valid = qrow < kv_lim;  // rows at or beyond the length are padding
  const float inv = valid ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* og = (uint16_t*)p.o + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::ND; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = valid ? o_acc[db][4 * g + e] * inv : 0.f;
        u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *(u32x2*)(og + d0) = w;
      }
    }
    if (h == 0) {
      p.lse[(int64_t)bh * N + qrow] = valid ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n_qtiles * p.B * p.H));
  const dim3 block(256);
  if (d == 128) {
    if (causal) hipLaunchKernelGGL((fa_fwd_bf16_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fa_fwd_bf16_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_bf16_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fa_fwd_bf16_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
