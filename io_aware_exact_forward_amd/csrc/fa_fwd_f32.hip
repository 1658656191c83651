// Fused attention forward for fp32 Q/K/V on gfx950.
//
// Same streamed computation as the bf16 kernel ("FlashAttention: Exact
// Attention as an IO-Aware Streaming Computation", section "Mathematical
// structure"): 128 query rows per workgroup, 32 per wave, running (m, l, a)
// per row, K/V tiles double-buffered through LDS.  Both products use the
// fp32 32x32x2 MFMA and the probabilities stay fp32, so nothing is rounded
// below single precision.
//
// Lane layout: the contraction index of both products is split between the
// two wave halves.  For S^T = K Q^T the half h covers head dims
// [h*D/2, (h+1)*D/2); for O^T = V^T P^T step r of a 32-key block pairs each
// half's own accumulator register r (key 8*(r/4) + 4*h + r%4) with that
// key's V row, so V is read row-major from LDS without a transpose.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int D>
struct F32Cfg {
  static constexpr int BQ = kQueryTile;
  static constexpr int BK = 4096 / D;             // 64 keys at D=64, 32 at D=128
  static constexpr int RS = D + 8;                // K and V row stride in LDS (floats)
  static constexpr int T_ELEMS = BK * RS;
  static constexpr int STAGE = 2 * T_ELEMS;       // K tile + V tile
  static constexpr int DCH = D / 4;               // 16-byte chunks per row
  static constexpr int LOADS = BK * DCH / 256;    // per thread, per tensor
  static constexpr int NB = BK / 32;
  static constexpr int ND = D / 32;
  static_assert(LOADS * 256 == BK * DCH, "tile must split evenly over 256 threads");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_fwd_f32_kernel(FwdParams p) {
  using C = F32Cfg<D>;
  __shared__ __attribute__((aligned(16))) float lds[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int BH = p.B * p.H;
  const int x = blockIdx.x;
  const int bh = x % BH;
  int qt = x / BH;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
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
  if (q0 >= kv_lim) n_kv = 0;
  const int ntiles = (n_kv + C::BK - 1) / C::BK;

  const int64_t base = (int64_t)bh * N * D;
  const float* __restrict__ qg = (const float*)p.q + base;
  const float* __restrict__ kg = (const float*)p.k + base;
  const float* __restrict__ vg = (const float*)p.v + base;

  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + l32;

  // Q fragment: this lane's query row, head dims [h*D/2, h*D/2 + D/2).
  float qf[D / 2];
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < N) w = *(const u32x4*)(qg + (int64_t)qrow * D + h * (D / 2) + 4 * j);
    w ^= p.q_sign;
    const f32x4 f = __builtin_bit_cast(f32x4, w);
    qf[4 * j + 0] = f[0];
    qf[4 * j + 1] = f[1];
    qf[4 * j + 2] = f[2];
    qf[4 * j + 3] = f[3];
  }

  u32x4 kreg[C::LOADS], vreg[C::LOADS];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int lin = i * 256 + tid;
      const int row = lin / C::DCH, ch = lin % C::DCH;
      const int key = kv0 + row;
      u32x4 wk = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};
      if (key < kv_lim) {
        wk = *(const u32x4*)(kg + (int64_t)key * D + 4 * ch);
        wv = *(const u32x4*)(vg + (int64_t)key * D + 4 * ch);
      }
      kreg[i] = wk;
      vreg[i] = wv;
    }
  };
  auto store_tile = [&](int stage) {
    float* ks = lds + stage * C::STAGE;
    float* vs = ks + C::T_ELEMS;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int lin = i * 256 + tid;
      const int row = lin / C::DCH, ch = lin % C::DCH;
      *(u32x4*)(ks + row * C::RS + 4 * ch) = kreg[i];
      *(u32x4*)(vs + row * C::RS + 4 * ch) = vreg[i];
    }
  };

  f32x16 o_acc[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) o_acc[i] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;
  const float c = p.c;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * C::BK;
    if (t + 1 < ntiles) load_tile(kv0 + C::BK);
    const float* ks = lds + (t & 1) * C::STAGE;
    const float* vs = ks + C::T_ELEMS;

    const bool skip = (CAUSAL && kv0 > qw0 + 31) || (qw0 >= kv_lim);
    if (!skip) {
      f32x16 s[C::NB];
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb) {
        s[bb] = f32x16{};
        const float* krow = ks + (32 * bb + l32) * C::RS + h * (D / 2);
#pragma unroll
        for (int j = 0; j < D / 8; ++j) {
          const f32x4 kf = *(const f32x4*)(krow + 4 * j);
          s[bb] = mfma_32x32x2_f32(kf[0], qf[4 * j + 0], s[bb]);
          s[bb] = mfma_32x32x2_f32(kf[1], qf[4 * j + 1], s[bb]);
          s[bb] = mfma_32x32x2_f32(kf[2], qf[4 * j + 2], s[bb]);
          s[bb] = mfma_32x32x2_f32(kf[3], qf[4 * j + 3], s[bb]);
        }
      }

      const bool masked = (CAUSAL && kv0 + C::BK - 1 > qw0) || (kv0 + C::BK > kv_lim);
      float mx = kNegInf;
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (masked) {
            const int key = kv0 + 32 * bb + acc_row(r, h);
            const bool vis = key < kv_lim && (!CAUSAL || key <= qrow);
            s[bb][r] = vis ? s[bb][r] : kNegInf;
          }
          mx = fmaxf(mx, s[bb][r]);
        }
      mx = halves_max(mx);

      const float m_blk = (mx == kNegInf) ? kNegInf : mx * c;
      const float m_new = fmaxf(m_run, m_blk);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      float lsum = 0.f;
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sv = s[bb][r];
          float pv = fast_exp2(__builtin_fmaf(sv, c, -m_use));
          if (masked) pv = (sv == kNegInf) ? 0.f : pv;
          s[bb][r] = pv;
          lsum += pv;
        }
      l_run = alpha * l_run + lsum;

      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < C::ND; ++i) o_acc[i] *= alpha;
      }

      // O^T += V^T P^T, one k-pair (keys acc_row(r,0), acc_row(r,1)) per step.
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* vrow = vs + (32 * bb + acc_row(r, h)) * C::RS + l32;
#pragma unroll
          for (int db = 0; db < C::ND; ++db)
            o_acc[db] = mfma_32x32x2_f32(vrow[32 * db], s[bb][r], o_acc[db]);
        }
    }

    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  const float l_tot = halves_sum(l_run);
  const bool valid = qrow < kv_lim;
  const float inv = valid ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    float* og = (float*)p.o + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = valid ? o_acc[db][4 * g + e] * inv : 0.f;
        *(f32x4*)(og + d0) = w;
      }
    if (h == 0) p.lse[(int64_t)bh * N + qrow] = valid ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n_qtiles * p.B * p.H));
  const dim3 block(256);
  if (d == 128) {
    if (causal) hipLaunchKernelGGL((fa_fwd_f32_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fa_fwd_f32_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_f32_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fa_fwd_f32_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
