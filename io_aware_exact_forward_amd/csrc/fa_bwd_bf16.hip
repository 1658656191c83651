// Attention backward for bf16 Q/K/V on gfx950 (CDNA4), by recomputation.
//
// "IO-aware exact attention" (section "Backward recomputation") keeps only
// the inputs, the output and a per-row normalisation record from the
// forward pass and rebuilds score and probability blocks while dQ, dK and dV
// accumulate, so nothing N x N is stored.  The record here is the forward's
// natural-log LSE: P_ij = exp(scale * q_i . k_j - LSE_i) is exact
// recomputation of the forward's probabilities.  With the upstream gradient
// dO and D_i = dO_i . O_i the gradients of the loss sum(dO * O) are
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, neither with atomics:
//  * fa_bwd_dq_kernel, one workgroup per 128 query rows (a wave per 32
//    rows), streams key/value tiles like the forward: S^T = K Q^T and
//    dP^T = V dO^T with Q and dO resident in registers, then
//    dQ^T += K^T dS^T.  It also computes D_i (each lane holds half of its
//    row of O and dO) and leaves it in the workspace.
//  * fa_bwd_dkdv_kernel, one workgroup per 128 keys (a wave per 32 keys),
//    streams query tiles with their LSE and D: S = Q K^T and dP = dO V^T
//    with K and V resident, then dV^T += dO^T P and dK^T += Q^T dS.
// Every product is a 32x32x16 bf16 MFMA with fp32 accumulation; P and dS are
// rounded to bf16 only as MFMA operands.  The transposed operands (K^T,
// dO^T, Q^T) come from row-major LDS tiles through transpose reads
// (ds_read_b64_tr_b16), with the contraction index permuted to match the
// register layout of P and dS, exactly as the forward reads V^T.
//
// With dropout (the forward's keep mask Z, kept weights scaled by 1/(1-p))
// the gradients are dV = (P*Z)^T dO / (1-p) and dS = P * (Z*dP/(1-p) - D);
// both kernels regenerate Z from the forward's Philox4x32-10 stream.  With an
// additive mask M the scores are scale * q . k + M and P is rebuilt from
// them; the rest is unchanged.  Kernel variants: VAR 0 plain, 1 dropout,
// 2 additive mask.
//
// Tiles go global -> registers -> LDS (two stages, one workgroup barrier
// per tile).  Rows and keys at or beyond a sequence's length are loaded as
// zeros and masked, so they contribute nothing, and their gradients are 0.
#include "fa_bf16_tiles.hpp"
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int ROW_BYTES = 2 * D;
  static constexpr int CPR = D / 8;   // 16-byte chunks per row
  static constexpr int ND = D / 32;   // 32-wide head-dim slices (accumulator blocks)
  static constexpr int KD = D / 16;   // 16-wide head-dim chunks (MFMA k steps)
};

// Byte offset of logical chunk c of row r in a tile stored with the
// transpose-friendly chunk permutation (read both plainly and transposed).
template <int D>
__device__ __forceinline__ int toff_t(int r, int c) {
  return r * BwdCfg<D>::ROW_BYTES + 16 * v_chunk<D>(r, c);
}
// The same for tiles only read plainly.
template <int D>
__device__ __forceinline__ int toff_p(int r, int c) {
  return r * BwdCfg<D>::ROW_BYTES + 16 * k_chunk<D>(r, c);
}

__device__ __forceinline__ bf16x8 lds_b128(const uint8_t* base, int off) {
  return *(const bf16x8*)(base + off);
}

// A operand of an MFMA whose contraction runs over 16 rows of a row-major
// tile (rows r0 .. r0+15 of the tile at `t`), for head-dim slice db: lane l
// receives dim 32*db + l%32 of rows {r0 + 4h + 0..3, r0 + 8 + 4h + 0..3}
// (h = l/32), which is the order in which the accumulator layout holds the
// 16 rows of one MFMA's worth of P or dS.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* t, int r0, int db, int lane) {
  const int r16 = lane & 15, g16 = (lane >> 4) & 1, h = lane >> 5;
  const int dim = 32 * db + 16 * g16 + 4 * (r16 & 3);
  const int ra = r0 + 4 * h + (r16 >> 2);
  const int rb = ra + 8;
  const bf16x4 x = lds_read_tr16(t + toff_t<D>(ra, dim >> 3) + (dim & 7) * 2);
  const bf16x4 y = lds_read_tr16(t + toff_t<D>(rb, dim >> 3) + (dim & 7) * 2);
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// Eight accumulator registers (one MFMA's worth of rows) -> bf16 B operand.
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  return bf16x8{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                (__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]};
}

// Row of a 16-byte bf16 chunk -> fp32 dot product of two chunks.
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += (float)x[e] * (float)y[e];
  return s;
}

// Layout of one (batch, query head) and the key/value head it reads: dense
// [B, H, Nq, d] / [B, Hkv, Nk, d], or a packed batch [T, H, d] / [T, Hkv, d]
// with sequence b at rows cu[b] .. cu[b+1]-1.  LSE and D share one layout
// ([B, H, Nq] dense, [T, H] packed).  Query row i sits at key position
// i + off (off = 0, or L_b - Nq with the rows at the end of the keys);
// keys j < kv_lim are valid.  Strides and bases in elements, all
// workgroup-uniform; a lane's offset from its base is below 2^31 elements
// (the host bounds a slice or packed sequence to 2^31 bytes), so offsets
// are 32-bit and the loads take the scalar-base form.
struct BwdLayout {
  int Nq, Nk, kv_lim, off;
  int q_ld, kv_ld, lse_ld;         // row strides
  int64_t q_hs, lse_hs;            // head strides (Q/O/dO/dQ, LSE/D)
  int64_t base, kvbase, lse_base;  // of query head hq and key/value head hk
};

template <int D>
__device__ __forceinline__ BwdLayout bwd_layout(const BwdParams& p, int b, int hq, int hk) {
  BwdLayout l;
  if (p.cu_q) {
    const int s0 = __builtin_amdgcn_readfirstlane(p.cu_q[b]);
    const int k0 = __builtin_amdgcn_readfirstlane(p.cu_k[b]);
    l.Nq = __builtin_amdgcn_readfirstlane(p.cu_q[b + 1]) - s0;
    l.Nk = __builtin_amdgcn_readfirstlane(p.cu_k[b + 1]) - k0;
    l.q_ld = p.H * D;
    l.kv_ld = p.Hkv * D;
    l.lse_ld = p.H;
    l.q_hs = D;
    l.lse_hs = 1;
    l.base = ((int64_t)s0 * p.H + hq) * D;
    l.kvbase = ((int64_t)k0 * p.Hkv + hk) * D;
    l.lse_base = (int64_t)s0 * p.H + hq;
  } else {
    l.Nq = p.N;
    l.Nk = p.Nk;
    l.q_ld = D;
    l.kv_ld = D;
    l.lse_ld = 1;
    l.q_hs = (int64_t)p.N * D;
    l.lse_hs = p.N;
    l.base = ((int64_t)b * p.H + hq) * p.N * D;
    l.kvbase = ((int64_t)b * p.Hkv + hk) * p.Nk * D;
    l.lse_base = ((int64_t)b * p.H + hq) * p.N;
  }
  int lim = l.Nk;
  if (p.key_len) {
    const int x = p.key_len[b];
    lim = x < 0 ? 0 : (x > l.Nk ? l.Nk : x);
  }
  l.kv_lim = __builtin_amdgcn_readfirstlane(lim);
  l.off = p.end_aligned ? l.kv_lim - l.Nq : 0;
  return l;
}

// ---------------------------------------------------------------------------
// dQ (and D): one workgroup per 128 query rows of one (batch, head)
// ---------------------------------------------------------------------------
// Two workgroups per CU (two waves per SIMD, so one wave's softmax work
// runs under the other's products).  At d = 128 the kernel takes 32-key
// tiles: a wave's dQ accumulators, Q and dO fragments, scores and staging
// registers then fit the 256 registers a lane has at two waves per SIMD.
// (With 64-key tiles it needed 364 and ran one workgroup per CU: the packed
// 16-sequence backward took 15.95 ms instead of 13.95.)  The products are the
// same 16-key steps in the same order either way.
constexpr int kDqOccupancy = 2;
// Workgroups per CU of the dK/dV kernel: two at d = 64; at d = 128 the
// accumulators of one workgroup take the registers of two.
template <int D>
constexpr int kBwdOccupancy = D == 64 ? 2 : 1;

// Grid order of both kernels: (batch, head) pairs in chunks of kChunk, every
// tile of a chunk before the next chunk, one tile of each pair of the chunk
// per round of kChunk workgroups, heaviest tiles first.  The hardware deals
// workgroup x to XCD x % 8 and, within it, to one of four shader engines by
// (x / 8) % 4.  Pair q + 8t (mod the chunk's pairs) takes slot q of round t,
// so a pair stays on one XCD (the rows its workgroups stream, K/V or Q/dO,
// are shared through that XCD's L2) while its tiles rotate over the four
// engines: pairs of unequal work (sequences of different lengths) then load
// every engine alike, and no engine fills up while the in-order dispatcher
// waits on it with the others idle.  The dQ kernel uses chunks of 32 pairs.
// The dK/dV kernel, whose workgroups of one pair all stream the same Q and
// dO rows, uses chunks of 8 when the key/value heads come in multiples of 8:
// a chunk is then the heads of one sequence (equal work), each XCD runs one
// pair at a time on all its CUs, and up to 32 workgroups share every Q/dO
// row through the L2 instead of 8 (on the packed 16-sequence backward its
// fetch fell from 7.4x to 1.7x the compulsory bytes; the kernel is bound by
// its products, and its time moved by 1-2.5 %).
struct GridPos {
  int pair, tile;
};
__device__ __forceinline__ GridPos grid_pos(int x, int pairs, int tiles, int kChunk = 32) {
  const int chunk_wgs = kChunk * tiles;
  const int chunk = x / chunk_wgs;
  const int in_chunk = x - chunk * chunk_wgs;
  const int chunk_pairs = min(kChunk, pairs - chunk * kChunk);
  const int tile = in_chunk / chunk_pairs;
  const int slot = in_chunk - tile * chunk_pairs;
  return {chunk * kChunk + (int)(((unsigned)slot + 8u * (unsigned)tile) % (unsigned)chunk_pairs), tile};
}

// Value of lane l ^ K within each group of four lanes (DPP quad permute).
template <int K>
__device__ __forceinline__ uint32_t quad_xor(uint32_t x) {
  constexpr int ctrl = (0 ^ K) | ((1 ^ K) << 2) | ((2 ^ K) << 4) | ((3 ^ K) << 6);
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, ctrl, 0xF, 0xF, false);
}

// The forward's dropout draws for query row `row` and the four keys
// 4*(key0/4) .. +3 of head bh: bit t set iff key 4*(key0/4) + t is kept.
__device__ __forceinline__ uint32_t keep_nibble(const BwdParams& p, uint32_t key0, uint32_t row,
                                                uint32_t bh) {
  const u32x4 w = philox4x32_10(u32x4{key0 >> 2, row, bh, p.drop_offset}, p.seed_lo, p.seed_hi);
  return (uint32_t)(w[0] >= p.drop_threshold) | ((uint32_t)(w[1] >= p.drop_threshold) << 1) |
         ((uint32_t)(w[2] >= p.drop_threshold) << 2) | ((uint32_t)(w[3] >= p.drop_threshold) << 3);
}

template <int D, bool CAUSAL, int VAR>
__global__ __launch_bounds__(256, kDqOccupancy) void fa_bwd_dq_kernel(BwdParams p) {
  constexpr bool DROP = VAR == 1, BIAS = VAR == 2;
  using C = BwdCfg<D>;
  constexpr int BQ = 128, BK = D == 128 ? 32 : 64, NB = BK / 32;
  constexpr int TILE = BK * C::ROW_BYTES;
  constexpr int LPT = BK * C::CPR / 256;  // 16-byte chunks per thread per tensor
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const GridPos gp = grid_pos(blockIdx.x, p.B * p.H, p.n_qtiles);
  const int bh = gp.pair;
  const int qt = CAUSAL ? p.n_qtiles - 1 - gp.tile : gp.tile;  // heaviest tiles first
  const int b = bh / p.H;
  const int hq = bh - b * p.H;
  const BwdLayout lay = bwd_layout<D>(p, b, hq, hq / (p.H / p.Hkv));
  const int Nq = lay.Nq, kv_lim = lay.kv_lim, off = lay.off;
  const int q0 = qt * BQ;
  // keys this query tile sees: below the length and, if causal, at or
  // before the position of its last row
  int n_kv = kv_lim;
  if (CAUSAL) n_kv = min(n_kv, max(0, q0 + BQ + off));
  if (q0 >= Nq || q0 + off >= kv_lim) n_kv = 0;
  const int ntiles = (n_kv + BK - 1) / BK;

  const uint16_t* qg = (const uint16_t*)p.q + lay.base;
  const uint16_t* kg = (const uint16_t*)p.k + lay.kvbase;
  const uint16_t* vg = (const uint16_t*)p.v + lay.kvbase;
  const uint16_t* og = (const uint16_t*)p.o + lay.base;
  const uint16_t* dog = (const uint16_t*)p.dout + lay.base;
  const int q_ld = lay.q_ld, kv_ld = lay.kv_ld;

  const int qw0 = q0 + 32 * wave;
  const int row = qw0 + l32;
  const int pos = row + off;  // key position of this lane's row
  // a row that sees at least one key
  const bool row_ok = row < Nq && pos < kv_lim && (CAUSAL ? pos >= 0 : kv_lim > 0);

  // Q and dO of this lane's row (half of the head dim, B-operand layout),
  // and D = dO . O over the whole row.
  bf16x8 qf[C::KD], dof[C::KD];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < C::KD; ++kk) {
    u32x4 wq = {0u, 0u, 0u, 0u}, wd = {0u, 0u, 0u, 0u}, wo = {0u, 0u, 0u, 0u};
    if (row_ok) {
      const uint32_t ro = (uint32_t)row * q_ld + 16 * kk + 8 * h;
      wq = *(const u32x4*)(qg + ro);
      wd = *(const u32x4*)(dog + ro);
      wo = *(const u32x4*)(og + ro);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, wq);
    dof[kk] = __builtin_bit_cast(bf16x8, wd);
    dsum += dot8(wd, wo);
  }
  const float dval = halves_sum(dsum);
  const uint32_t lse_at = (uint32_t)row * lay.lse_ld;
  float lse2 = row_ok ? p.lse[lay.lse_base + lse_at] * kLog2e : 0.f;
  // a row the additive mask hides entirely has LSE -inf (and mask -inf on
  // every key, so its weights are exactly 0 with lse2 = 0)
  if (BIAS && lse2 == kNegInf) lse2 = 0.f;
  // additive mask of this lane's row (clamped to a row of the slice; the
  // values of rows and keys outside the sequence are masked out)
  const float* bias_row = nullptr;
  if constexpr (BIAS)
    bias_row = p.bias + (int64_t)b * p.bias_sb + (int64_t)hq * p.bias_sh +
               (int64_t)min(row, Nq - 1) * p.bias_ld;
  if (h == 0 && row < Nq) (p.dvec + lay.lse_base)[lse_at] = row_ok ? dval : 0.f;

  f32x16 dq[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) dq[i] = f32x16{};

  // K tile: read plainly (S^T) and transposed (dQ^T); V tile: plainly (dP^T).
  // Chunk i of a thread is row tid/CPR + i*256/CPR of the tile, at a byte
  // offset from the tile's first row that is the same for every tile; keys
  // at or beyond the length lie outside the buffer range and read as zeros.
  u32x4 kst[LPT], vst[LPT];
  const uint32_t kv_off0 = ((uint32_t)(tid / C::CPR) * kv_ld + 8 * (tid % C::CPR)) * 2;
  const uint32_t kv_step = (256 / C::CPR) * (uint32_t)kv_ld * 2;
  auto load_regs = [&](int kv0) __attribute__((always_inline)) {
    const uint32_t nb = (uint32_t)max(0, kv_lim - kv0) * kv_ld * 2;
    const int64_t at = (int64_t)kv0 * kv_ld;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      kst[i] = load_ranged_16(kg + at, nb, kv_off0 + i * kv_step);
      vst[i] = load_ranged_16(vg + at, nb, kv_off0 + i * kv_step);
    }
  };
  auto store_lds = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + 256 * i, r = c / C::CPR, lc = c % C::CPR;
      *(u32x4*)(&lds[st][toff_t<D>(r, lc)]) = kst[i];
      *(u32x4*)(&lds[st][TILE + toff_p<D>(r, lc)]) = vst[i];
    }
  };

  auto compute = [&](int st, int kv0) __attribute__((always_inline)) {
    // keys all after the wave's last row, or the wave's rows all padding
    if ((CAUSAL && kv0 > qw0 + off + 31) || qw0 + off >= kv_lim || qw0 >= Nq) return;
    const uint8_t* kt = lds[st];
    const uint8_t* vt = lds[st] + TILE;
    f32x16 s[NB], dp[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      s[bb] = f32x16{};
      dp[bb] = f32x16{};
      const int kr = 32 * bb + l32;
#pragma unroll
      for (int kk = 0; kk < C::KD; ++kk) {
        s[bb] = mfma_32x32x16_bf16(lds_b128(kt, toff_t<D>(kr, 2 * kk + h)), qf[kk], s[bb]);
        dp[bb] = mfma_32x32x16_bf16(lds_b128(vt, toff_p<D>(kr, 2 * kk + h)), dof[kk], dp[bb]);
      }
    }
    // P^T and dS^T: lane = query row, register r of block bb = key 32bb + acc_row(r, h).
    // Element masks only where the tile crosses the diagonal or a length
    // (wave-uniform test).
    bf16x8 dsb[NB][2];
    const bool full = (!CAUSAL || kv0 + BK - 1 <= qw0 + off) && kv0 + BK <= kv_lim &&
                      qw0 + 31 < Nq && qw0 + 31 + off < kv_lim;
    // Key kv0 + 32 bb + acc_row(r, h) is visible to this lane's row iff
    // its compile-time offset 32 bb + acc_row(r, 0) is at most one per-lane
    // bound (below the length, at or before the row's position if causal;
    // nothing for a row outside the sequence).
    const int kbound = row_ok ? (CAUSAL ? min(kv_lim - 1, pos) : kv_lim - 1) - kv0 - 4 * h : -1;
    auto grads = [&](auto masked_tag) __attribute__((always_inline)) {
      constexpr bool masked = decltype(masked_tag)::value;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        float ds[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          // registers 4*q4 .. +3: keys kv0 + 32bb + 8q4 + 4h + 0..3 of this lane's row
          uint32_t keep = 0xFu;
          if constexpr (DROP)
            keep = keep_nibble(p, (uint32_t)(kv0 + 32 * bb + 8 * q4 + 4 * h), (uint32_t)row,
                               (uint32_t)bh);
          // mask values of the four keys (a 16-byte group inside the padded row)
          f32x4 m4 = {0.f, 0.f, 0.f, 0.f};
          if constexpr (BIAS)
            m4 = *(const f32x4*)(bias_row + min(kv0 + 32 * bb + 8 * q4 + 4 * h,
                                                (kv_lim - 1) & ~3));
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = 4 * q4 + t;
            const float shift = BIAS ? m4[t] * kLog2e - lse2 : -lse2;
            float pr = fast_exp2(__builtin_fmaf(s[bb][r], p.c2, shift));
            if constexpr (masked) pr = 32 * bb + acc_row(r, 0) <= kbound ? pr : 0.f;
            float g = dp[bb][r];
            if constexpr (DROP) g = (keep >> t) & 1u ? g * p.keep_scale : 0.f;
            ds[r] = pr * (g - dval);
          }
        }
        dsb[bb][0] = pack8(ds);
        dsb[bb][1] = pack8(ds + 8);
      }
    };
    if (full) grads(std::false_type{});
    else grads(std::true_type{});
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          dq[db] = mfma_32x32x16_bf16(tr_operand<D>(kt, 32 * bb + 16 * m, db, lane), dsb[bb][m], dq[db]);
  };

  if (ntiles > 0) {
    load_regs(0);
    store_lds(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      if (more) load_regs((t + 1) * BK);
      compute(t & 1, t * BK);
      if (more) store_lds((t + 1) & 1);
      __syncthreads();
    }
  }

  // dQ = scale * (dQ^T)^T: lane = row, register r of slice db = dim 32db + acc_row(r, h)
  if (row < Nq) {
    uint16_t* dqg = (uint16_t*)p.dq + lay.base + (uint32_t)row * q_ld;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        const f32x16& a = dq[db];
        u32x2 w = {pack_bf16x2(p.scale * a[4 * g], p.scale * a[4 * g + 1]),
                   pack_bf16x2(p.scale * a[4 * g + 2], p.scale * a[4 * g + 3])};
        *(u32x2*)(dqg + d0) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys of one (batch, key/value head); it
// streams the query tiles of every query head that reads this key/value
// head (H / Hkv of them), so the sum over the group needs no atomics
// ---------------------------------------------------------------------------
// The dK/dV kernel with dropout or a mask holds its draws or mask values as
// well: one workgroup per CU (twice the registers) at d = 64 too.
template <int D, int VAR>
constexpr int kDkdvOccupancy = VAR != 0 ? 1 : kBwdOccupancy<D>;
// Waves per dK/dV workgroup.  Eight (two per SIMD, a wave pair splitting the
// rows) wherever the four-wave form runs one wave per SIMD: at d = 128 (the
// packed 16-sequence backward 14.0 -> 10.45 ms, a dense causal one 20-25 %
// faster; with dropout or a mask 3-48 % faster although a few registers
// spill) and at d = 64 with dropout or a mask (18-31 % faster).  Plain d = 64
// keeps four waves at two workgroups per CU (8-10 % faster than eight).
template <int D, int VAR>
constexpr int kDkdvWaves = (D == 128 || VAR != 0) ? 8 : 4;

// WAVES = 4: wave w owns keys 32w .. 32w+31 and every row of a query tile.
// WAVES = 8: waves w and w + 4 own the same 32 keys and split each query
// tile's rows between them (two waves per SIMD, each with half the score
// registers); their dK and dV partial sums are added through LDS at the end.
template <int D, bool CAUSAL, int VAR, int WAVES>
__global__ __launch_bounds__(64 * WAVES, (WAVES == 8 ? 1 : kDkdvOccupancy<D, VAR>))
void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr bool DROP = VAR == 1, BIAS = VAR == 2;
  using C = BwdCfg<D>;
  // 64-row query tiles (at d = 128 with four waves the workgroup then holds
  // 490 of the 512 registers a lane has at one workgroup per CU)
  constexpr int BKW = 128, BQ = 64, NQB = BQ / 32;
  constexpr int NT = 64 * WAVES;     // threads
  constexpr int RS = WAVES / 4;      // waves sharing a key group (row split)
  constexpr int WQB = NQB / RS;      // 32-row blocks of a query tile per wave
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  constexpr int TILE = BQ * C::ROW_BYTES;
  constexpr int LPT = BQ * C::CPR / NT;
  // [stage][Q tile | dO tile | LSE2 (BQ floats) | D (BQ floats)]
  constexpr int STAGE = 2 * TILE + 2 * BQ * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][STAGE];
  // Eight waves: the workgroup's K and V rows stay in LDS ([K | V], chunks
  // permuted as a plainly read tile) instead of in each wave's registers.
  constexpr int KVT = BKW * C::ROW_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[RS == 2 ? 2 * KVT : 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  // causal: lower key tiles see more rows, so ascending is heaviest first
  const GridPos gp = grid_pos(blockIdx.x, p.B * p.Hkv, p.n_ktiles, p.Hkv % 8 == 0 ? 8 : 32);
  const int bhk = gp.pair;
  const int kt_idx = gp.tile;
  const int b = bhk / p.Hkv;
  const int hk = bhk - b * p.Hkv;
  const int G = p.H / p.Hkv;  // query heads hk*G .. hk*G+G-1 read this head
  const int bh_drop = b * p.H + hk * G;  // dropout stream (dense, G == 1)
  const BwdLayout lay = bwd_layout<D>(p, b, hk * G, hk);
  const int kv_lim = lay.kv_lim, off = lay.off;
  const int k0 = kt_idx * BKW;
  // key group; row half (eight waves; 0 with four)
  const int kgrp = RS == 2 ? (wave & 3) : wave, rh = RS == 2 ? (wave >> 2) : 0;
  const int kw0 = k0 + 32 * kgrp;
  const int key = kw0 + l32;
  const bool key_ok = key < kv_lim;
  // additive mask column of this lane's key (clamped into the slice; values
  // of rows and keys outside the sequence are masked out)
  const float* bias_col = nullptr;
  if constexpr (BIAS)
    bias_col = p.bias + (int64_t)b * p.bias_sb + (int64_t)(hk * G) * p.bias_sh +
               min(kw0 + l32, max(kv_lim - 1, 0));

  const uint16_t* kg = (const uint16_t*)p.k + lay.kvbase;
  const uint16_t* vg = (const uint16_t*)p.v + lay.kvbase;
  const int q_ld = lay.q_ld, kv_ld = lay.kv_ld;

  bf16x8 kf[RS == 2 ? 1 : C::KD], vf[RS == 2 ? 1 : C::KD];
  if constexpr (RS == 2) {
    // chunk c of the 128-key tile: row c / CPR, logical chunk c % CPR; keys
    // at or past the length read as zeros (buffer range); the first barrier
    // of the loop orders these stores before the reads
    const uint32_t nb = (uint32_t)max(0, kv_lim - k0) * kv_ld * 2;
    const int64_t at = lay.kvbase + (int64_t)k0 * kv_ld;
#pragma unroll
    for (int i = 0; i < BKW * C::CPR / NT; ++i) {
      const int c = tid + NT * i, r = c / C::CPR, lc = c % C::CPR;
      const uint32_t off = ((uint32_t)r * kv_ld + 8 * lc) * 2;
      *(u32x4*)(&kv_lds[toff_p<D>(r, lc)]) = load_ranged_16((const uint16_t*)p.k + at, nb, off);
      *(u32x4*)(&kv_lds[KVT + toff_p<D>(r, lc)]) = load_ranged_16((const uint16_t*)p.v + at, nb, off);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < C::KD; ++kk) {
      u32x4 a = {0u, 0u, 0u, 0u}, v = {0u, 0u, 0u, 0u};
      if (key_ok) {
        const uint32_t ko = (uint32_t)key * kv_ld + 16 * kk + 8 * h;
        a = *(const u32x4*)(kg + ko);
        v = *(const u32x4*)(vg + ko);
      }
      kf[kk] = __builtin_bit_cast(bf16x8, a);
      vf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // K and V fragments of this lane's key (row 32 kgrp + l32 of the tile),
  // 16-wide head-dim chunk kk
  auto k_frag = [&](int kk) __attribute__((always_inline)) {
    if constexpr (RS == 2) return lds_b128(kv_lds, toff_p<D>(32 * kgrp + l32, 2 * kk + h));
    else return kf[kk];
  };
  auto v_frag = [&](int kk) __attribute__((always_inline)) {
    if constexpr (RS == 2) return lds_b128(kv_lds + KVT, toff_p<D>(32 * kgrp + l32, 2 * kk + h));
    else return vf[kk];
  };

  f32x16 dk[C::ND], dv[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  // Rows whose position is below the key length (the others are padding
  // or see no key), and the query tiles that see any key of this
  // workgroup: rows at positions >= k0 if causal.  Tile t of the loop is
  // query tile qend - 1 - t / G of query head hk*G + t % G (the G heads of a
  // tile, then the next tile down): every key tile of a sequence shares its
  // last query tile, so the workgroups of one (batch, key/value head) pair
  // that run together start on the same rows and stream them in step (from
  // L2), through every head, until each reaches its own first tile.
  const int qlim = max(0, min(lay.Nq, kv_lim - off));
  const int qfirst = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int qend = k0 < kv_lim ? (qlim + BQ - 1) / BQ : 0;
  const int nt = max(0, qend - qfirst);
  const int total = G * nt;

  // Q and dO tiles: chunk i of a thread at a fixed byte offset from the
  // tile's first row; rows at or beyond qlim read as zeros (buffer range).
  u32x4 qst[LPT], dst[LPT];
  float aux = 0.f;  // LSE2 (threads 0..BQ-1) or D (threads BQ..2BQ-1) of one row
  const uint32_t q_off0 = ((uint32_t)(tid / C::CPR) * q_ld + 8 * (tid % C::CPR)) * 2;
  const uint32_t q_step = (NT / C::CPR) * (uint32_t)q_ld * 2;
  auto load_regs = [&](int g, int q0) __attribute__((always_inline)) {
    const int64_t hb = lay.base + g * lay.q_hs + (int64_t)q0 * q_ld;
    const uint32_t nb = (uint32_t)max(0, qlim - q0) * q_ld * 2;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      qst[i] = load_ranged_16((const uint16_t*)p.q + hb, nb, q_off0 + i * q_step);
      dst[i] = load_ranged_16((const uint16_t*)p.dout + hb, nb, q_off0 + i * q_step);
    }
    if (tid < 2 * BQ) {
      const int qr = q0 + (tid % BQ);
      aux = 0.f;
      if (qr < qlim) {
        const int64_t hb = lay.lse_base + g * lay.lse_hs;
        const uint32_t at = (uint32_t)qr * lay.lse_ld;
        if (tid < BQ) {
          // a causal row before the first key has LSE -inf and sees no key
          const float l = (p.lse + hb)[at];
          aux = l == kNegInf ? 0.f : l * kLog2e;
        } else {
          aux = (p.dvec + hb)[at];
        }
      }
    }
  };
  auto store_lds = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + NT * i, r = c / C::CPR, lc = c % C::CPR;
      *(u32x4*)(&lds[st][toff_t<D>(r, lc)]) = qst[i];
      *(u32x4*)(&lds[st][TILE + toff_t<D>(r, lc)]) = dst[i];
    }
    if (tid < 2 * BQ) *(float*)(&lds[st][2 * TILE + 4 * tid]) = aux;
  };

  auto compute = [&](int st, int q0) __attribute__((always_inline)) {
    // the wave's rows (blocks WQB*rh .. +WQB-1) all before its first key, or
    // its keys all padding
    const int wq0 = q0 + 32 * WQB * rh;
    if ((CAUSAL && wq0 + 32 * WQB - 1 + off < kw0) || kw0 >= kv_lim) return;
    const uint8_t* qt = lds[st];
    const uint8_t* dt = lds[st] + TILE;
    const float* lse2 = (const float*)(lds[st] + 2 * TILE);
    const float* dd = lse2 + BQ;
    bf16x8 pb[WQB][2], dsb[WQB][2];
#pragma unroll
    for (int j = 0; j < WQB; ++j) {
      const int qb = WQB * rh + j;
      f32x16 s = f32x16{}, dp = f32x16{};
      const int qr = 32 * qb + l32;
#pragma unroll
      for (int kk = 0; kk < C::KD; ++kk) {
        s = mfma_32x32x16_bf16(lds_b128(qt, toff_t<D>(qr, 2 * kk + h)), k_frag(kk), s);
        dp = mfma_32x32x16_bf16(lds_b128(dt, toff_t<D>(qr, 2 * kk + h)), v_frag(kk), dp);
      }
      // lane = key, register r = row 32qb + acc_row(r, h)
      float pr[16], ds[16];
      // Row q0 + 32 qb + 4 h + c sees this lane's key iff c lies in
      // [rlo, rhi]: below the query count (nothing for a key outside the
      // sequence) and, if causal, at or after the key's position.
      const int rbase = q0 + 32 * qb + 4 * h;
      const int rhi = key_ok ? qlim - 1 - rbase : -1;
      const int rlo = key - off - rbase;
      auto probs = [&](auto masked_tag) __attribute__((always_inline)) {
        constexpr bool masked = decltype(masked_tag)::value;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r0 = 32 * qb + 8 * q4 + 4 * h;  // four consecutive rows
          const f32x4 l4 = *(const f32x4*)(lse2 + r0);
          const f32x4 d4 = *(const f32x4*)(dd + r0);
          // Dropout: the four lanes of a quad hold keys 4m .. 4m+3, one draw
          // group of each row.  Lane u draws for row r0 + u; bit 4t + u of
          // `keep` is then the mask of this lane's key in row r0 + t.
          uint32_t keep = 0xFFFFu;
          if constexpr (DROP) {
            const uint32_t u = (uint32_t)(l32 & 3);
            const uint32_t nib =
                keep_nibble(p, (uint32_t)key, (uint32_t)(q0 + r0) + u, (uint32_t)bh_drop);
            keep = (nib << (4 * u)) | (quad_xor<1>(nib) << (4 * (u ^ 1))) |
                   (quad_xor<2>(nib) << (4 * (u ^ 2))) | (quad_xor<3>(nib) << (4 * (u ^ 3)));
            keep >>= u;
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = 4 * q4 + t;
            float shift = -l4[t];
            if constexpr (BIAS)
              shift += bias_col[(int64_t)min(q0 + r0 + t, max(qlim - 1, 0)) * p.bias_ld] * kLog2e;
            float e = fast_exp2(__builtin_fmaf(s[r], p.c2, shift));
            if constexpr (masked) {
              const int c = 8 * (r >> 2) + (r & 3);  // row q0 + 32 qb + 4 h + c
              const bool vis = CAUSAL ? (c <= rhi && c >= rlo) : c <= rhi;
              e = vis ? e : 0.f;
            }
            if constexpr (DROP) {
              const bool kept = (keep >> (4 * t)) & 1u;
              pr[r] = kept ? e * p.keep_scale : 0.f;
              ds[r] = e * ((kept ? dp[r] * p.keep_scale : 0.f) - d4[t]);
            } else {
              pr[r] = e;
              ds[r] = e * (dp[r] - d4[t]);
            }
          }
        }
      };
      // masks only where the block crosses the diagonal or a length (wave-uniform)
      const int qb0 = q0 + 32 * qb;
      if ((!CAUSAL || kw0 + 31 <= qb0 + off) && qb0 + 31 < qlim && kw0 + 31 < kv_lim)
        probs(std::false_type{});
      else probs(std::true_type{});
      pb[j][0] = pack8(pr);
      pb[j][1] = pack8(pr + 8);
      dsb[j][0] = pack8(ds);
      dsb[j][1] = pack8(ds + 8);
    }
    // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int j = 0; j < WQB; ++j)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int r0 = 32 * (WQB * rh + j) + 16 * m;
          dv[db] = mfma_32x32x16_bf16(tr_operand<D>(dt, r0, db, lane), pb[j][m], dv[db]);
          dk[db] = mfma_32x32x16_bf16(tr_operand<D>(qt, r0, db, lane), dsb[j][m], dk[db]);
        }
  };

  if (total > 0) {
    load_regs(0, (qend - 1) * BQ);
    store_lds(0);
    __syncthreads();
    int g = 0, qi = qend - 1;  // head and query tile of step t
    for (int t = 0; t < total; ++t) {
      const bool more = t + 1 < total;
      const int q0 = qi * BQ;
      if (++g == G) {
        g = 0;
        --qi;
      }
      if (more) load_regs(g, qi * BQ);
      compute(t & 1, q0);
      if (more) store_lds((t + 1) & 1);
      __syncthreads();
    }
  }

  if constexpr (RS == 2) {
    // Waves 4..7 hand their partial sums to waves 0..3 through LDS, dK then
    // dV, laid out [key group][slice][register][lane] in fp32 (64 KiB per
    // tensor at d = 128; every wave has passed the loop's last barrier).
    static_assert(4 * C::ND * 16 * 64 * 4 <= (int)sizeof(lds), "reduction buffer");
    float* red = reinterpret_cast<float*>(&lds[0][0]);
    auto hand_over = [&](f32x16 (&acc)[C::ND]) __attribute__((always_inline)) {
      if (rh == 1) {
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((kgrp * C::ND + db) * 16 + r) * 64 + lane] = acc[db][r];
      }
      __syncthreads();
      if (rh == 0) {
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] += red[((kgrp * C::ND + db) * 16 + r) * 64 + lane];
      }
      __syncthreads();
    };
    hand_over(dk);
    hand_over(dv);
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane = key, register r of slice db = dim
  if (key < lay.Nk && rh == 0) {
    uint16_t* dkg = (uint16_t*)p.dk + lay.kvbase + (uint32_t)key * kv_ld;
    uint16_t* dvg2 = (uint16_t*)p.dv + lay.kvbase + (uint32_t)key * kv_ld;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        const f32x16& a = dk[db];
        const f32x16& v = dv[db];
        u32x2 wk = {pack_bf16x2(p.scale * a[4 * g], p.scale * a[4 * g + 1]),
                    pack_bf16x2(p.scale * a[4 * g + 2], p.scale * a[4 * g + 3])};
        u32x2 wv = {pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3])};
        *(u32x2*)(dkg + d0) = wk;
        *(u32x2*)(dvg2 + d0) = wv;
      }
  }
}

template <int D, bool CAUSAL, int VAR>
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  const int64_t dq_wgs = (int64_t)p.n_qtiles * p.B * p.H;
  const int64_t dkdv_wgs = (int64_t)p.n_ktiles * p.B * p.Hkv;
  if (dq_wgs > 0) {
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, VAR>), dim3((unsigned)dq_wgs), dim3(256), 0,
                       stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dkdv_wgs > 0) {
    constexpr int W = kDkdvWaves<D, VAR>;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, VAR, W>), dim3((unsigned)dkdv_wgs),
                       dim3(64 * W), 0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

template <int VAR>
hipError_t launch_bwd_d(const BwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_bwd<128, true, VAR>(p, stream) : launch_bwd<128, false, VAR>(p, stream);
  if (d != 64) return hipErrorInvalidValue;
  return causal ? launch_bwd<64, true, VAR>(p, stream) : launch_bwd<64, false, VAR>(p, stream);
}

hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, hipStream_t stream) {
  if (p.drop) return launch_bwd_d<1>(p, d, causal, stream);
  if (p.bias) return launch_bwd_d<2>(p, d, causal, stream);
  return launch_bwd_d<0>(p, d, causal, stream);
}

}  // namespace fa
