// Fused attention forward for bf16 Q/K/V on gfx950 (CDNA4).
//
// One workgroup owns a tile of 32*WAVES query rows of one (batch, head) and
// keeps, per row, the running maximum m, denominator l and unnormalised
// numerator a of "FlashAttention: Exact Attention as an IO-Aware Streaming
// Computation" (section "Mathematical structure"), while key/value tiles
// stream through LDS ("IO-aware exact attention", section "One tiled
// forward-pass iteration").  Score tiles live only in registers; only O and
// the per-row log-sum-exp are written.
//
// Data movement.  K and V tiles go from HBM straight into LDS with buffer
// loads (no register staging), through a ring of NSTAGE LDS stages: the
// loads for tile t + NSTAGE - 1 are issued while tile t is computed.  The
// buffer range is the sequence's valid keys, so rows past the end arrive as
// zeros.  Both tiles are row-major [key][dim] with the 16-byte chunks of each
// row permuted by an XOR of the row index, which makes the fragment reads
// below free of bank conflicts.
//
// Products.  Each wave (32 query rows) computes the transposed score tile
// S^T = K Q^T on 32x32x16 bf16 MFMA (K fragments from LDS, Q fragments
// resident in registers), so that each lane holds the scores of one query
// row: row max and row sum are in-lane reductions plus one exchange between
// the two wave halves.  The probabilities are packed to bf16 in place; that
// packing is already the B operand of O^T = V^T P^T.  The matching V^T
// operand comes from the row-major V tile through transpose reads
// (ds_read_b64_tr_b16), which hand each lane one head-dim column across four
// consecutive keys.  O^T keeps one query row per lane, so rescaling the
// numerator is one multiply per register.
//
// Reference maximum.  Scores are exponentiated against a per-row reference
// value, which is raised to the running maximum only when a tile's weights
// against the old one would exceed kWeightBound (the test is on the sums
// the denominator needs anyway, so the common path computes no row
// maximum).  The denominator and numerator always share the reference, so
// o = a / l is unchanged: this is the glossary page's observation ("Why a
// tile can be discarded") that any common reference maximum preserves the
// exponential sums, and it skips most rescales of the accumulator.
//
// Causal tiles run heaviest first; consecutive workgroups cycle over
// (batch, head) so all tiles of a head land on one XCD when B*H is a
// multiple of 8 (workgroups are dealt round-robin to the 8 XCDs).  A causal
// grid of 128-row tiles that fits the device at most twice over splits each
// tile's keys between two wave groups, and when its pairs of tiles (j,
// n - 1 - j) fill the device a workgroup takes a whole pair.  With
// per-sequence key lengths a non-causal batch runs its sequences longest
// first, and a causal one its query tiles by index, last first, across all
// sequences.
#include "fa_bf16_tiles.hpp"
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

// Bound on one lane's sum of the weights of a tile (and so on each weight)
// before the reference maximum is raised: weights stay below 2^16.
constexpr float kWeightBound = 65536.0f;

// LDS stages of the ping-pong schedule (4 x 32 KiB).  Five fit in 160 KiB
// but the extra address state spills registers at 8 waves per CU and
// measured slower.
constexpr int kPingPongStages = 4;


// Largest batch for which a launch over sequences of different lengths
// orders its tiles longest sequence first (the order is worked out in every
// workgroup, in O(B^2) scalar steps).
constexpr int kLptBatches = 8;

template <int S>
struct StageTag {
  static constexpr int value = S;
};

// BKX, if not 0, sets the keys per streamed tile.  KS = 2 splits the waves
// into two groups over the same query rows, each taking every other key tile
// (an LDS stage then holds the two groups' tiles side by side).
template <int D, int WAVES, int NSTAGE, int BKX = 0, int KS = 1>
struct Bf16Cfg {
  static constexpr int BQ = 32 * WAVES / KS;     // query rows per workgroup
  static constexpr int BK = BKX ? BKX : (D == 128 ? 64 : 128);  // keys per streamed tile
  static constexpr int SK = KS * BK;             // keys per LDS stage
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int TILE_BYTES = SK * ROW_BYTES;  // the K (or V) rows of one stage
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES; // K tile + V tile
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
  static constexpr int LOADS = TILE_BYTES / 1024 / WAVES;  // 1 KiB loads per wave per tensor
  static constexpr int LOADS_PER_TILE = 2 * LOADS;         // K and V, per wave
  static constexpr int NB = BK / 32;             // 32-key blocks per tile
  static constexpr int ND = D / 32;              // 32-wide slices of the head dim
  static_assert(LOADS * WAVES * 1024 == TILE_BYTES, "tile must split into 1 KiB wave loads");
  static_assert(NSTAGE >= 2 && NSTAGE <= 5, "2..5 LDS stages");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};


template <int D, bool CAUSAL, int WAVES, int NSTAGE, bool PINGPONG, bool DROP = false,
          bool BIAS = false, bool PERSIST = false, int BKX = 0, int KS = 1, bool PAIR = false>
// Two lockstep workgroups per CU (256 registers per lane), except with an
// additive mask at d = 64, whose extra registers do not fit: one workgroup;
// and three with 64-key tiles at d = 64 (168 registers).
__global__ __launch_bounds__(64 * WAVES,
                             (WAVES == 4 && D == 64 && BKX == 64 && !BIAS && !DROP) ? 3
                             : (WAVES == 4 && NSTAGE == 2 && !(BIAS && D == 64)) ? 2 : 1)
void fa_fwd_bf16_kernel(FwdParams p) {
  static_assert(!(DROP || BIAS) || !PINGPONG, "dropout and bias run in the lockstep schedule");
  static_assert(!PERSIST || PINGPONG, "the persistent form is the ping-pong schedule's");
  static_assert(KS == 1 || (KS == 2 && WAVES == 8 && !PINGPONG && !DROP && !BIAS),
                "the key split is a plain lockstep form of eight waves");
  static_assert(!PAIR || (KS == 2 && CAUSAL), "the paired form is a causal key split");
  using C = Bf16Cfg<D, WAVES, NSTAGE, BKX, KS>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];

  const int tid = threadIdx.x;
  // wave index as a scalar (it is uniform), so LDS destinations of the
  // direct loads are computed on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- tile assignment ----------------------------------------------------
  // Workgroup = (key range, (batch, head), query tile); consecutive ids
  // cycle over a chunk of at most 32 (batch, head) pairs, then over the
  // query tiles, then over the chunks, then over the key ranges.  Within a
  // chunk all the query tiles of a head run close together, so its K/V rows
  // are reused from L2; with 32 pairs per chunk every head's tiles, of every
  // range, land on one XCD (workgroups are dealt round-robin to the 8 XCDs),
  // and the heads of a sequence are spread evenly over the XCDs, so ranges
  // left empty by a short sequence do not idle some XCDs.
  const int BH = p.B * p.H;
  // Persistent form (dense layout, one key range): workgroup w takes the
  // units w, w + G, w + 2G, ... (G workgroups, p.persist units each); unit
  // u is the query tiles n_qtiles - 1 - j and j of (batch, head) u % BH,
  // j = u / BH, in that order.  The two tiles of a unit see n_qtiles + 1
  // query tiles' worth of keys together under the causal mask, so every
  // workgroup gets the same work; with G a multiple of 8 and BH a multiple
  // of 8, all the units of a (batch, head) run on the XCD of its workgroups.
  auto item_of = [&](const int i, int& ibh, int& iqt) __attribute__((always_inline)) {
    const int u = (int)blockIdx.x + (i >> 1) * (int)gridDim.x;
    ibh = u % BH;
    const int j = u / BH;
    iqt = (i & 1) ? j : p.n_qtiles - 1 - j;
  };
  int split = 0, bh, qt;
  int pair_j = 0;  // paired form: the light query tile of this workgroup's pair
  if constexpr (PERSIST) {
    item_of(0, bh, qt);
  } else if (PAIR) {
    // Paired form (causal, dense, as many keys as queries): workgroup x
    // takes query tiles n_qtiles - 1 - j and j of (batch, head) x % BH,
    // j = x / BH, which together see n_qtiles + 1 tiles' worth of keys
    // (one tile when the two coincide: the middle tile of an odd count), so
    // every workgroup has the same work; (batch, head) fastest, so a head
    // keeps one XCD when BH is a multiple of 8.
    const int x = (int)blockIdx.x;
    pair_j = x / BH;
    bh = x - pair_j * BH;
    qt = p.n_qtiles - 1 - pair_j;
  } else if (!CAUSAL && p.key_len && !p.cu_q && p.splits == 1 && !p.end_aligned &&
             p.B <= kLptBatches) {
    // Dense batch with per-sequence key lengths, not causal: a query tile of
    // sequence b costs ceil(L_b / BK) key tiles (a tile of rows past L_b
    // only writes zeros), so the work differs between sequences only.  The
    // grid takes the sequences in order of decreasing length (ties by
    // index), each one's tiles query-tile major with the heads fastest (so
    // a head's tiles keep one XCD when H is a multiple of 8): the longest
    // work starts first, and each sequence's padding tiles, which finish at
    // once, sit between it and the next.
    const int per_seq = p.H * p.n_qtiles;
    const int rank = (int)blockIdx.x / per_seq;
    const int local = (int)blockIdx.x - rank * per_seq;
    int len[kLptBatches];
#pragma unroll
    for (int i = 0; i < kLptBatches; ++i) {
      const int L = i < p.B ? p.key_len[i] : -1;
      len[i] = L < 0 ? (i < p.B ? 0 : -1) : (L > p.Nk ? p.Nk : L);
    }
    int sb = 0;
#pragma unroll
    for (int i = 0; i < kLptBatches; ++i) {
      int ahead = 0;  // sequences before i in the order
#pragma unroll
      for (int j = 0; j < kLptBatches; ++j)
        ahead += (j < p.B && (len[j] > len[i] || (len[j] == len[i] && j < i))) ? 1 : 0;
      if (i < p.B && ahead == rank) sb = i;
    }
    sb = __builtin_amdgcn_readfirstlane(sb);
    qt = local / p.H;
    bh = sb * p.H + (local - qt * p.H);
  } else if (CAUSAL && p.key_len && !p.cu_q && p.splits == 1 && !p.end_aligned) {
    // Causal batch with per-sequence key lengths: a query tile's work grows
    // with its index up to its sequence's length, so the grid runs the query
    // tiles of every (batch, head) from the last to the first, one round
    // per tile index ((batch, head) fastest; a head keeps one XCD when B*H is
    // a multiple of 8), which puts the heaviest tiles of every sequence
    // first instead of those of the first sequences.
    const int x = (int)blockIdx.x;
    const int r = x / BH;
    bh = x - r * BH;
    qt = p.n_qtiles - 1 - r;
  } else {
    const int per_split = BH * p.n_qtiles;
    split = (int)blockIdx.x / per_split;
    const int x = (int)blockIdx.x - split * per_split;
    constexpr int kChunk = 32;
    const int chunk_wgs = kChunk * p.n_qtiles;
    const int chunk = x / chunk_wgs;
    const int in_chunk = x - chunk * chunk_wgs;
    const int chunk_heads = min(kChunk, BH - chunk * kChunk);
    bh = chunk * kChunk + in_chunk % chunk_heads;
    qt = in_chunk / chunk_heads;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest tiles first
  }
  int b = bh / p.H;
  int hq = bh - b * p.H;
  int hk = hq / (p.H / p.Hkv);  // the key/value head this query head reads
  // Layout of this (batch, head): dense [B, H, N, d] / [B, Hkv, Nk, d], or a
  // packed batch [T, H, d] / [T, Hkv, d] with sequence b at rows cu[b] ..
  // cu[b+1]-1.  Row strides and bases in elements; all workgroup-uniform.
  int N, Nk, q_ld, kv_ld, lse_ld;
  int64_t base, kvbase, lse_base;
  if (p.cu_q) {
    const int s0 = p.cu_q[b], k0 = p.cu_k[b];
    N = __builtin_amdgcn_readfirstlane(p.cu_q[b + 1] - s0);
    Nk = __builtin_amdgcn_readfirstlane(p.cu_k[b + 1] - k0);
    q_ld = p.H * D;
    kv_ld = p.Hkv * D;
    base = ((int64_t)__builtin_amdgcn_readfirstlane(s0) * p.H + hq) * D;
    kvbase = ((int64_t)__builtin_amdgcn_readfirstlane(k0) * p.Hkv + hk) * D;
    lse_base = (int64_t)__builtin_amdgcn_readfirstlane(s0) * p.H + hq;
    lse_ld = p.H;
  } else {
    N = p.N;
    Nk = p.Nk;
    q_ld = D;
    kv_ld = D;
    base = (int64_t)bh * N * D;
    kvbase = ((int64_t)b * p.Hkv + hk) * Nk * D;
    lse_base = (int64_t)bh * N;
    lse_ld = 1;
  }
  int q0 = qt * C::BQ;
  int kv_lim = Nk;
  if (p.key_len) {
    const int L = p.key_len[b];
    kv_lim = L < 0 ? 0 : (L > Nk ? Nk : L);
  }
  // uniform across the workgroup; keep it (and all that derives from it,
  // such as the buffer ranges) in scalar registers
  kv_lim = __builtin_amdgcn_readfirstlane(kv_lim);
  // Query row i sits at key position i + off: i itself, or, with the rows
  // aligned to the end of the sequence's keys, i + L_b - N (then no row is
  // padding).
  const int off = p.end_aligned ? kv_lim - N : 0;
  // Keys this query tile can see: below the length and, if causal, at or
  // before the position of its last row.
  int n_kv = kv_lim;
  if (CAUSAL) n_kv = min(n_kv, max(0, q0 + C::BQ + off));
  if (q0 + off >= kv_lim) n_kv = 0;  // every row of the tile is padding
  // This workgroup's key range; ranges are whole tiles, so only the
  // sequence end and the diagonal need element masks.
  const int kv_first = split * p.split_keys;
  const int kv_last = min(n_kv, kv_first + p.split_keys);
  int ntiles = kv_last > kv_first ? (kv_last - kv_first + C::BK - 1) / C::BK : 0;
  // Paired form: the heavy query tile qt has ntiles key tiles, the light
  // one n_l (none when it is qt itself).  Group 0 takes the heavy tile's
  // key tiles 0 .. g0 - 1; group 1 the light tile's n_l key tiles, then the
  // heavy tile's from the last one down to g0: g0 = ceil((ntiles + n_l) / 2)
  // steps, group 1 idle in the last one when the total is odd.  In the
  // first n_l steps both groups work on the same keys, so group 1 reads
  // group 0's half of the stage and its own half is not fetched.
  const int n_l = PAIR && pair_j != qt ? (min(kv_lim, pair_j * C::BQ + C::BQ) + C::BK - 1) / C::BK : 0;
  const int g0 = PAIR ? (ntiles + n_l + 1) / 2 : 0;

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + base;

  // with the key split, waves w and w + WAVES/2 own the same rows; kgrp is
  // the key group (even or odd key tiles)
  const int kgrp = KS == 2 ? wave / (WAVES / 2) : 0;
  int qw0 = q0 + 32 * (KS == 2 ? wave % (WAVES / 2) : wave);  // first query row of this wave
  int qrow = qw0 + l32;      // the query row this lane owns
  int qwpos = qw0 + off;     // key position of the wave's first row
  int qpos = qrow + off;     // key position of this lane's row

  // Paired form: group 1 starts on the light tile's rows (the heavy tile's
  // are taken over after its last light key tile).
  const int qw0_heavy = qw0;
  bool light_pending = PAIR && kgrp == 1 && n_l > 0;
  if (light_pending) {
    qw0 = pair_j * C::BQ + 32 * (wave % (WAVES / 2));
    qrow = qw0 + l32;
    qwpos = qw0 + off;
    qpos = qrow + off;
  }

  // ---- Q fragments (B operand of S^T = K Q^T) -----------------------------
  // (the persistent form loads them at the start of each query tile)
  bf16x8 qf[D / 16];
  auto load_q = [&](const int row, bf16x8 (&dst)[D / 16]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < N) w = *(const u32x4*)(qg + (int64_t)row * q_ld + 16 * kk + 8 * h);
      w ^= p.q_sign;
      dst[kk] = __builtin_bit_cast(bf16x8, w);
    }
  };
  if constexpr (!PERSIST) load_q(qrow, qf);
  // paired form, group 1: the heavy tile's rows (loaded during the first step)
  bf16x8 qf_heavy[PAIR ? D / 16 : 1];

  // ---- K/V tile loads: HBM -> LDS, range-checked ---------------------------
  // Buffer range = the valid keys of this (batch, head): loads beyond it
  // return zeros, so padded keys contribute exact zeros to both products.
  const uint32_t row_stride = (uint32_t)kv_ld * 2;  // bytes between key rows in memory
  const uint32_t valid_bytes = (uint32_t)kv_lim * row_stride;
  const void* kbase = (const uint16_t*)p.k + kvbase;
  const void* vbase = (const uint16_t*)p.v + kvbase;
  // Per-lane source offsets within a tile (bytes): load i of this wave fills
  // the 1 KiB LDS block WAVES*i + wave; lane l fills its 16-byte chunk l.
  uint32_t koff[C::LOADS], voff[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int pch = (WAVES * i + wave) * 64 + lane;  // physical chunk index in the tile
    const int row = pch / C::CPR, phys = pch % C::CPR;
    koff[i] = row * row_stride + 16 * k_chunk<D>(row, phys);  // XOR is its own inverse
    voff[i] = row * row_stride + 16 * v_chunk<D>(row, phys);
  }
  // With nbytes = 0 every lane is out of range: the stage is filled with
  // zeros and no memory is read.
  auto load_tile_n = [&](int kv0, int stage, uint32_t nbytes) __attribute__((always_inline)) {
    uint8_t* ks = lds + stage * C::STAGE_BYTES;
    uint8_t* vs = ks + C::TILE_BYTES;
    const uint32_t tile_off = __builtin_amdgcn_readfirstlane((uint32_t)kv0 * row_stride);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int blk = (WAVES * i + wave) * 1024;
      // The whole offset goes in the per-lane operand: the range check
      // covers that operand (not the scalar one).
      load_lds_16(kbase, nbytes, ks + blk, koff[i] + tile_off);
      load_lds_16(vbase, nbytes, vs + blk, voff[i] + tile_off);
    }
  };
  auto load_tile = [&](int kv0, int stage) __attribute__((always_inline)) {
    load_tile_n(kv0, stage, valid_bytes);
  };

  // ---- running state (one query row per lane) -----------------------------
  f32x16 o_acc[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) o_acc[i] = f32x16{};
  float m_ref = kNegInf;  // reference maximum of scale*log2(e)*s
  float l_run = 0.f;      // this lane's part of the fp32 denominator
  float lp_run = 0.f;     // the same over the bf16-rounded probabilities
  float lp_run2 = 0.f;    // its second chain in the ping-pong schedule (o uses the sum)
  // With an additive mask the scores are taken to log2 units (and the mask
  // added) before the softmax step, which then works with a unit scale.
  const float c = BIAS ? 1.f : p.c;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Waves whose rows see no key of the tile at kv0 skip it (wave-uniform).
  auto skip_tile = [&](const int kv0) __attribute__((always_inline)) {
    return (CAUSAL && kv0 > qwpos + 31) || (qwpos >= kv_lim) || (qw0 >= N);
  };

  // ---- LDS fragment reads ---------------------------------------------------
  // Both products read their LDS operands in groups of four MFMAs' worth,
  // issued one group ahead of the MFMAs that use them (untracked reads with
  // explicit waits; LDS operations of a wave complete in order).
  //
  // K fragment (kk, bb): row 32*bb + l32 of the tile, logical chunk 2*kk + h.
  // The swizzle depends on the row only through l32, so each kk has one
  // per-lane offset and bb is an immediate.
  uint32_t k_lane_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    k_lane_off[kk] = l32 * C::ROW_BYTES + 16 * k_chunk<D>(l32, 2 * kk + h);
  constexpr int KG = (D / 16) * C::NB / 4;  // K read groups per tile (4 reads each)
  auto k_issue = [&](auto gc, const uint32_t kbase, bf16x8 (&dst)[4])
      __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value;
    static_for<4>([&](auto jc) __attribute__((always_inline)) {
      constexpr int i = 4 * g + decltype(jc)::value;
      constexpr int kk = i / C::NB, bb = i % C::NB;
      dst[decltype(jc)::value] =
          lds_read_b128_async<bb * 32 * C::ROW_BYTES>(kbase + k_lane_off[kk]);
    });
  };
  bf16x8 kr[KG][4];

  // S^T = K Q^T for the K tile at kbase: NB accumulators of 32 keys x 32
  // queries.  With PRE = 1, K group 0 must already be in flight (k_issue
  // into kr[0]) and each later group is issued one group ahead; with
  // PRE = KG all groups are already in flight, in order, in kr[g].
  auto compute_s = [&](const uint32_t kbase, f32x16 (&s)[C::NB], auto pre_tag)
      __attribute__((always_inline)) {
    constexpr int PRE = decltype(pre_tag)::value;
    static_assert(PRE == 1 || PRE == KG, "chained or all in flight");
#pragma unroll
    for (int bb = 0; bb < C::NB; ++bb) s[bb] = f32x16{};
    static_for<KG>([&](auto gc) __attribute__((always_inline)) {
      constexpr int g = decltype(gc)::value;
      constexpr int buf = PRE == 1 ? (g & 1) : g;
      if constexpr (PRE == 1) {
        if constexpr (g + 1 < KG) {
          k_issue(std::integral_constant<int, g + 1>{}, kbase, kr[(g + 1) & 1]);
          lds_wait4<4>(kr[buf]);
        } else {
          lds_wait4<0>(kr[buf]);
        }
      } else {
        lds_wait4<4 * (KG - 1 - g)>(kr[buf]);
      }
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int i = 4 * g + decltype(jc)::value;
        constexpr int kk = i / C::NB, bb = i % C::NB;
        s[bb] = mfma_32x32x16_bf16(kr[buf][decltype(jc)::value], qf[kk], s[bb]);
      });
      // each group's MFMAs stay between its wait and the next one (the
      // compiler would otherwise gather the waits ahead of all MFMAs)
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Scores of the tile at kv0 -> bf16 probabilities (the B operand of the
  // second product), with the running reference maximum and denominators
  // brought up to date.
  // P = exp2(c*s + neg_m), packed to bf16 into pf (the B operand of the
  // second product); returns this lane's sum of the fp32 values, which feeds
  // the log-sum-exp (the sum of the bf16-rounded values, lp_run, for o is
  // taken in the second product's step).
  auto exp_pack = [&](f32x16 (&s)[C::NB], bf16x8 (&pf)[C::NB][2], const float neg_m)
      __attribute__((always_inline)) {
    // -0 is the identity of fp32 addition (0 is not, for -0 operands), so the
    // compiler drops the first addition of each chain
    float part[4] = {-0.f, -0.f, -0.f, -0.f};
#pragma unroll
    for (int bb = 0; bb < C::NB; ++bb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // a group's eight FMAs, then its eight exponentials, then its sums
        // and packing (the compiler would pair each FMA with its
        // exponential; the blocked order measured 0.2-0.7 % faster)
        float e[8];
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
          e[t8] = __builtin_fmaf(s[bb][8 * half + t8], c, neg_m);
        asm volatile("" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]),
                     "+v"(e[6]), "+v"(e[7]));
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
          // masked scores are -inf and c > 0, so they give exactly 0
          e[t8] = fast_exp2(e[t8]);
        asm volatile("" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]),
                     "+v"(e[6]), "+v"(e[7]));
        bf16x2 pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          part[j] += e[2 * j] + e[2 * j + 1];
          pr[j] = bf16x2{(__bf16)e[2 * j], (__bf16)e[2 * j + 1]};
        }
        pf[bb][half] = bf16x8{pr[0][0], pr[0][1], pr[1][0], pr[1][1],
                              pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
      }
    }
    return (part[0] + part[1]) + (part[2] + part[3]);
  };

  // Scores of the tile at kv0 -> bf16 probabilities, with the reference
  // maximum and the fp32 denominator brought up to date.  mid() runs after
  // the masking, before the exponentials.
  //
  // The weights are first taken against the current reference.  Each
  // weight of a lane is at most the lane's sum, so a sum within
  // kWeightBound bounds them all and the tile is accepted as it is; inf and
  // NaN fail that test.  Only otherwise (and for a row's first tile, when
  // the reference is still -inf) does the wave find the tile's row maxima,
  // raise the reference to the running maximum, rescale its state and redo
  // the exponentials.  The reference therefore moves only when some weight
  // would exceed the bound, and the row maximum costs nothing on the
  // common path.
  // Additive mask (fp32, row-major with row stride bias_ld): the lane's row,
  // keys kv0 + 32*bb + 8*q4 + 4*h + 0..3 as one 16-byte load per (bb, q4).
  // With two 32-key blocks per tile the loads are issued before the first
  // product of the tile; with four (d = 64) the registers are not there, and
  // each block's values are loaded just before they are added.
  constexpr bool kBiasAhead = C::NB <= 2;
  f32x4 bias_r[BIAS && kBiasAhead ? C::NB : 1][4];
  const float* bias_row = BIAS && qrow < N
                              ? p.bias + (int64_t)b * p.bias_sb + (int64_t)hq * p.bias_sh +
                                    (int64_t)qrow * p.bias_ld
                              : nullptr;
  auto bias_load = [&](const int kv0, const int bb, f32x4 (&dst)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int key0 = kv0 + 32 * bb + 8 * q4 + 4 * h;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (bias_row && key0 < kv_lim) x = *(const f32x4*)(bias_row + key0);
      dst[q4] = x;
    }
  };
  auto bias_issue = [&](const int kv0) __attribute__((always_inline)) {
    if constexpr (BIAS && kBiasAhead) {
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb) bias_load(kv0, bb, bias_r[bb]);
    }
  };

  auto softmax = [&](const int kv0, f32x16 (&s)[C::NB], bf16x8 (&pf)[C::NB][2], auto&& mid)
      __attribute__((always_inline)) {
    // Element masks only where the tile crosses the diagonal or the
    // sequence end (wave-uniform test).
    if constexpr (BIAS) {
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb) {
        f32x4 x[4];
        if constexpr (kBiasAhead) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) x[q4] = bias_r[bb][q4];
        } else {
          bias_load(kv0, bb, x);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[bb][r] = __builtin_fmaf(s[bb][r], p.c, x[r >> 2][r & 3] * kLog2e);
      }
    }
    const bool masked = (CAUSAL && kv0 + C::BK - 1 > qwpos) || (kv0 + C::BK > kv_lim);
    if (masked) {
      // Key kv0 + 32 bb + acc_row(r, h) is visible iff it is below the
      // length and (causal) at or before the row's position, i.e. iff the
      // compile-time offset 32 bb + acc_row(r, 0) is at most one per-lane
      // bound: one compare and one select per score.
      int bound = kv_lim - 1 - kv0;
      if (CAUSAL) bound = min(bound, qpos - kv0);
      bound -= 4 * h;
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[bb][r] = 32 * bb + acc_row(r, 0) <= bound ? s[bb][r] : kNegInf;
    }
    mid();
    bool slow = __any(m_ref == kNegInf);
    float lt = 0.f;
    if (!slow) {
      lt = exp_pack(s, pf, -m_ref);
      slow = __any(!(lt <= kWeightBound));
    }
    if (slow) {
      // Row maximum: four independent partial maxima, then the wave halves.
      float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[bb][r]);
      const float mx = halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      // -inf - (-inf) is never formed
      const float m_blk = (mx == kNegInf) ? kNegInf : mx * c;
      const float m_new = fmaxf(m_ref, m_blk);
      const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
      lp_run *= alpha;
      lp_run2 *= alpha;
#pragma unroll
      for (int i = 0; i < C::ND; ++i) o_acc[i] *= alpha;
      lt = exp_pack(s, pf, (m_ref == kNegInf) ? 0.f : -m_ref);
    }
    l_run += lt;
  };

  // O^T += V^T P^T.  V^T fragments come from transpose reads of the V tile,
  // eight reads (four MFMAs) per group.  In each 16-lane group, lane r
  // reads key +r/4 and dims +4*(r%4), so lane r receives dim r of four
  // consecutive keys; the swizzle chunk of such a read depends on the lane
  // and the head-dim slice only, so each slice has one per-lane offset and
  // the key offsets are immediates.
  // MFMA m of the second product multiplies head-dim slice pv_db(m) by the
  // 16-key chunk pv_kc(m) of the tile.  The lockstep schedule alternates the
  // slices (consecutive MFMAs write different accumulators: 3 % faster at
  // d = 64 with 64-key tiles); the ping-pong keeps each slice's chunks
  // together (no difference measured there).
  auto pv_db = [](const int m) constexpr { return PINGPONG ? m / (2 * C::NB) : m % C::ND; };
  auto pv_kc = [](const int m) constexpr { return PINGPONG ? m % (2 * C::NB) : m / C::ND; };
  uint32_t v_lane_off[C::ND];
#pragma unroll
  for (int db = 0; db < C::ND; ++db) {
    const int r16 = lane & 15, g16 = (lane >> 4) & 1;
    const int key = 4 * h + (r16 >> 2);
    const int dim = 32 * db + 16 * g16 + 4 * (r16 & 3);
    v_lane_off[db] = key * C::ROW_BYTES + 16 * v_chunk<D>(key, dim >> 3) + (dim & 7) * 2;
  }
  constexpr int VG = C::ND * C::NB * 2 / 4;  // V read groups per tile (8 reads each)
  auto v_issue = [&](auto gc, const uint32_t vbase, bf16x4 (&dst)[8])
      __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value;
    static_for<8>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      constexpr int m = 4 * g + i / 2;  // MFMA index
      constexpr int db = pv_db(m), bb = pv_kc(m) / 2, half = pv_kc(m) % 2;
      constexpr int off = (32 * bb + 16 * half + 8 * (i % 2)) * C::ROW_BYTES;
      dst[i] = lds_read_tr16_async<off>(vbase + v_lane_off[db]);
    });
  };
  bf16x4 vr[2][8];

  // The second product for the V tile at vbase, V group 0 already in flight
  // (v_issue into vr[0]).  With chain_k, K group 0 of the tile at kbase is
  // issued behind the last V group, so the first product can follow without
  // waiting for LDS.
  auto pv = [&](const uint32_t vbase, const bf16x8 (&pf)[C::NB][2], auto chain_tag,
                const uint32_t kbase) __attribute__((always_inline)) {
    constexpr bool chain_k = decltype(chain_tag)::value;
    constexpr bool sum_weights = !DROP;  // with dropout the sum is taken before the mask
    static_for<VG>([&](auto gc) __attribute__((always_inline)) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 1 < VG) {
        v_issue(std::integral_constant<int, g + 1>{}, vbase, vr[(g + 1) & 1]);
        lds_wait8<8>(vr[g & 1]);  // group g complete; g + 1 may be in flight
      } else if constexpr (chain_k) {
        k_issue(std::integral_constant<int, 0>{}, kbase, kr[0]);
        lds_wait8<4>(vr[g & 1]);
      } else {
        lds_wait8<0>(vr[g & 1]);
      }
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int m = 4 * g + decltype(jc)::value;
        constexpr int db = pv_db(m), bb = pv_kc(m) / 2, half = pv_kc(m) % 2;
        const bf16x4 v0 = vr[g & 1][2 * (m % 4)], v1 = vr[g & 1][2 * (m % 4) + 1];
        const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o_acc[db] = mfma_32x32x16_bf16(vf, pf[bb][half], o_acc[db]);
      });
      // lp_run, the sum of the bf16 weights the product multiplies, so that
      // a / lp_run is an exact convex combination of V rows under those
      // weights (a dominant key is then reproduced without the 2^-9 error
      // of its rounded weight).  The dot products run on the matrix pipe:
      // here they slot in between this wave's own MFMAs, where in the
      // softmax step each would wait for a whole MFMA of the other wave
      // sharing the SIMD.  Group g sums 2*NB/NG of the weight vectors.
      constexpr int PER = 2 * C::NB / VG;
      if constexpr (sum_weights) {
        static_for<PER>([&](auto ic) __attribute__((always_inline)) {
          constexpr int f = g * PER + decltype(ic)::value;
          const bf16x8 w = pf[f / 2][f % 2];
          static_for<4>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            lp_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[2 * j], w[2 * j + 1]}, ones,
                                                     lp_run, false);
          });
        });
        // keeps the compiler from sinking the sum into the softmax step
        asm volatile("" : "+v"(lp_run));
      }
    });
  };

  // The second product from V fragments already in flight in vpre (all
  // groups, issued in that order), followed by KPRE more LDS reads.  A wave
  // has at most 15 LDS operations outstanding (the issue of a 16th waits),
  // so a count above 15 is the same as 15: those outstanding are always the
  // most recent ones.
  bf16x4 vpre[VG][8];
  // Groups [G0, G1) of the V fragments, issued at this point of the code.
  auto v_issue_range = [&](const uint32_t vbase, auto g0_tag, auto g1_tag)
      __attribute__((always_inline)) {
    static_for<VG>([&](auto gc) __attribute__((always_inline)) {
      if constexpr (decltype(gc)::value >= decltype(g0_tag)::value &&
                    decltype(gc)::value < decltype(g1_tag)::value)
        v_issue(gc, vbase, vpre[gc]);
    });
    __builtin_amdgcn_sched_barrier(0);  // issued here, ahead of the work that follows
  };
  // KPRE reads were issued after the V groups, before this call; after(g)
  // runs behind the MFMAs of group g and issues KPER reads (g < VG - 1).
  auto pv_pre = [&](const bf16x8 (&pf)[C::NB][2], auto kpre_tag, auto kper_tag, auto&& after)
      __attribute__((always_inline)) {
    constexpr int KPRE = decltype(kpre_tag)::value;
    constexpr int KPER = decltype(kper_tag)::value;
    // lp_run + lp_run2, the sum of the bf16 weights the product multiplies,
    // so that a / (lp_run + lp_run2) is an exact convex combination of V
    // rows under those weights (a dominant key is then reproduced without
    // the 2^-9 error of its rounded weight).  The dot products run on the
    // matrix pipe: here, back to back ahead of this wave's own MFMAs
    // (interleaved with them, each one costs the pipe a turnaround; in the
    // softmax step each would wait for a whole MFMA of the other wave
    // sharing the SIMD), in two independent chains (one chain waits out
    // each product's latency: 1 % slower on the whole kernel).
    static_for<2 * C::NB>([&](auto fc) __attribute__((always_inline)) {
      constexpr int f = decltype(fc)::value;
      const bf16x8 w = pf[f / 2][f % 2];
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        float& acc = j % 2 == 0 ? lp_run : lp_run2;
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[2 * j], w[2 * j + 1]}, ones, acc, false);
      });
    });
    asm volatile("" : "+v"(lp_run), "+v"(lp_run2));  // keeps the sums here
    __builtin_amdgcn_sched_barrier(0);
    static_for<VG>([&](auto gc) __attribute__((always_inline)) {
      constexpr int g = decltype(gc)::value;
      constexpr int later = 8 * (VG - 1 - g) + KPRE + KPER * g;
      lds_wait8<(later > 15 ? 15 : later)>(vpre[g]);
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int m = 4 * g + decltype(jc)::value;
        constexpr int db = pv_db(m), bb = pv_kc(m) / 2, half = pv_kc(m) % 2;
        const bf16x4 v0 = vpre[g][2 * (m % 4)], v1 = vpre[g][2 * (m % 4) + 1];
        const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o_acc[db] = mfma_32x32x16_bf16(vf, pf[bb][half], o_acc[db]);
      });
      after(gc);
      __builtin_amdgcn_sched_barrier(0);  // keeps the group's MFMAs here
    });
  };

  // Dropout on the probabilities: the weight sum that normalises O is taken
  // over the undropped bf16 weights first, then each weight whose draw is
  // below the threshold is zeroed (the 1 / (1 - p) scale is applied to O at
  // the end).  The draw of query row i and key j is word j % 4 of Philox
  // on the counter (j / 4, i, b * H + h, offset); a lane's 16 keys of a
  // 32-key block are four aligned groups of four, one Philox call each.
  auto dropout = [&](const int kv0, bf16x8 (&pf)[C::NB][2]) __attribute__((always_inline)) {
    static_for<2 * C::NB>([&](auto fc) __attribute__((always_inline)) {
      constexpr int f = decltype(fc)::value;
      const bf16x8 w = pf[f / 2][f % 2];
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        lp_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[2 * j], w[2 * j + 1]}, ones, lp_run,
                                                 false);
      });
    });
#pragma unroll
    for (int bb = 0; bb < C::NB; ++bb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w = __builtin_bit_cast(u32x4, pf[bb][half]);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          // registers 8*half + 4*q2 .. +3: keys kv0 + 32bb + 16half + 8q2 + 4h + 0..3
          const uint32_t key0 = (uint32_t)(kv0 + 32 * bb + 16 * half + 8 * q2 + 4 * h);
          const u32x4 u = philox4x32_10(u32x4{key0 >> 2, (uint32_t)qrow, (uint32_t)bh,
                                              p.drop_offset},
                                        p.seed_lo, p.seed_hi);
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            const uint32_t lo = u[2 * t2] >= p.drop_threshold ? 0x0000FFFFu : 0u;
            const uint32_t hi = u[2 * t2 + 1] >= p.drop_threshold ? 0xFFFF0000u : 0u;
            w[2 * q2 + t2] &= lo | hi;
          }
        }
        pf[bb][half] = __builtin_bit_cast(bf16x8, w);
      }
    }
  };

  f32x16 s[C::NB];
  bf16x8 pf[C::NB][2];
  const uint32_t lds0 = lds_addr(lds);
  constexpr auto G0 = std::integral_constant<int, 0>{};

  if constexpr (!PINGPONG) {
    // ---- lockstep schedule: every wave runs S, softmax and PV of a tile
    // between two barriers -------------------------------------------------
    // steps: one LDS stage each (KS key tiles, one per key group)
    const int nsteps = PAIR ? g0 : (ntiles + KS - 1) / KS;
    // Paired form: the first key of group g's tile in step t, and whether
    // the group has one (its stage half is zero-filled otherwise).
    auto pair_kv = [&](const int g, const int t) __attribute__((always_inline)) {
      return (g == 0 || t < n_l ? t : ntiles - 1 - (t - n_l)) * C::BK;
    };
    auto pair_has = [&](const int g, const int t) __attribute__((always_inline)) {
      return t < (g == 0 ? g0 : ntiles + n_l - g0);
    };
    // The loads of step t into a stage: KS consecutive tiles, or in the
    // paired form the two groups' tiles (the first half of each wave's
    // loads fills group 0's half of the stage).
    auto load_step = [&](const int t, const int stage) __attribute__((always_inline)) {
      if constexpr (PAIR) {
        static_assert(C::LOADS % 2 == 0, "a wave's loads split evenly between the halves");
        uint8_t* ks = lds + stage * C::STAGE_BYTES;
        uint8_t* vs = ks + C::TILE_BYTES;
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
          const int g = i < C::LOADS / 2 ? 0 : 1;
          const int blk = (WAVES * i + wave) * 1024;
          const bool fetch = g == 0 ? t < g0 : t >= n_l && pair_has(1, t);
          const uint32_t nb = __builtin_amdgcn_readfirstlane(fetch ? valid_bytes : 0u);
          // koff/voff hold the row within the stage, which for group 1's
          // half is BK rows on: the tile start is taken back by BK rows
          // (modulo 2^32; the per-lane sum is the true offset)
          const uint32_t toff = __builtin_amdgcn_readfirstlane(
              (uint32_t)(pair_kv(g, t) - g * C::BK) * row_stride);
          load_lds_16(kbase, nb, ks + blk, koff[i] + toff);
          load_lds_16(vbase, nb, vs + blk, voff[i] + toff);
        }
      } else {
        load_tile(kv_first + t * C::SK, stage);
      }
    };
    // Paired form, group 1 after its last light key tile: the light rows
    // are written out (as in the epilogue below) and the wave takes over
    // the heavy tile's rows with a fresh state.
    auto finish_light = [&]() __attribute__((always_inline)) {
      light_pending = false;
      const float l_tot = halves_sum(l_run);
      const float lp_tot = halves_sum(lp_run + lp_run2);
      const bool valid = qpos < kv_lim && lp_tot > 0.f;
      const float inv = valid ? 1.f / lp_tot : 0.f;
      const float lse_row = valid ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
      if (qrow < N) {
        uint16_t* og = (uint16_t*)p.o + base + (int64_t)qrow * q_ld;
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
        if (h == 0) p.lse[lse_base + (int64_t)qrow * lse_ld] = lse_row;
      }
#pragma unroll
      for (int i = 0; i < C::ND; ++i) o_acc[i] = f32x16{};
      m_ref = kNegInf;
      l_run = 0.f;
      lp_run = 0.f;
      lp_run2 = 0.f;
      qw0 = qw0_heavy;
      qrow = qw0 + l32;
      qwpos = qw0 + off;
      qpos = qrow + off;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[kk] = qf_heavy[PAIR ? kk : 0];
    };
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
      if (st < nsteps) load_step(st, st);

    // One streamed tile, read from LDS stage S (a compile-time constant:
    // the loop below cycles through the NSTAGE instantiations).
    auto step = [&](const int t, auto stage_tag) __attribute__((always_inline)) {
      constexpr int S = decltype(stage_tag)::value;
      // first key of this group's tile
      const int kv0 = PAIR ? pair_kv(kgrp, t) : kv_first + t * C::SK + kgrp * C::BK;
      // Tile t has landed once at most the loads of the tiles issued after
      // it are still in flight; after the barrier every wave's part has
      // landed and every wave is done with tile t - 1, whose stage is
      // refilled.
      const int later = min(NSTAGE - 2, nsteps - 1 - t);  // 0 .. NSTAGE - 2 (uniform)
      if (NSTAGE > 3 && later >= 2) vmem_wait<(NSTAGE > 3 ? 2 : 0) * C::LOADS_PER_TILE>();
      else if (later >= 1) vmem_wait<C::LOADS_PER_TILE>();
      else vmem_wait<0>();
      barrier_no_fence();
      if (t + NSTAGE - 1 < nsteps) load_step(t + NSTAGE - 1, (S + NSTAGE - 1) % NSTAGE);
      // group 1's half of the stage (group 0's during the light steps of
      // the paired form)
      int half = kgrp;
      if constexpr (PAIR) {
        if (t == 0 && light_pending) load_q(qw0_heavy + l32, qf_heavy);
        if (light_pending && t >= n_l) finish_light();
        if (!pair_has(kgrp, t) || skip_tile(kv0)) return;
        if (t < n_l) half = 0;
      } else {
        if (skip_tile(kv0) || (KS == 2 && kv0 >= kv_last)) return;
      }
      uint32_t kbase = lds0 + S * C::STAGE_BYTES + half * C::BK * C::ROW_BYTES;
      asm volatile("" : "+s"(kbase));  // see the ping-pong schedule
      k_issue(G0, kbase, kr[0]);
      if constexpr (BIAS) bias_issue(kv0);
      compute_s(kbase, s, std::integral_constant<int, 1>{});
      softmax(kv0, s, pf, [] {});
      if constexpr (DROP) dropout(kv0, pf);
      v_issue(G0, kbase + C::TILE_BYTES, vr[0]);
      pv(kbase + C::TILE_BYTES, pf, std::false_type{}, 0u);
    };
    for (int t = 0; t < nsteps; t += NSTAGE) {
      step(t, StageTag<0>{});
      if (t + 1 < nsteps) step(t + 1, StageTag<1>{});
      if constexpr (NSTAGE > 2) {
        if (t + 2 < nsteps) step(t + 2, StageTag<2>{});
      }
      if constexpr (NSTAGE > 3) {
        if (t + 3 < nsteps) step(t + 3, StageTag<3>{});
      }
    }
    if constexpr (PAIR) {
      if (light_pending) finish_light();  // group 1 had no heavy key tile
    }
    if constexpr (KS == 2) {
      // Key group 1 hands its running state (numerator, reference maximum,
      // denominators; same lanes, same rows) to group 0 through LDS, and
      // group 0 combines the two partial sums over disjoint key sets against
      // their larger reference, as the block summaries of "FlashAttention"
      // (section "Why a tile can be discarded") combine, then writes the rows.
      constexpr int NV = C::ND * 16 + 3;
      static_assert((WAVES / 2) * NV * 64 * 4 <= C::LDS_BYTES, "exchange fits the ring");
      float* xs = (float*)lds + (wave % (WAVES / 2)) * NV * 64 + lane;
      barrier_no_fence();  // every wave is done reading the ring (all loads have landed)
      if (kgrp == 1) {
#pragma unroll
        for (int i = 0; i < C::ND; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) xs[(i * 16 + r) * 64] = o_acc[i][r];
        xs[(C::ND * 16) * 64] = m_ref;
        xs[(C::ND * 16 + 1) * 64] = l_run;
        xs[(C::ND * 16 + 2) * 64] = lp_run + lp_run2;
      }
      __syncthreads();
      if (kgrp == 1) return;
      const float m1 = xs[(C::ND * 16) * 64];
      const float m = fmaxf(m_ref, m1);
      // -inf - (-inf) is never formed: a reference of -inf weighs 0
      const float a0 = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - m);
      const float a1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - m);
      m_ref = m;
      l_run = l_run * a0 + xs[(C::ND * 16 + 1) * 64] * a1;
      lp_run = (lp_run + lp_run2) * a0 + xs[(C::ND * 16 + 2) * 64] * a1;
      lp_run2 = 0.f;
#pragma unroll
      for (int i = 0; i < C::ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[i][r] = o_acc[i][r] * a0 + xs[(i * 16 + r) * 64] * a1;
    }
  } else {
    // ---- ping-pong schedule ----------------------------------------------
    // The two waves that share a SIMD belong to different groups (waves
    // 0-3 and 4-7; the hardware deals a workgroup's waves to the four SIMDs
    // in turn).  Each wave alternates an MFMA phase t (PV of tile t - 1,
    // then S of tile t) with a softmax phase t (VALU only), and the second
    // group runs one phase behind the first: while one wave of a SIMD keeps
    // the matrix core busy, the other has the vector ALU to itself.  The
    // MFMA phase runs at raised issue priority: otherwise the older of the
    // two waves wins the arbitration whatever it runs, and the matrix core
    // idles whenever that is the VALU wave.  Since phases overlap across the
    // groups, waves do not skip tiles their rows cannot see here: the scores
    // come out masked and the probabilities zero.
    //
    // One workgroup barrier per tile.  Barrier t opens the first group's
    // MFMA phase t and the second group's softmax phase t - 1 (a barrier
    // only counts arrivals, so the groups may arrive from different points
    // of their code); that offset is all that pairs the phases.  Before
    // barrier t each wave waits for its own loads of tile t, so the tile is
    // complete at barrier t.
    //
    // LDS ring of four stages.  Every MFMA phase t issues the loads of tile
    // t + 2 (past the last tile a zero fill, an empty buffer range) into the
    // stage of tile t - 2.  Its last readers are the PV products of the MFMA
    // phases t - 1, which both groups finish before barrier t, and the
    // refill is issued after it.  K of tile t is read in MFMA phases t
    // (after barrier t); V of tile t is read in softmax phases t (after
    // barrier t) and waited for in MFMA phases t + 1, before barrier t + 2,
    // after which its stage is refilled.
    //
    // Fragment reads run ahead of their MFMAs untracked by the compiler, so
    // no control-flow join (where the compiler may copy registers) lies
    // between a read and its wait: each group runs its own straight-line
    // copy of the loop, in which a softmax phase and the MFMA phase that
    // multiplies its V fragments fall in one iteration.
    static_assert(WAVES == 8 && NSTAGE >= 4, "ping-pong needs 8 waves and 4 or more stages");
    constexpr int LA = NSTAGE - 2;  // tiles loaded ahead of the one being multiplied
    const int grp = wave >> 2;
    // Persistent form: the tiles of all this workgroup's query tiles form one
    // stream through the ring; sbase is the stream position of the current
    // query tile's first key tile.
    int sbase = 0;
    auto stage_of = [&](const int t) __attribute__((always_inline)) {
      if constexpr (PERSIST) {
        static_assert(NSTAGE == 4, "stream positions map to stages by their low bits");
        return (uint32_t)((sbase + t) & 3);
      } else {
        return (uint32_t)(NSTAGE == 4 ? (t & 3) : t % NSTAGE);
      }
    };
    auto k_stage = [&](const int t) __attribute__((always_inline)) {
      return lds0 + stage_of(t) * C::STAGE_BYTES;
    };
    auto v_stage = [&](const int t) __attribute__((always_inline)) {
      return lds0 + stage_of(t) * C::STAGE_BYTES + C::TILE_BYTES;
    };
    // Loads of tile u (a zero fill at or past the last tile, so that every
    // wave always has the same number of loads in flight).
    auto load_ahead = [&](const int u) __attribute__((always_inline)) {
      const uint32_t nb = u < ntiles ? valid_bytes : 0u;
      load_tile_n(kv_first + u * C::BK, stage_of(u), __builtin_amdgcn_readfirstlane(nb));
    };
    // Persistent form: a cursor over the stream.  Each call loads the next
    // stream position (the next key tile of the query tile the cursor is in,
    // else the first of the next query tile; past the last one a zero fill),
    // so the loads that run ahead of a query tile's last products bring in
    // the first tiles of the next one.
    const int n_items = PERSIST ? 2 * p.persist : 1;
    auto item_ntiles = [&](const int iqt) __attribute__((always_inline)) {
      const int nk = CAUSAL ? min(Nk, iqt * C::BQ + C::BQ) : Nk;
      return (nk + C::BK - 1) / C::BK;
    };
    auto item_kv = [&](const int ibh) __attribute__((always_inline)) {
      const int ib = ibh / p.H, ihq = ibh - ib * p.H;
      return ((int64_t)ib * p.Hkv + ihq / (p.H / p.Hkv)) * Nk * D;
    };
    int l_item = 0, l_tile = 0, l_nt = ntiles, l_pos = 0;
    int64_t l_kv = kvbase;
    auto load_next = [&]() __attribute__((always_inline)) {
      const bool live = l_item < n_items;
      uint8_t* ks = lds + (l_pos & 3) * C::STAGE_BYTES;
      uint8_t* vs = ks + C::TILE_BYTES;
      const uint32_t nb = __builtin_amdgcn_readfirstlane(live ? valid_bytes : 0u);
      const uint32_t tile_off =
          __builtin_amdgcn_readfirstlane((uint32_t)(l_tile * C::BK) * row_stride);
      const void* kb = (const uint16_t*)p.k + l_kv;
      const void* vb = (const uint16_t*)p.v + l_kv;
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const int blk = (WAVES * i + wave) * 1024;
        load_lds_16(kb, nb, ks + blk, koff[i] + tile_off);
        load_lds_16(vb, nb, vs + blk, voff[i] + tile_off);
      }
      ++l_pos;
      if (live && ++l_tile == l_nt) {
        ++l_item;
        l_tile = 0;
        if (l_item < n_items) {
          int ibh, iqt;
          item_of(l_item, ibh, iqt);
          l_nt = item_ntiles(iqt);
          l_kv = item_kv(ibh);
        }
      }
    };
    auto issue_loads = [&](const int t) __attribute__((always_inline)) {
      if constexpr (PERSIST) load_next();
      else load_ahead(t + LA);
    };
    if constexpr (PERSIST) {
      load_next();
      load_next();
    } else {
#pragma unroll
      for (int u = 0; u < LA; ++u) load_ahead(u);
      vmem_wait<(LA - 1) * C::LOADS_PER_TILE>();  // tile 0
    }
    // Softmax phase t.  The V fragments of tile t are read at its end, where
    // this wave's SIMD has LDS bandwidth to spare, so the MFMA phase that
    // multiplies them reads only K.  (Issued after the exponentials, when
    // the score registers are free: issued earlier they cost 15 registers
    // more at the peak and ran no faster.)
    auto softmax_phase = [&](const int t) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(0);
      softmax(kv_first + t * C::BK, s, pf, [] {});
      v_issue_range(v_stage(t), G0, std::integral_constant<int, VG>{});
    };
    constexpr auto K4 = std::integral_constant<int, 4>{};
    constexpr auto K0 = std::integral_constant<int, 0>{};
    constexpr auto PRE1 = std::integral_constant<int, 1>{};
    constexpr auto PREALL = std::integral_constant<int, KG>{};
    // MFMA phase 0 < t < ntiles.  PV of tile t - 1 starts right away (its
    // V fragments are in flight or in registers); the tile loads and the K
    // groups of tile t are issued behind its MFMA groups, one K group each,
    // so that all of K is in registers when the first product starts.
    auto mfma_phase = [&](const int t) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);
      const uint32_t kb = k_stage(t);
      k_issue(G0, kb, kr[0]);
      pv_pre(pf, K4, K4, [&](auto gc) __attribute__((always_inline)) {
        constexpr int g = decltype(gc)::value;
        if constexpr (g == 0) issue_loads(t);
        if constexpr (g + 1 < KG && g + 1 < VG)
          k_issue(std::integral_constant<int, g + 1>{}, kb, kr[g + 1]);
      });
      compute_s(kb, s, PREALL);
    };
    auto run = [&](auto grp_tag) __attribute__((always_inline)) {
      constexpr bool first = decltype(grp_tag)::value == 0;
      barrier_no_fence();  // barrier 0
      if (ntiles == 0) return;
      // MFMA phase 0: S of tile 0 only
      __builtin_amdgcn_s_setprio(1);
      issue_loads(0);
      k_issue(G0, k_stage(0), kr[0]);
      compute_s(k_stage(0), s, PRE1);
      for (int t = 1; t < ntiles; ++t) {
        if constexpr (first) softmax_phase(t - 1);
        vmem_wait<(LA - 1) * C::LOADS_PER_TILE>();  // this wave's loads of tile t
        barrier_no_fence();              // barrier t
        if constexpr (!first) softmax_phase(t - 1);
        mfma_phase(t);
      }
      if constexpr (first) softmax_phase(ntiles - 1);
      barrier_no_fence();  // barrier ntiles
      if constexpr (!first) softmax_phase(ntiles - 1);
      // last MFMA phase: PV of the last tile only
      __builtin_amdgcn_s_setprio(1);
      issue_loads(ntiles);
      pv_pre(pf, K0, K0, [](auto) {});
    };
    // Persistent form.  Query tile X's own loop is the one above, with these
    // differences.  Its first key tiles were loaded by the previous query
    // tile's last phases (the loads that would otherwise be zero fills);
    // its Q rows are loaded at its start (buffer loads into the Q fragments;
    // rows past N read zeros), and the epilogue of X runs right after its
    // last product, then the state is reset.  Stage reuse across the
    // boundary is the same as within a query tile: the last phase of X and
    // the first phase of X + 1 together are one phase of the stream.
    //
    // Before barrier 0 only key tile 0 must have landed.  The loads issued
    // after it are its successors in the stream (tile 1, and for X > 0
    // tile 2) and the Q rows; loads complete in issue order, so while tile
    // 0 is in flight all of those are too, and waiting until no more than
    // their number are outstanding waits for tile 0 and nothing later
    // (stores in between only make the wait stricter).
    auto epilogue_dense = [&](const int ebh, const int eq0) __attribute__((always_inline)) {
      const float l_tot = halves_sum(l_run);
      const float lp_tot = halves_sum(lp_run + lp_run2);
      const int row = eq0 + 32 * wave + l32;
      const bool valid = row < N && lp_tot > 0.f;
      const float inv = valid ? 1.f / lp_tot : 0.f;
      const float lse_row = valid ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
      if (row < N) {
        uint16_t* og = (uint16_t*)p.o + ((int64_t)ebh * N + row) * D;
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
        if (h == 0) p.lse[(int64_t)ebh * N + row] = lse_row;
      }
#pragma unroll
      for (int i = 0; i < C::ND; ++i) o_acc[i] = f32x16{};
      m_ref = kNegInf;
      l_run = 0.f;
      lp_run = 0.f;
      lp_run2 = 0.f;
    };
    auto run_p = [&](auto grp_tag) __attribute__((always_inline)) {
      constexpr bool first = decltype(grp_tag)::value == 0;
      for (int it = 0;; ++it) {
        {
          const void* qn = (const uint16_t*)p.q + (int64_t)bh * N * D;
          const uint32_t qoff = (uint32_t)(qrow * C::ROW_BYTES + 16 * h);
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = __builtin_bit_cast(bf16x8, load_ranged_16(qn, (uint32_t)N * C::ROW_BYTES,
                                                               qoff + 32 * kk));
        }
        constexpr int QL = D / 16;  // Q loads per wave
        if (it == 0) vmem_wait<C::LOADS_PER_TILE + QL>();  // tile 0 (tile 1, Q in flight)
        else vmem_wait<2 * C::LOADS_PER_TILE + QL>();      // tile 0 (tiles 1, 2, Q in flight)
        barrier_no_fence();  // barrier 0
        __builtin_amdgcn_s_setprio(1);
        if (it == 0) load_next();
        k_issue(G0, k_stage(0), kr[0]);
        compute_s(k_stage(0), s, PRE1);
        for (int t = 1; t < ntiles; ++t) {
          if constexpr (first) softmax_phase(t - 1);
          vmem_wait<(LA - 1) * C::LOADS_PER_TILE>();  // this wave's loads of tile t
          barrier_no_fence();              // barrier t
          if constexpr (!first) softmax_phase(t - 1);
          mfma_phase(t);
        }
        if constexpr (first) softmax_phase(ntiles - 1);
        barrier_no_fence();  // barrier ntiles
        if constexpr (!first) softmax_phase(ntiles - 1);
        __builtin_amdgcn_s_setprio(1);
        issue_loads(ntiles);
        pv_pre(pf, K0, K0, [](auto) {});
        if (it + 1 >= n_items) break;
        epilogue_dense(bh, q0);
        int nbh, nqt;
        item_of(it + 1, nbh, nqt);
        sbase += ntiles;
        bh = nbh;
        q0 = nqt * C::BQ;
        ntiles = item_ntiles(nqt);
        qw0 = q0 + 32 * wave;
        qrow = qw0 + l32;
        qwpos = qw0;
        qpos = qrow;
      }
    };
    if constexpr (PERSIST) {
      if (grp == 0) run_p(std::integral_constant<int, 0>{});
      else run_p(std::integral_constant<int, 1>{});
      // the last query tile's epilogue below writes through these
      base = (int64_t)bh * N * D;
      lse_base = (int64_t)bh * N;
    } else {
      if (grp == 0) run(std::integral_constant<int, 0>{});
      else run(std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_setprio(0);
    // No load into LDS may still be in flight when the workgroup ends.
    vmem_wait<0>();
  }

  // ---- epilogue: o = a / l, LSE = ln(2) * (m + log2 l) ---------------------
  // Rows at or beyond the key length are padding (o = 0, LSE = -inf); so is
  // a row that saw no key in this workgroup's range.
  const float l_tot = halves_sum(l_run);
  const float lp_tot = halves_sum(lp_run + lp_run2);
  const bool valid = qpos < kv_lim && lp_tot > 0.f;
  const float inv = valid ? (DROP ? p.keep_scale : 1.f) / lp_tot : 0.f;
  const float lse_row = valid ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
  if (qrow < N) {
    if (p.o_part) {
      // one key range of several: fp32 partial result and its log-sum-exp
      const int64_t prow = ((int64_t)split * BH + bh) * N + qrow;
      float* og = p.o_part + prow * D;
#pragma unroll
      for (int db = 0; db < C::ND; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          f32x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = valid ? o_acc[db][4 * g + e] * inv : 0.f;
          *(f32x4*)(og + d0) = y;
        }
      }
      if (h == 0) p.lse_part[prow] = lse_row;
    } else {
      uint16_t* og = (uint16_t*)p.o + base + (int64_t)qrow * q_ld;
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
      if (h == 0) p.lse[lse_base + (int64_t)qrow * lse_ld] = lse_row;
    }
  }
}

template <int D, bool CAUSAL, int WAVES, int NSTAGE, bool PINGPONG, bool DROP = false,
          bool BIAS = false, bool PERSIST = false, int BKX = 0, int KS = 1, bool PAIR = false>
hipError_t launch_cfg(FwdParams p, hipStream_t stream) {
  using C = Bf16Cfg<D, WAVES, NSTAGE, BKX, KS>;
  p.n_qtiles = (p.N + C::BQ - 1) / C::BQ;
  // paired form: one workgroup per pair of query tiles
  const int64_t items = PAIR ? (int64_t)((p.n_qtiles + 1) / 2) * p.B * p.H
                             : (int64_t)p.n_qtiles * p.B * p.H * p.splits;
  // persistent: items / 2 units, p.persist per workgroup
  const dim3 grid((unsigned)(PERSIST ? items / 2 / p.persist : items));
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, WAVES, NSTAGE, PINGPONG, DROP, BIAS, PERSIST, BKX, KS, PAIR>),
                     grid, dim3(64 * WAVES), 0, stream, p);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; 0 if unknown).
int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

// Units (pairs of 256-row query tiles) per workgroup of the persistent
// launch, or 0 where it does not apply: it needs the dense layout with as
// many keys as queries and no per-sequence lengths (so every row sits at its
// own key position and every query tile sees at least two key tiles), one
// key range, a non-negative scale, and a number of units that the compute
// units divide exactly (the static assignment is then balanced; otherwise
// the hardware dispatcher's dynamic order balances better).
int persist_units(const FwdParams& p) {
  if (p.key_len || p.cu_q || p.splits != 1 || p.Nk != p.N || p.q_sign || p.o_part || p.drop ||
      p.bias || p.N < 256)
    return 0;
  const int64_t nq = (p.N + 255) / 256;
  if (nq % 2) return 0;
  const int64_t units = (int64_t)p.B * p.H * nq / 2;
  const int cus = device_cus();
  if (cus <= 0 || cus % 8 || units % cus) return 0;
  return (int)(units / cus);
}

template <int D, bool CAUSAL>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  // 256-row tiles (8 waves, one workgroup per CU, ping-pong schedule) when
  // the query tiles are full and there are enough workgroups to fill the
  // chip twice over; 128-row tiles (4 waves, two workgroups per CU, lockstep
  // schedule, which skips rows past the end) otherwise.
  if (p.drop) return launch_cfg<D, CAUSAL, 4, 2, false, true>(p, stream);
  if (p.bias) return launch_cfg<D, CAUSAL, 4, 2, false, false, true>(p, stream);
  const int64_t big_tiles = (int64_t)p.B * p.H * ((p.N + 255) / 256) * p.splits;
  // At d = 64 with per-sequence key lengths the lockstep schedule is the
  // faster one: the ping-pong computes masked tiles and padding rows in
  // full, and at d = 64 their softmax work dominates (8 x 16 x 4096 with
  // ragged lengths: 327 -> 295 us); at d = 128 it is not.
  const bool ragged64 = D == 64 && p.key_len;
  if (p.N >= 256 && big_tiles >= 512 && !ragged64) {
    const int units = persist_units(p);
    if (units > 0) {
      FwdParams pp = p;
      pp.persist = units;
      return launch_cfg<D, CAUSAL, 8, kPingPongStages, true, false, false, true>(pp, stream);
    }
    return launch_cfg<D, CAUSAL, 8, kPingPongStages, true>(p, stream);
  }
  // d = 64 with per-sequence lengths: 64-key tiles, three workgroups per CU
  // (more waves to hide the softmax's dependency stalls: 8 x 16 x 4096 with
  // ragged lengths 349 -> 330 us; without lengths, on the 32-head N = 2048
  // causal workload, 128-key tiles at two per CU stay faster, 34.5 vs 37 us)
  if (ragged64) return launch_cfg<D, CAUSAL, 4, 2, false, false, false, false, 64>(p, stream);
  // A causal grid of 128-row tiles that the device holds at once (two per
  // CU) is as slow as its heaviest tile, which sees the most keys: there each
  // workgroup gets eight waves in two groups over alternate key tiles, so
  // the heaviest tiles take half as long and the light ones fill in behind.
  if constexpr (CAUSAL) {
    const int cus = device_cus();
    if (!p.key_len && !p.cu_q && p.splits == 1 && cus > 0 &&
        (int64_t)p.B * p.H * ((p.N + 127) / 128) <= 2 * (int64_t)cus) {
      // When the pairs of query tiles (j, n - 1 - j) fill the device, one
      // workgroup per pair: each CU then runs one workgroup of equal work
      // instead of a heavy and a light one in turn, and pays one start and
      // one drain (about 2 us each) instead of two (32 x 2048 at d = 64:
      // 32.0 -> 29.8 us; 64 x 1024: 20.9 -> 18.5).  With fewer pairs the
      // unpaired tiles spread wider (32 x 1024, 128 pairs: 14.5 vs 18.0 us).
      if (p.Nk == p.N && !p.end_aligned && !p.o_part &&
          (int64_t)p.B * p.H * (((p.N + 127) / 128 + 1) / 2) >= (int64_t)cus)
        return launch_cfg<D, CAUSAL, 8, 2, false, false, false, false, 0, 2, true>(p, stream);
      return launch_cfg<D, CAUSAL, 8, 2, false, false, false, false, 0, 2>(p, stream);
    }
  }
  return launch_cfg<D, CAUSAL, 4, 2, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
  return causal ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
}

}  // namespace fa
