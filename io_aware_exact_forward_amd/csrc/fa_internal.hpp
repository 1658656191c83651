// Internal interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a forward kernel needs, passed by value as one kernel argument.
struct FwdParams {
  const void* q;           // [B, H, N, d]
  const void* k;           // [B, H, Nk, d]
  const void* v;           // [B, H, Nk, d]
  void* o;                 // [B, H, N, d] (unused when o_part is set)
  float* lse;              // [B, H, N]    (unused when o_part is set)
  const int32_t* key_len;  // device [B] or nullptr
  int B, H, N;             // N: query rows (packed batches: the longest sequence)
  int Hkv;                 // key/value heads; query head h reads head h / (H / Hkv)
  int Nk;                  // key rows (dense layout)
  const int32_t* cu_q;     // packed batch: device [B + 1] query row offsets, or nullptr
  const int32_t* cu_k;     // packed batch: device [B + 1] key row offsets
  int end_aligned;         // 0: query row i sits at key position i; 1: at i + L_b - N
  int n_qtiles;            // ceil(N / query-tile rows)
  int splits;              // key ranges per (batch, head, query tile), >= 1
  int split_keys;          // keys per range, a multiple of 128
  float* o_part;           // [splits, B, H, N, d] fp32 partial outputs, or nullptr
  float* lse_part;         // [splits, B, H, N] their log-sum-exp
  const float* bias;       // additive mask, fp32, or nullptr (lockstep schedule)
  int64_t bias_sb, bias_sh, bias_ld;  // its batch, head and row strides (elements)
  int drop;                // dropout on the probabilities (lockstep schedule)
  uint32_t drop_threshold; // a weight is dropped when its draw is below this
  uint32_t seed_lo, seed_hi, drop_offset;  // Philox key and counter word 3
  float keep_scale;        // 1 / (1 - p)
  int persist;             // > 0: persistent launch, this many units (query-tile pairs) per workgroup
  float c;                 // |scale| * log2(e): scores enter exp2 in log2 units
  uint32_t q_sign;         // sign bits xor-ed into Q when scale < 0 (0 otherwise)
};

// Merge of split partial results into the final output.
struct MergeParams {
  const float* o_part;     // [splits, rows, d]
  const float* lse_part;   // [splits, rows]
  void* o;                 // [rows, d] in the input dtype
  float* lse;              // [rows]
  int64_t rows;            // B * H * N
  int splits;
  // balanced decode shares (cum non-null): row bh's partials sit at slots
  // 4 (w + bh) + wave ([4 (P + B*H), d] and [4 (P + B*H)]) for the shares w
  // that touch it
  const int64_t* cum;      // [B + 1] units (64 keys of one row) before sequence b; cum[B] = total
  const int32_t* key_len;  // device [B] or nullptr
  int B, H, Nk;
  int workgroups;          // P: shares (workgroups) of the decode kernel
};

// Parameters of the materialised (three-pass) path's softmax pass.
struct NaiveSoftmaxParams {
  const void* s;           // [B*H, N, N] scores already multiplied by scale
  void* p;                 // [B*H, N, N] probabilities (same dtype as s)
  float* lse;              // [B*H, N]
  const int32_t* key_len;  // device [B] or nullptr
  int B, H, N;
  int causal;
};

// Everything the two backward kernels need.
struct BwdParams {
  const void* q;           // [B, H, N, d] bf16 (packed: [T, H, d])
  const void* k;           // [B, Hkv, Nk, d] (packed: [Tk, Hkv, d])
  const void* v;
  const void* o;           // forward output, layout of q
  const void* dout;        // upstream gradient dO, layout of q
  const float* lse;        // [B, H, N] forward log-sum-exp (natural log); packed [T, H]
  void* dq;                // bf16 outputs in the layouts of q, k, v
  void* dk;
  void* dv;
  float* dvec;             // workspace in the layout of lse: D_i = dO_i . O_i
  const int32_t* key_len;  // device [B] or nullptr (dense only)
  int B, H, N;             // N: query rows per sequence (dense)
  int Hkv, Nk;             // key/value heads (H % Hkv == 0); keys per sequence (dense)
  const int32_t* cu_q;     // packed batch: sequence b at rows cu_q[b] .. cu_q[b+1]-1, else nullptr
  const int32_t* cu_k;
  int end_aligned;         // query row i at key position i + L_b - N_b (else i)
  int n_qtiles;            // ceil(max N / 128): workgroups per (b, h) of the dQ kernel
  int n_ktiles;            // ceil(max Nk / 128): workgroups per (b, hkv) of the dK/dV kernel
  float scale;             // signed
  float c2;                // scale * log2(e), signed
  // dropout of the forward (dense, Hkv == H): keep mask regenerated from the
  // same Philox4x32-10 stream, dP masked and scaled by keep_scale
  int drop;
  uint32_t drop_threshold;  // keep iff draw >= threshold (floor(p * 2^32))
  uint32_t seed_lo, seed_hi, drop_offset;
  float keep_scale;         // 1 / (1 - p)
  // additive mask of the forward (dense, Hkv == H): fp32, element (b, h, i, j)
  // at bias[b * bias_sb + h * bias_sh + i * bias_ld + j], or nullptr
  const float* bias;
  int64_t bias_sb, bias_sh, bias_ld;
};

// Row passes of the stored-state (materialised) backward.
struct NaiveBwdParams {
  void* sp;                // [B*H, N, N] bf16: S on entry, P after the first pass
  void* dpds;              // [B*H, N, N] bf16: dP on entry, dS after the second pass
  const float* lse;        // [B*H, N]
  const int32_t* key_len;  // device [B] or nullptr
  int B, H, N;
  int causal;
};

// Query rows per workgroup of the fused kernels.
constexpr int kQueryTile = 128;

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream);
// One query row per (batch, head) (Nq = 1, rows at the end of the keys), bf16.
hipError_t launch_decode_bf16(const FwdParams& p, int d, hipStream_t stream);
// The same with the visible keys of all rows cut into `shares` equal shares,
// one per workgroup; writes cum[0..B] (see MergeParams) and partials for
// every row, which the merge completes.
hipError_t launch_decode_balanced_bf16(const FwdParams& p, int d, int shares, int64_t* cum,
                                       hipStream_t stream);
hipError_t launch_naive_softmax(const NaiveSoftmaxParams& p, bool bf16, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int d, bool bf16, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_naive_bwd_p(const NaiveBwdParams& p, hipStream_t stream);
hipError_t launch_naive_bwd_ds(const NaiveBwdParams& p, hipStream_t stream);

}  // namespace fa
