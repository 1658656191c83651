// C ABI of the attention forward library: argument validation, kernel
// selection and launch.  Declared and documented in include/fa_mi355x.h.
#include "fa_mi355x.h"

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <climits>
#include <cmath>
#include <algorithm>
#include <cstdint>
#include <limits>
#include <mutex>

#include "fa_internal.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 62;

struct Shape {
  int64_t elems = 0;  // B*H*N*d
  int64_t rows = 0;   // B*H*N
  int esz = 0;        // bytes per q/k/v/o element
};

bool is_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(nb) && b0 < a0 + static_cast<uintptr_t>(na);
}

// Checks that do not look at pointers.  Sets *empty when there is no work.
int check_scalars(int B, int H, int N, int d, float scale, int dtype, Shape* s, bool* empty) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  const double c = std::fabs(static_cast<double>(scale)) * 1.4426950408889634;
  if (!std::isfinite(static_cast<float>(c))) return FA_ERR_SCALE;
  *empty = (B == 0 || H == 0 || N == 0);
  if (*empty) return FA_OK;
  const int64_t bh = int64_t(B) * H;
  if (bh > INT_MAX) return FA_ERR_SHAPE;
  const int64_t rows = bh * N;
  if (rows > kMaxElems / d) return FA_ERR_SHAPE;
  const int64_t qtiles = (int64_t(N) + fa::kQueryTile - 1) / fa::kQueryTile;
  if (qtiles * bh > INT_MAX) return FA_ERR_SHAPE;
  // byte offsets within one (batch, head) slice are 32-bit in the kernels
  if (int64_t(N) * d * (dtype == FA_DTYPE_BF16 ? 2 : 4) > INT_MAX) return FA_ERR_SHAPE;
  s->rows = rows;
  s->elems = rows * d;
  s->esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
  return FA_OK;
}

int check_pointers(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int32_t* key_len, int B, const Shape& s) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(o, 16))
    return FA_ERR_ALIGN;
  if (!is_aligned(lse, 4) || (key_len && !is_aligned(key_len, 4))) return FA_ERR_ALIGN;
  const int64_t nb = s.elems * s.esz;
  const int64_t nl = s.rows * 4;
  const int64_t nk = key_len ? int64_t(B) * 4 : 0;
  for (const void* in : {q, k, v}) {
    if (overlaps(o, nb, in, nb) || overlaps(lse, nl, in, nb)) return FA_ERR_ALIAS;
  }
  if (overlaps(o, nb, lse, nl) || overlaps(o, nb, key_len, nk) || overlaps(lse, nl, key_len, nk))
    return FA_ERR_ALIAS;
  return FA_OK;
}

fa::FwdParams make_params(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, float scale, const int32_t* key_len, int dtype) {
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.key_len = key_len;
  p.B = B;
  p.H = H;
  p.N = N;
  p.Nk = N;
  p.Hkv = H;
  p.cu_q = nullptr;
  p.cu_k = nullptr;
  p.end_aligned = 0;
  p.n_qtiles = (N + fa::kQueryTile - 1) / fa::kQueryTile;
  p.splits = 1;
  p.split_keys = static_cast<int>(std::min<int64_t>((int64_t(N) + 127) / 128 * 128, INT_MAX - 127));
  p.o_part = nullptr;
  p.lse_part = nullptr;
  // exp(x) = exp2(x * log2 e): the kernels keep scores in log2 units.  c is
  // kept >= the smallest normal float so that a masked score (-inf) times c
  // is -inf, never NaN; for scale = 0 that changes no exp2 result, since
  // |s| * FLT_MIN is far below 2^-24 for any finite score s.
  p.c = std::max(static_cast<float>(std::fabs(static_cast<double>(scale)) * 1.4426950408889634),
                 std::numeric_limits<float>::min());
  // A negative scale is applied by negating Q (exact) and using |scale|.
  p.q_sign = std::signbit(scale) && scale != 0.f
                 ? (dtype == FA_DTYPE_BF16 ? 0x80008000u : 0x80000000u)
                 : 0u;
  return p;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- split-KV -----------------------------------------------------------------

constexpr int kMaxSplits = 65536;
constexpr int kSplitBlock = 128;  // keys: ranges are whole blocks of this size

struct SplitShape {
  int64_t bh = 0;
  int64_t rows = 0;      // B*H*Nq
  int64_t kv_elems = 0;  // B*H*Nk*d
  int splits = 1;        // ranges actually used
  int split_keys = kSplitBlock;
  // decode step split into balanced shares of the visible keys
  bool balanced = false;
  int workgroups = 0;    // shares
  int B = 0;
};

// Shares of a balanced decode step, one per 4-wave workgroup: two per CU
// (the decode kernel's register use allows two at d = 128), all resident at
// once.
constexpr int kDecodeShares = 512;
constexpr int kDecodeWaves = 4;  // partials per share and row

// Ranges are whole 128-key blocks.  With num_splits = 0: enough ranges that
// 128-row query tiles times ranges reach 512 workgroups (two per CU).
void plan_split(int B, int H, int Hkv, int Nq, int Nk, int num_splits, SplitShape* sp) {
  const int64_t kblocks = (int64_t(Nk) + kSplitBlock - 1) / kSplitBlock;
  if (kblocks == 0) {
    sp->splits = 1;
    sp->split_keys = kSplitBlock;
    return;
  }
  int64_t want = num_splits;
  if (want == 0) {
    // workgroups per range: one per query tile and head; a decode step with
    // grouped heads runs one query tile per key/value head (grouped_decode)
    const bool grouped = Nq == 1 && Hkv > 0 && Hkv < H;
    const int64_t tiles = grouped ? int64_t(B) * Hkv
                                  : int64_t(B) * H *
                                        ((int64_t(Nq) + fa::kQueryTile - 1) / fa::kQueryTile);
    want = tiles > 0 ? (512 + tiles - 1) / tiles : 1;
  }
  want = std::max<int64_t>(1, std::min<int64_t>(want, kblocks));
  const int64_t per = (kblocks + want - 1) / want;  // blocks per range
  sp->splits = static_cast<int>((kblocks + per - 1) / per);
  sp->split_keys = static_cast<int>(per * kSplitBlock);
}

int check_split_scalars(int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int dtype,
                        int num_splits, SplitShape* sp, bool* empty) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || num_splits < 0 || num_splits > kMaxSplits)
    return FA_ERR_SHAPE;
  if (Hkv < 1 || (H > 0 && H % Hkv != 0)) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  const double c = std::fabs(static_cast<double>(scale)) * 1.4426950408889634;
  if (!std::isfinite(static_cast<float>(c))) return FA_ERR_SCALE;
  *empty = (B == 0 || H == 0 || Nq == 0);
  if (*empty) return FA_OK;
  const int64_t bh = int64_t(B) * H;
  if (bh > INT_MAX) return FA_ERR_SHAPE;
  if (bh * Nq > kMaxElems / d || bh * Nk > kMaxElems / d) return FA_ERR_SHAPE;
  // byte offsets within one (batch, head) slice are 32-bit in the kernels
  if (int64_t(Nq) * d * 2 > INT_MAX || int64_t(Nk) * d * 2 > INT_MAX) return FA_ERR_SHAPE;
  plan_split(B, H, Hkv, Nq, Nk, num_splits, sp);
  // A decode step (one query row, a key/value head per query head) that the
  // automatic plan would split: the visible keys of all rows are instead cut
  // into equal shares on the device, whatever the per-sequence lengths, so no
  // workgroup is left with a long sequence's range while the rest idle.
  if (num_splits == 0 && Nq == 1 && Hkv == H && sp->splits > 1) {
    const int64_t units = bh * ((int64_t(Nk) + 63) / 64);
    sp->balanced = true;
    sp->workgroups = static_cast<int>(std::min<int64_t>(kDecodeShares, units));
    sp->splits = 1;
  }
  const int64_t qtiles = (int64_t(Nq) + fa::kQueryTile - 1) / fa::kQueryTile;
  if (qtiles * bh * sp->splits > INT_MAX) return FA_ERR_SHAPE;
  sp->bh = bh;
  sp->B = B;
  sp->rows = bh * Nq;
  sp->kv_elems = int64_t(B) * Hkv * Nk * d;
  return FA_OK;
}

// Partial results: [splits, rows] for key ranges, 4 (P + B*H) slots for
// balanced decode shares (one per wave of each share and row).
size_t split_slots(const SplitShape& sp) {
  return sp.balanced ? kDecodeWaves * (size_t(sp.workgroups) + size_t(sp.rows))
                     : size_t(sp.splits) * size_t(sp.rows);
}

size_t split_part_bytes(const SplitShape& sp, int d) {
  return round256(split_slots(sp) * size_t(d) * sizeof(float));
}

size_t split_lse_bytes(const SplitShape& sp) { return round256(split_slots(sp) * sizeof(float)); }

size_t split_workspace(const SplitShape& sp, int d) {
  if (sp.balanced)  // partials, their LSE, then cum [B + 1] (int64)
    return split_part_bytes(sp, d) + split_lse_bytes(sp) +
           round256((size_t(sp.B) + 1) * sizeof(int64_t));
  if (sp.splits <= 1) return 0;
  return split_part_bytes(sp, d) + split_lse_bytes(sp);
}

// One rocBLAS handle per device for the materialised path's two products.
std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};

}  // namespace

extern "C" int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal,
                          const int32_t* key_len_mask, int dtype, void* stream) {
  Shape s;
  bool empty = false;
  int st = check_scalars(B, H, N, d, scale, dtype, &s, &empty);
  if (st != FA_OK || empty) return st;
  st = check_pointers(q, k, v, o, lse, key_len_mask, B, s);
  if (st != FA_OK) return st;
  const fa::FwdParams p = make_params(q, k, v, o, lse, B, H, N, scale, key_len_mask, dtype);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(p, d, causal != 0, hs)
                                              : fa::launch_fwd_f32(p, d, causal != 0, hs);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" size_t fa_naive_workspace_bytes(int B, int H, int N, int dtype) {
  Shape s;
  bool empty = false;
  if (check_scalars(B, H, N, 64, 1.f, dtype, &s, &empty) != FA_OK || empty) return 0;
  const size_t esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
  const size_t mat = size_t(B) * size_t(H) * size_t(N) * size_t(N) * esz;
  return 2 * round256(mat);
}

extern "C" int fa_naive_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, int d, float scale, int causal,
                                const int32_t* key_len_mask, int dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Shape s;
  bool empty = false;
  int st = check_scalars(B, H, N, d, scale, dtype, &s, &empty);
  if (st != FA_OK || empty) return st;
  st = check_pointers(q, k, v, o, lse, key_len_mask, B, s);
  if (st != FA_OK) return st;
  const size_t need = fa_naive_workspace_bytes(B, H, N, dtype);
  if (!workspace || workspace_bytes < need || !is_aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  {
    const int64_t nb = s.elems * s.esz, nw = static_cast<int64_t>(need);
    if (overlaps(workspace, nw, q, nb) || overlaps(workspace, nw, k, nb) ||
        overlaps(workspace, nw, v, nb) || overlaps(workspace, nw, o, nb) ||
        overlaps(workspace, nw, lse, s.rows * 4) ||
        overlaps(workspace, nw, key_len_mask, key_len_mask ? int64_t(B) * 4 : 0))
      return FA_ERR_ALIAS;
  }
  if (int64_t(N) * N > (int64_t(1) << 62) / (int64_t(B) * H)) return FA_ERR_SHAPE;

  const bool bf16 = dtype == FA_DTYPE_BF16;
  const size_t mat = need / 2;
  void* smat = workspace;
  void* pmat = static_cast<char*>(workspace) + mat;
  hipStream_t hs = static_cast<hipStream_t>(stream);

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_blas_mu);
  if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
    g_blas[dev] = nullptr;
    return FA_ERR_HIP;
  }
  rocblas_handle hb = g_blas[dev];
  if (rocblas_set_stream(hb, hs) != rocblas_status_success) return FA_ERR_HIP;
  const rocblas_datatype t = bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const float alpha_s = scale, one = 1.f, zero = 0.f;
  const int bh = B * H;
  const rocblas_stride snd = int64_t(N) * d, snn = int64_t(N) * N;

  // Pass 1: S = scale * Q K^T for every (b, h).  Column-major view: the
  // row-major [N, N] S is S^T = K Q^T with K^T, Q^T stored as [d, N].
  rocblas_status bs = rocblas_gemm_strided_batched_ex(
      hb, rocblas_operation_transpose, rocblas_operation_none, N, N, d, &alpha_s, k, t, d, snd,
      q, t, d, snd, &zero, smat, t, N, snn, smat, t, N, snn, bh, rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  if (bs != rocblas_status_success) return FA_ERR_HIP;

  // Pass 2: P = softmax(S + M) row by row, plus LSE.
  fa::NaiveSoftmaxParams sp{};
  sp.s = smat;
  sp.p = pmat;
  sp.lse = lse;
  sp.key_len = key_len_mask;
  sp.B = B;
  sp.H = H;
  sp.N = N;
  sp.causal = causal != 0;
  if (fa::launch_naive_softmax(sp, bf16, hs) != hipSuccess) return FA_ERR_HIP;

  // Pass 3: O = P V.  Column-major: O^T [d, N] = V^T [d, N] * P^T [N, N].
  bs = rocblas_gemm_strided_batched_ex(
      hb, rocblas_operation_none, rocblas_operation_none, d, N, N, &one, v, t, d, snd, pmat, t, N,
      snn, &zero, o, t, d, snd, o, t, d, snd, bh, rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  if (bs != rocblas_status_success) return FA_ERR_HIP;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" size_t fa_split_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  // The automatic range count of a decode step depends on the number of
  // key/value heads: the largest over every Hkv that divides H.
  size_t most = 0;
  for (int hkv = 1; hkv <= std::max(H, 1); ++hkv) {
    if (H > 0 && H % hkv) continue;
    if (Nq != 1 && hkv > 1) break;  // only decode depends on it
    SplitShape sp;
    bool empty = false;
    if (check_split_scalars(B, H, hkv, Nq, Nk, d, 1.f, FA_DTYPE_BF16, num_splits, &sp,
                            &empty) != FA_OK ||
        empty)
      return 0;
    most = std::max(most, split_workspace(sp, d));
  }
  return most;
}

// Scratch of fa_forward_split_noalloc: the key ranges' fp32 partial results.
// Every device the library runs on holds its own copy until the process
// ends.  In host code the name is only a stand-in for the device array:
// host code uses the device address scratch_address() returns.
static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch[64] = {};  // device address of scratch, per device

// The current device's address of scratch, looked up once per device (with
// that device current) and kept.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

// fa_forward_split with the partial results in the caller's workspace, or
// (use_scratch) in the library's scratch, whose size bounds the problem.
int forward_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Hkv, int Nq, int Nk, int d, float scale, int causal,
                  const int32_t* key_len_mask, int dtype, int num_splits, void* workspace,
                  size_t workspace_bytes, bool use_scratch, void* stream) {
  SplitShape sp;
  bool empty = false;
  int st = check_split_scalars(B, H, Hkv, Nq, Nk, d, scale, dtype, num_splits, &sp, &empty);
  if (st != FA_OK || empty) return st;
  if (use_scratch && split_workspace(sp, d) > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  // an empty cache (Nk = 0) is never read: k and v may then be NULL
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return FA_ERR_NULL;
  if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(o, 16))
    return FA_ERR_ALIGN;
  if (!is_aligned(lse, 4) || (key_len_mask && !is_aligned(key_len_mask, 4))) return FA_ERR_ALIGN;
  const int64_t nq = sp.rows * d * 2, nkv = sp.kv_elems * 2, nl = sp.rows * 4;
  const int64_t nkl = key_len_mask ? int64_t(B) * 4 : 0;
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
      overlaps(o, nq, lse, nl) || overlaps(o, nq, key_len_mask, nkl) ||
      overlaps(lse, nl, key_len_mask, nkl))
    return FA_ERR_ALIAS;
  const size_t need = split_workspace(sp, d);
  if (need > 0 && use_scratch) {
    st = scratch_address(&workspace);
    if (st != FA_OK) return st;
    workspace_bytes = FA_NOALLOC_SCRATCH_BYTES;
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need || !is_aligned(workspace, 256)) return FA_ERR_WORKSPACE;
    const int64_t nw = static_cast<int64_t>(need);
    if (overlaps(workspace, nw, q, nq) || overlaps(workspace, nw, k, nkv) ||
        overlaps(workspace, nw, v, nkv) || overlaps(workspace, nw, o, nq) ||
        overlaps(workspace, nw, lse, nl) || overlaps(workspace, nw, key_len_mask, nkl))
      return FA_ERR_ALIAS;
  }

  // A decode step with grouped heads: the G = H / Hkv query heads of a
  // key/value head hold one row each, at stride d in q and o (and 1 in the
  // LSE), which is the layout of G query rows of one head.  Every decode row
  // sees the keys below its sequence's length, causal or not.  So the step
  // runs as Hkv heads of G rows each, not causal, on the main kernel, whose
  // products then go to the matrix cores and whose key/value tiles serve all
  // G rows: each K and V row is read once per key range.
  const bool grouped_decode = Nq == 1 && Hkv < H;
  const int vH = grouped_decode ? Hkv : H, vN = grouped_decode ? H / Hkv : Nq;
  fa::FwdParams p = make_params(q, k, v, o, lse, B, vH, vN, scale, key_len_mask, dtype);
  p.Nk = Nk;
  p.Hkv = Hkv;
  p.end_aligned = 1;
  p.splits = sp.splits;
  p.split_keys = sp.split_keys;
  if (grouped_decode) causal = 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* const ws = static_cast<char*>(workspace);
  if (sp.splits > 1 || sp.balanced) {
    p.o_part = reinterpret_cast<float*>(ws);
    p.lse_part = reinterpret_cast<float*>(ws + split_part_bytes(sp, d));
  }
  fa::MergeParams mp{};
  mp.o_part = p.o_part;
  mp.lse_part = p.lse_part;
  mp.o = o;
  mp.lse = lse;
  mp.rows = sp.rows;
  mp.splits = sp.splits;
  if (sp.balanced) {
    // the decode kernel leaves partials of every row; the merge completes
    // them
    int64_t* cum =
        reinterpret_cast<int64_t*>(ws + split_part_bytes(sp, d) + split_lse_bytes(sp));
    if (fa::launch_decode_balanced_bf16(p, d, sp.workgroups, cum, hs) != hipSuccess)
      return FA_ERR_HIP;
    mp.cum = cum;
    mp.key_len = key_len_mask;
    mp.B = B;
    mp.H = H;
    mp.Nk = Nk;
    mp.workgroups = sp.workgroups;
    return fa::launch_merge(mp, d, true, hs) == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  // one query row: the row sees every key below its sequence's length
  // whether or not the mask is causal
  const hipError_t e = Nq == 1 && !grouped_decode ? fa::launch_decode_bf16(p, d, hs)
                                                  : fa::launch_fwd_bf16(p, d, causal != 0, hs);
  if (e != hipSuccess) return FA_ERR_HIP;
  if (sp.splits > 1 && fa::launch_merge(mp, d, true, hs) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

}  // namespace

extern "C" int fa_forward_split(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                                int causal, const int32_t* key_len_mask, int dtype, int num_splits,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return forward_split(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, key_len_mask, dtype,
                       num_splits, workspace, workspace_bytes, false, stream);
}

extern "C" int fa_forward_split_noalloc(const void* q, const void* k, const void* v, void* o,
                                        float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                                        float scale, int causal, const int32_t* key_len_mask,
                                        int dtype, int num_splits, void* stream) {
  return forward_split(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, key_len_mask, dtype,
                       num_splits, nullptr, 0, true, stream);
}

extern "C" size_t fa_backward_workspace_bytes(int B, int H, int N, int d, int dtype) {
  Shape s;
  bool empty = false;
  if (dtype != FA_DTYPE_BF16 || (d != 64 && d != 128)) return 0;
  if (check_scalars(B, H, N, d, 1.f, dtype, &s, &empty) != FA_OK || empty) return 0;
  return round256(size_t(s.rows) * sizeof(float));
}

namespace {

// Keep threshold of a dropout rate p in [0, 1): a draw u is kept iff
// u >= floor(p * 2^32).  p * 2^32 only moves the binary exponent, so the
// product is exact in double and the floor is that of the real number.
uint32_t keep_threshold(const double p) {
  const double t = std::floor(p * 4294967296.0);
  return static_cast<uint32_t>(std::min(t, 4294967295.0));
}

// Dropout of the forward whose gradients are taken (fa_forward_dropout's
// arguments); nullptr for none.
struct DropArgs {
  double p;
  uint64_t seed;
  uint32_t offset;
};

// Additive mask of the forward whose gradients are taken (fa_forward_bias's
// arguments); nullptr for none.
struct BiasArgs {
  const float* bias;
  int64_t sb, sh, ld;
};

// Validates a mask of fa_forward_bias's form for a [B, H, N, N] problem and
// returns its extent in elements (rows read up to the next multiple of 4,
// inside bias_ld), or -1 for a bad shape.
int64_t bias_extent(int B, int H, int N, int64_t sb, int64_t sh, int64_t ld) {
  if (sb < 0 || sh < 0 || ld < N || ld % 4 != 0 || sb % 4 != 0 || sh % 4 != 0) return -1;
  const int64_t row = (int64_t(N) + 3) / 4 * 4;
  const double ext_d = double(B - 1) * double(sb) + double(H - 1) * double(sh) +
                       double(N - 1) * double(ld) + double(row);
  if (ext_d > double(int64_t(1) << 60)) return -1;
  return int64_t(B - 1) * sb + int64_t(H - 1) * sh + int64_t(N - 1) * ld + row;
}

int backward_dense(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* key_len_mask, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream, const DropArgs* drop,
                   const BiasArgs* mask = nullptr) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (drop && !(drop->p >= 0.0 && drop->p < 1.0)) return FA_ERR_SCALE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  Shape s;
  bool empty = false;
  int st = check_scalars(B, H, N, d, scale, dtype, &s, &empty);
  if (st != FA_OK || empty) return st;
  const void* ins[] = {q, k, v, o, dout};
  void* outs[] = {dq, dk, dv};
  for (const void* x : ins)
    if (!x) return FA_ERR_NULL;
  for (void* x : outs)
    if (!x) return FA_ERR_NULL;
  if (!lse) return FA_ERR_NULL;
  for (const void* x : ins)
    if (!is_aligned(x, 16)) return FA_ERR_ALIGN;
  for (void* x : outs)
    if (!is_aligned(x, 16)) return FA_ERR_ALIGN;
  if (!is_aligned(lse, 4) || (key_len_mask && !is_aligned(key_len_mask, 4))) return FA_ERR_ALIGN;
  const int64_t nb = s.elems * s.esz, nl = s.rows * 4, nk = key_len_mask ? int64_t(B) * 4 : 0;
  const size_t need = round256(size_t(s.rows) * sizeof(float));
  if (!workspace || workspace_bytes < need || !is_aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  const int64_t nw = static_cast<int64_t>(need);
  // the outputs (and the workspace) overlap no input and no other output
  struct Region { const void* p; int64_t n; };
  const Region written[] = {{dq, nb}, {dk, nb}, {dv, nb}, {workspace, nw}};
  const Region read[] = {{q, nb}, {k, nb}, {v, nb}, {o, nb}, {dout, nb}, {lse, nl},
                         {key_len_mask, nk}};
  for (int i = 0; i < 4; ++i) {
    for (const Region& r : read)
      if (overlaps(written[i].p, written[i].n, r.p, r.n)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(written[i].p, written[i].n, written[j].p, written[j].n)) return FA_ERR_ALIAS;
  }
  if (mask) {
    const int64_t ext = bias_extent(B, H, N, mask->sb, mask->sh, mask->ld);
    if (ext < 0) return FA_ERR_SHAPE;
    if (!mask->bias) return FA_ERR_NULL;
    if (!is_aligned(mask->bias, 16)) return FA_ERR_ALIGN;
    for (int i = 0; i < 4; ++i)
      if (overlaps(written[i].p, written[i].n, mask->bias, ext * 4)) return FA_ERR_ALIAS;
  }

  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dvec = static_cast<float*>(workspace);
  p.key_len = key_len_mask;
  p.B = B;
  p.H = H;
  p.N = N;
  p.Hkv = H;
  p.Nk = N;
  p.n_qtiles = (N + 127) / 128;
  p.n_ktiles = (N + 127) / 128;
  p.scale = scale;
  p.c2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  if (drop) {
    // the forward's stream and threshold (fa_forward_dropout)
    p.drop = 1;
    p.drop_threshold = keep_threshold(drop->p);
    p.seed_lo = static_cast<uint32_t>(drop->seed & 0xFFFFFFFFu);
    p.seed_hi = static_cast<uint32_t>(drop->seed >> 32);
    p.drop_offset = drop->offset;
    p.keep_scale = static_cast<float>(1.0 / (1.0 - drop->p));
  }
  if (mask) {
    p.bias = mask->bias;
    p.bias_sb = mask->sb;
    p.bias_sh = mask->sh;
    p.bias_ld = mask->ld;
  }
  if (fa::launch_bwd_bf16(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

}  // namespace

extern "C" int fa_backward(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int N, int d, float scale, int causal,
                           const int32_t* key_len_mask, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return backward_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                        key_len_mask, dtype, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, void* dq, void* dk,
                                   void* dv, int B, int H, int N, int d, float scale, int causal,
                                   const int32_t* key_len_mask, int dtype, double p_drop,
                                   uint64_t seed, uint32_t offset, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const DropArgs drop{p_drop, seed, offset};
  return backward_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                        key_len_mask, dtype, workspace, workspace_bytes, stream, &drop);
}

extern "C" int fa_backward_bias(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                const float* bias, int B, int H, int N, int d, float scale,
                                int causal, const int32_t* key_len_mask, int dtype,
                                int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_ld,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const BiasArgs mask{bias, bias_stride_b, bias_stride_h, bias_ld};
  return backward_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                        key_len_mask, dtype, workspace, workspace_bytes, stream, nullptr, &mask);
}

namespace {

// Pointer, alignment, workspace and aliasing checks shared by the grouped and
// packed backward entry points.  nq: bytes of q, o, dout and dq; nkv: bytes
// of k, v, dk and dv; nl: bytes of lse and of the D workspace; extra: other
// read-only arrays (lengths, sequence offsets).
struct Region {
  const void* p;
  int64_t n;
};

int check_backward_buffers(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int64_t nq, int64_t nkv, int64_t nl, const Region* extra, int n_extra,
                           void* workspace, size_t workspace_bytes) {
  if (nq > 0 && (!q || !o || !dout || !dq || !lse)) return FA_ERR_NULL;
  if (nkv > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL;
  for (int i = 0; i < n_extra; ++i)
    if (extra[i].n > 0 && !extra[i].p) return FA_ERR_NULL;
  const void* tensors[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* x : tensors)
    if (!is_aligned(x, 16)) return FA_ERR_ALIGN;
  if (!is_aligned(lse, 4)) return FA_ERR_ALIGN;
  for (int i = 0; i < n_extra; ++i)
    if (!is_aligned(extra[i].p, 4)) return FA_ERR_ALIGN;
  const size_t need = round256(static_cast<size_t>(nl));
  if (need > 0 && (!workspace || workspace_bytes < need || !is_aligned(workspace, 256)))
    return FA_ERR_WORKSPACE;
  const int64_t nw = static_cast<int64_t>(need);
  // the outputs (and the workspace) overlap no input and no other output
  const Region written[] = {{dq, nq}, {dk, nkv}, {dv, nkv}, {workspace, nw}};
  const Region read[] = {{q, nq}, {k, nkv}, {v, nkv}, {o, nq}, {dout, nq}, {lse, nl}};
  for (int i = 0; i < 4; ++i) {
    for (const Region& r : read)
      if (overlaps(written[i].p, written[i].n, r.p, r.n)) return FA_ERR_ALIAS;
    for (int e = 0; e < n_extra; ++e)
      if (overlaps(written[i].p, written[i].n, extra[e].p, extra[e].n)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(written[i].p, written[i].n, written[j].p, written[j].n)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

fa::BwdParams backward_params(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              void* workspace, int B, int H, int Hkv, float scale) {
  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dvec = static_cast<float*>(workspace);
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.scale = scale;
  p.c2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  return p;
}

int backward_scalars(int H, int Hkv, int d, float scale, int dtype) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (H < 0 || Hkv < 1 || (H > 0 && H % Hkv != 0)) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  const double c = std::fabs(static_cast<double>(scale)) * 1.4426950408889634;
  if (!std::isfinite(static_cast<float>(c))) return FA_ERR_SCALE;
  return FA_OK;
}

}  // namespace

extern "C" int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                               int causal, const int32_t* key_len_mask, int dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  int st = backward_scalars(H, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (B < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (B == 0) return FA_OK;
  // offsets within one (batch, head) slice are 32-bit; grids fit an int
  if (int64_t(Nq) * d * 2 > INT_MAX || int64_t(Nk) * d * 2 > INT_MAX) return FA_ERR_SHAPE;
  const int64_t qtiles = (int64_t(Nq) + 127) / 128, ktiles = (int64_t(Nk) + 127) / 128;
  if (int64_t(B) * H * qtiles > INT_MAX || int64_t(B) * Hkv * ktiles > INT_MAX)
    return FA_ERR_SHAPE;
  const int64_t nq = int64_t(B) * H * Nq * d * 2, nkv = int64_t(B) * Hkv * Nk * d * 2;
  const int64_t nl = int64_t(B) * H * Nq * 4;
  const Region extra[] = {{key_len_mask, key_len_mask ? int64_t(B) * 4 : 0}};
  st = check_backward_buffers(q, k, v, o, lse, dout, dq, dk, dv, nq, nkv, nl, extra, 1, workspace,
                              workspace_bytes);
  if (st != FA_OK) return st;
  fa::BwdParams p = backward_params(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Hkv, scale);
  p.N = Nq;
  p.Nk = Nk;
  p.key_len = key_len_mask;
  p.end_aligned = 1;
  p.n_qtiles = static_cast<int>(qtiles);
  p.n_ktiles = static_cast<int>(ktiles);
  if (fa::launch_bwd_bf16(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

extern "C" int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                  int H, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                  int max_seqlen_k, int d, float scale, int causal, int dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  int st = backward_scalars(H, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (B < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return FA_ERR_SHAPE;
  if (B == 0) return FA_OK;
  // offsets within one sequence are 32-bit in the kernels; grids fit an int
  if (int64_t(max_seqlen_q) * H * d * 2 > INT_MAX || int64_t(max_seqlen_k) * Hkv * d * 2 > INT_MAX)
    return FA_ERR_SHAPE;
  const int64_t qtiles = (int64_t(max_seqlen_q) + 127) / 128;
  const int64_t ktiles = (int64_t(max_seqlen_k) + 127) / 128;
  if (int64_t(B) * H * qtiles > INT_MAX || int64_t(B) * Hkv * ktiles > INT_MAX)
    return FA_ERR_SHAPE;
  const int64_t nq = int64_t(total_q) * H * d * 2, nkv = int64_t(total_k) * Hkv * d * 2;
  const int64_t nl = int64_t(total_q) * H * 4, ncu = (int64_t(B) + 1) * 4;
  const Region extra[] = {{cu_seqlens_q, ncu}, {cu_seqlens_k, ncu}};
  st = check_backward_buffers(q, k, v, o, lse, dout, dq, dk, dv, nq, nkv, nl, extra, 2, workspace,
                              workspace_bytes);
  if (st != FA_OK) return st;
  fa::BwdParams p = backward_params(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Hkv, scale);
  p.N = max_seqlen_q;
  p.Nk = max_seqlen_k;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.end_aligned = 1;
  // with no query rows (or no key rows) in the batch only the other kernel runs
  p.n_qtiles = total_q > 0 ? static_cast<int>(qtiles) : 0;
  p.n_ktiles = total_k > 0 ? static_cast<int>(ktiles) : 0;
  if (fa::launch_bwd_bf16(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

extern "C" int fa_naive_backward(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                 int B, int H, int N, int d, float scale, int causal,
                                 const int32_t* key_len_mask, int dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  Shape s;
  bool empty = false;
  int st = check_scalars(B, H, N, d, scale, dtype, &s, &empty);
  if (st != FA_OK || empty) return st;
  const void* ins[] = {q, k, v, o, dout};
  void* outs[] = {dq, dk, dv};
  for (const void* x : ins)
    if (!x || !is_aligned(x, 16)) return x ? FA_ERR_ALIGN : FA_ERR_NULL;
  for (void* x : outs)
    if (!x || !is_aligned(x, 16)) return x ? FA_ERR_ALIGN : FA_ERR_NULL;
  if (!lse) return FA_ERR_NULL;
  if (!is_aligned(lse, 4) || (key_len_mask && !is_aligned(key_len_mask, 4))) return FA_ERR_ALIGN;
  if (int64_t(N) * N > (int64_t(1) << 62) / (int64_t(B) * H)) return FA_ERR_SHAPE;
  const size_t need = fa_naive_workspace_bytes(B, H, N, dtype);
  if (!workspace || workspace_bytes < need || !is_aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  const int64_t nb = s.elems * s.esz, nl = s.rows * 4, nk = key_len_mask ? int64_t(B) * 4 : 0;
  struct Region { const void* p; int64_t n; };
  const Region written[] = {{dq, nb}, {dk, nb}, {dv, nb}, {workspace, static_cast<int64_t>(need)}};
  const Region read[] = {{q, nb}, {k, nb}, {v, nb}, {o, nb}, {dout, nb}, {lse, nl},
                         {key_len_mask, nk}};
  for (int i = 0; i < 4; ++i) {
    for (const Region& r : read)
      if (overlaps(written[i].p, written[i].n, r.p, r.n)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(written[i].p, written[i].n, written[j].p, written[j].n)) return FA_ERR_ALIAS;
  }
  (void)o;  // D is formed from P and dP here; o is validated for the shared contract

  void* spm = workspace;
  void* dpm = static_cast<char*>(workspace) + need / 2;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_blas_mu);
  if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
    g_blas[dev] = nullptr;
    return FA_ERR_HIP;
  }
  rocblas_handle hb = g_blas[dev];
  if (rocblas_set_stream(hb, hs) != rocblas_status_success) return FA_ERR_HIP;
  const rocblas_datatype t = rocblas_datatype_bf16_r;
  const float one = 1.f, zero = 0.f;
  const int bh = B * H;
  const rocblas_stride snd = int64_t(N) * d, snn = int64_t(N) * N;
  const rocblas_operation NN = rocblas_operation_none, TT = rocblas_operation_transpose;
  // Row-major X [r, c] is the column-major X^T [c, r]; every product below is
  // written for the column-major views.
  auto gemm = [&](rocblas_operation oa, rocblas_operation ob, int m, int n, int kk, float alpha,
                  const void* a, int lda, rocblas_stride sa, const void* bm, int ldb,
                  rocblas_stride sb, void* c, int ldc, rocblas_stride sc) {
    return rocblas_gemm_strided_batched_ex(hb, oa, ob, m, n, kk, &alpha, a, t, lda, sa, bm, t, ldb,
                                           sb, &zero, c, t, ldc, sc, c, t, ldc, sc, bh,
                                           rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                                           0) == rocblas_status_success;
  };
  fa::NaiveBwdParams np{};
  np.sp = spm;
  np.dpds = dpm;
  np.lse = lse;
  np.key_len = key_len_mask;
  np.B = B;
  np.H = H;
  np.N = N;
  np.causal = causal != 0;
  // S = scale Q K^T  (S^T = K Q^T), then P over it.
  if (!gemm(TT, NN, N, N, d, scale, k, d, snd, q, d, snd, spm, N, snn)) return FA_ERR_HIP;
  if (fa::launch_naive_bwd_p(np, hs) != hipSuccess) return FA_ERR_HIP;
  // dV = P^T dO  (dV^T = dO^T P)
  if (!gemm(NN, TT, d, N, N, one, dout, d, snd, spm, N, snn, dv, d, snd)) return FA_ERR_HIP;
  // dP = dO V^T  (dP^T = V dO^T), then dS over it.
  if (!gemm(TT, NN, N, N, d, one, v, d, snd, dout, d, snd, dpm, N, snn)) return FA_ERR_HIP;
  if (fa::launch_naive_bwd_ds(np, hs) != hipSuccess) return FA_ERR_HIP;
  // dQ = scale dS K  (dQ^T = K^T dS^T);  dK = scale dS^T Q  (dK^T = Q^T dS)
  if (!gemm(NN, NN, d, N, N, scale, k, d, snd, dpm, N, snn, dq, d, snd)) return FA_ERR_HIP;
  if (!gemm(NN, TT, d, N, N, scale, q, d, snd, dpm, N, snn, dk, d, snd)) return FA_ERR_HIP;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                 int H, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                 int max_seqlen_k, int d, float scale, int causal, int dtype,
                                 void* stream) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (B < 0 || H < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return FA_ERR_SHAPE;
  if (Hkv < 1 || (H > 0 && H % Hkv != 0)) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  const double c = std::fabs(static_cast<double>(scale)) * 1.4426950408889634;
  if (!std::isfinite(static_cast<float>(c))) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || total_q == 0 || max_seqlen_q == 0) return FA_OK;
  // offsets within one sequence are 32-bit in the kernel
  if (int64_t(max_seqlen_q) * H * d * 2 > INT_MAX || int64_t(max_seqlen_k) * Hkv * d * 2 > INT_MAX)
    return FA_ERR_SHAPE;
  const int64_t qtiles = (int64_t(max_seqlen_q) + fa::kQueryTile - 1) / fa::kQueryTile;
  if (int64_t(B) * H > INT_MAX || qtiles * B * H > INT_MAX) return FA_ERR_SHAPE;
  if (!q || !o || !lse || !cu_seqlens_q || !cu_seqlens_k || (total_k > 0 && (!k || !v)))
    return FA_ERR_NULL;
  if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(o, 16))
    return FA_ERR_ALIGN;
  if (!is_aligned(lse, 4) || !is_aligned(cu_seqlens_q, 4) || !is_aligned(cu_seqlens_k, 4))
    return FA_ERR_ALIGN;
  const int64_t nq = int64_t(total_q) * H * d * 2, nkv = int64_t(total_k) * Hkv * d * 2;
  const int64_t nl = int64_t(total_q) * H * 4, ncu = (int64_t(B) + 1) * 4;
  struct Region { const void* p; int64_t n; };
  const Region written[] = {{o, nq}, {lse, nl}};
  const Region read[] = {{q, nq}, {k, nkv}, {v, nkv}, {cu_seqlens_q, ncu}, {cu_seqlens_k, ncu}};
  for (const Region& w : written)
    for (const Region& r : read)
      if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_ALIAS;
  if (overlaps(o, nq, lse, nl)) return FA_ERR_ALIAS;

  fa::FwdParams p = make_params(q, k, v, o, lse, B, H, max_seqlen_q, scale, nullptr, dtype);
  p.Nk = max_seqlen_k;
  p.Hkv = Hkv;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.end_aligned = 1;
  p.split_keys = static_cast<int>(
      std::min<int64_t>((int64_t(max_seqlen_k) + 127) / 128 * 128, INT_MAX - 127));
  if (fa::launch_fwd_bf16(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

extern "C" int fa_forward_dropout(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int B, int H, int N, int d, float scale, int causal,
                                  const int32_t* key_len_mask, int dtype, double p_drop,
                                  uint64_t seed, uint32_t offset, void* stream) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!(p_drop >= 0.0 && p_drop < 1.0)) return FA_ERR_SCALE;
  Shape s;
  bool empty = false;
  int st = check_scalars(B, H, N, d, scale, dtype, &s, &empty);
  if (st != FA_OK || empty) return st;
  st = check_pointers(q, k, v, o, lse, key_len_mask, B, s);
  if (st != FA_OK) return st;
  fa::FwdParams p = make_params(q, k, v, o, lse, B, H, N, scale, key_len_mask, dtype);
  p.drop = 1;
  p.drop_threshold = keep_threshold(p_drop);
  p.seed_lo = static_cast<uint32_t>(seed & 0xFFFFFFFFu);
  p.seed_hi = static_cast<uint32_t>(seed >> 32);
  p.drop_offset = offset;
  p.keep_scale = static_cast<float>(1.0 / (1.0 - p_drop));
  if (fa::launch_fwd_bf16(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

extern "C" int fa_forward_bias(const void* q, const void* k, const void* v, void* o, float* lse,
                               const float* bias, int B, int H, int N, int d, float scale,
                               int causal, const int32_t* key_len_mask, int dtype,
                               int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_ld,
                               void* stream) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  Shape s;
  bool empty = false;
  int st = check_scalars(B, H, N, d, scale, dtype, &s, &empty);
  if (st != FA_OK || empty) return st;
  // extent of the bias in elements (the largest offset read, plus one)
  const int64_t ext = bias_extent(B, H, N, bias_stride_b, bias_stride_h, bias_ld);
  if (ext < 0) return FA_ERR_SHAPE;
  st = check_pointers(q, k, v, o, lse, key_len_mask, B, s);
  if (st != FA_OK) return st;
  if (!bias) return FA_ERR_NULL;
  if (!is_aligned(bias, 16)) return FA_ERR_ALIGN;
  if (overlaps(o, s.elems * s.esz, bias, ext * 4) || overlaps(lse, s.rows * 4, bias, ext * 4))
    return FA_ERR_ALIAS;
  fa::FwdParams p = make_params(q, k, v, o, lse, B, H, N, scale, key_len_mask, dtype);
  p.bias = bias;
  p.bias_sb = bias_stride_b;
  p.bias_sh = bias_stride_h;
  p.bias_ld = bias_ld;
  if (fa::launch_fwd_bf16(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is negative or the sizes overflow";
    case FA_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
    case FA_ERR_DTYPE: return "dtype not supported by this entry point";
    case FA_ERR_ALIGN: return "a pointer is misaligned (q, k, v, o: 16 bytes; lse, key_len: 4)";
    case FA_ERR_SCALE: return "scale must be finite (and a dropout rate in [0, 1))";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_WORKSPACE: return "workspace is NULL, misaligned or too small";
    case FA_ERR_HIP: return "the HIP runtime reported an error";
    default: return "unknown status";
  }
}

extern "C" int fa_abi_version(void) { return FA_ABI_VERSION; }
