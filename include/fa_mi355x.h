/*
 * fa_mi355x.h -- C ABI of the MI355X (gfx950) exact attention forward.
 *
 * The operation is exact scaled dot-product attention with an additive mask,
 *     O = softmax(scale * Q K^T + M) V,
 * softmax taken over keys for each query row, as defined on the pages
 * "FlashAttention: Exact Attention as an IO-Aware Streaming Computation"
 * (section "Problem setting") and "FlashAttention" (glossary, section "Move
 * less data", which adds the optional additive mask M).  Besides O the call
 * writes one log-sum-exp per query row, the compact per-row normalisation
 * record that "IO-aware exact attention" (section "Backward recomputation")
 * keeps instead of the probability matrix.
 *
 * fa_forward computes it tile by tile with a running maximum, denominator and
 * unnormalised numerator per query row ("FlashAttention: Exact Attention as
 * an IO-Aware Streaming Computation", section "Mathematical structure";
 * "IO-aware exact attention", section "One tiled forward-pass iteration"):
 * no N x N score or probability matrix is ever written to device memory.
 *
 * fa_naive_forward computes the same result along the materialised dataflow
 * the pages contrast it with ("IO-aware exact attention", section "Traffic in
 * the materialized implementation"): S = scale Q K^T is written to device
 * memory, a softmax pass reads S and writes P, and a third pass computes
 * O = P V.  It exists to measure the N^2 traffic the fused kernel removes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout   q, k, v, o: [B, H, N, d] row-major, d innermost, contiguous.
 *           lse: [B, H, N] float32, natural-log units.
 *           key_len_mask: [B] int32 or NULL.
 *  Dtypes   FA_DTYPE_BF16: q, k, v, o are bfloat16; arithmetic is bf16 matrix
 *           products with fp32 accumulation and fp32 softmax state; the
 *           probabilities enter the second product rounded to bf16
 *           (nearest-even) and O is rounded to bf16 (nearest-even).
 *           FA_DTYPE_F32: q, k, v, o are float32; everything is fp32.
 *  Head dim d in {64, 128}.
 *  Sizes    B, H, N >= 0.  If any is 0 there is nothing to do: the call
 *           returns FA_OK without touching memory (pointers may be NULL).
 *           B*H*N*d must be below 2^62, the number of 128-row query tiles
 *           times B*H below 2^31, and one (batch, head) slice of q
 *           (N*d elements) at most 2^31 - 1 bytes.
 *  Mask M   causal != 0: key j is visible to query i only if j <= i.
 *           key_len_mask != NULL: L_b = clamp(key_len_mask[b], 0, N); keys
 *           j >= L_b are masked and query rows i >= L_b are padding.
 *           A row with no visible key (only padding rows) gets O = 0 and
 *           LSE = -inf; this is the explicit fully-masked handling the
 *           glossary's section "Why a tile can be discarded" asks for.
 *  Scale    used as given (any finite value; the usual choice is 1/sqrt(d)).
 *  Memory   every pointer is device memory owned by the caller, on the
 *           device current for the calling thread.  q, k, v, o must be
 *           16-byte aligned; lse, key_len_mask 4-byte aligned.  o and lse
 *           must not overlap q, k, v, key_len_mask or each other.  The
 *           library keeps no per-call state and allocates no memory.
 *  Stream   stream is a hipStream_t (NULL = the legacy default stream).
 *           Work is enqueued asynchronously; the call returns once it is
 *           enqueued.  A device fault surfaces at the caller's next
 *           synchronisation on that stream.
 *  Errors   arguments are validated on the host before any HIP call; a bad
 *           argument returns a negative fa_status_t and writes nothing.  A
 *           launch failure returns FA_ERR_HIP.  No C++ exception crosses
 *           this interface.  Calls are thread-safe.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_BF16 = 0,
  FA_DTYPE_F32 = 1
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  FA_ERR_SHAPE = -2,       /* B, H or N negative, or sizes overflow            */
  FA_ERR_HEAD_DIM = -3,    /* d not in {64, 128}                               */
  FA_ERR_DTYPE = -4,       /* dtype not an fa_dtype_t                          */
  FA_ERR_ALIGN = -5,       /* a pointer is not aligned as required             */
  FA_ERR_SCALE = -6,       /* scale not finite, or dropout rate outside [0, 1) */
  FA_ERR_ALIAS = -7,       /* an output overlaps an input or the other output */
  FA_ERR_WORKSPACE = -8,   /* workspace NULL, misaligned or too small          */
  FA_ERR_HIP = -9          /* the HIP runtime reported an error at launch      */
} fa_status_t;

/*
 * Fused attention forward (the streamed tile-by-tile computation).
 *   q, k, v      inputs [B, H, N, d] of `dtype`.
 *   o            output [B, H, N, d] of `dtype`; every element is written.
 *   lse          output [B, H, N] float32; every element is written:
 *                LSE_i = ln sum_{visible j} exp(scale * q_i . k_j), or -inf.
 *   scale        multiplies Q K^T before the mask is added.
 *   causal       0 or non-zero, see the mask convention above.
 *   key_len_mask device int32 [B] or NULL.
 *   stream       hipStream_t to enqueue on.
 * Returns FA_OK or a negative fa_status_t.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const int32_t* key_len_mask, int dtype, void* stream);

/*
 * Bytes of device workspace fa_naive_forward needs: the materialised score
 * and probability matrices, B*H*N*N elements each, stored in `dtype`, each
 * rounded up to 256 bytes.  Returns 0 for invalid arguments.
 */
size_t fa_naive_workspace_bytes(int B, int H, int N, int dtype);

/*
 * Materialised three-pass attention forward, same arguments and results as
 * fa_forward plus a caller-owned device workspace of at least
 * fa_naive_workspace_bytes(B, H, N, dtype) bytes (256-byte aligned).  The
 * workspace must not overlap any other argument.  S and P are stored in
 * `dtype` (bf16 for bf16 inputs), so results differ from fa_forward by the
 * extra rounding of S.
 */
int fa_naive_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal,
                     const int32_t* key_len_mask, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-KV attention forward: Nq query rows against Nk key rows, with the
 * keys of every query tile divided into ranges that separate workgroups
 * compute, each leaving a normalised partial output and its log-sum-exp in
 * the workspace; a second kernel combines them with the block-summary rule
 * of the page "FlashAttention" (sections "Why a tile can be discarded" and
 * "One row, checked two ways": each block's denominator and numerator are
 * expressed against a common reference maximum, then added).  It is for the
 * shapes where one workgroup per query tile leaves the device idle -- few
 * query rows against many keys (decode), or few (batch, head) pairs at long
 * Nk -- which "IO-aware exact attention" (section "Common errors") names as
 * needing a different schedule.
 *   q, o         [B, H, Nq, d] of `dtype`; k, v [B, Hkv, Nk, d]; lse [B, H, Nq].
 *   Hkv          key/value heads, >= 1, dividing H: query head h reads key/value
 *                head h / (H / Hkv) (grouped-query attention; Hkv = H is plain
 *                multi-head attention, Hkv = 1 multi-query attention).
 *   Positions    L_b = clamp(key_len_mask[b], 0, Nk), or Nk when key_len_mask
 *                is NULL: sequence b holds keys 0 .. L_b - 1 and its query
 *                rows are the last Nq positions of that sequence, row i at key
 *                position p = i + L_b - Nq (decode: Nq = 1 sits at L_b - 1).
 *                Without key_len_mask and with Nq = Nk this is position i, and
 *                the call computes what fa_forward computes (up to the order
 *                of the additions).
 *   Mask         keys j >= L_b are never visible; causal != 0 also hides keys
 *                j > p.  No row is padding: every row sees keys 0 .. L_b - 1
 *                (0 .. min(p, L_b - 1) if causal).  A row that sees no key
 *                (L_b = 0, or p < 0 under causal, which needs Nq > L_b) gets
 *                O = 0 and LSE = -inf.
 *   dtype        FA_DTYPE_BF16 only (FA_ERR_DTYPE otherwise).
 *   num_splits   key ranges per query tile, >= 1, or 0 to let the library
 *                choose.  With 0, a decode step (Nq = 1) with Hkv = H that
 *                would need more than one range per row to fill the device
 *                is cut instead into P <= 512 equal shares of all rows'
 *                visible keys (64-key units, rows laid end to end), one per
 *                workgroup, whatever the per-sequence lengths (which are
 *                read on the device); every other shape gets enough ranges
 *                to fill the device (with Nq = 1 and Hkv < H one workgroup
 *                serves the H / Hkv query heads of a key/value head, and the
 *                choice counts those workgroups).  Ranges are whole 128-key
 *                blocks, so fewer ranges than asked may be used.
 *   workspace    device memory, 256-byte aligned, of at least
 *                fa_split_workspace_bytes(B, H, Nq, Nk, d, num_splits) bytes
 *                (enough for every Hkv dividing H),
 *                overlapping no other argument: fp32 partial outputs
 *                [ranges, B, H, Nq, d] and their log-sum-exp [ranges, B, H, Nq]
 *                for key ranges; for balanced shares 4 (P + B H) partial rows
 *                of d floats, their log-sum-exp, then B + 1 int64 unit
 *                offsets.  When a single range is used it is not touched
 *                (NULL and 0 are then accepted).
 *   Sizes        B, H, Nq, Nk >= 0 (nothing to do if B, H or Nq is 0; Nk = 0
 *                gives O = 0, LSE = -inf, and k, v may then be NULL); one
 *                (batch, head) slice of q and of
 *                k at most 2^31 - 1 bytes; num_splits <= 65536.
 * Enqueues two kernels on `stream` (one when a single range is used).  The
 * remaining conventions (alignment, aliasing, errors, streams) are those of
 * fa_forward; a workspace that is NULL, misaligned or too small returns
 * FA_ERR_WORKSPACE.
 */
size_t fa_split_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);
int fa_forward_split(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                     const int32_t* key_len_mask, int dtype, int num_splits,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention forward over a packed batch of variable-length sequences with
 * grouped key/value heads ("IO-aware exact attention", section "Why
 * implementations form a family": packing and grouped heads change the
 * indexing, not the result).
 *   q, o         [total_q, H, d] of `dtype`: sequence b owns query rows
 *                cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 (token-major, heads
 *                interleaved); k, v [total_k, Hkv, d] likewise with cu_seqlens_k;
 *                lse [total_q, H] fp32.
 *   cu_seqlens_q, cu_seqlens_k  device int32 [B + 1], non-decreasing, starting
 *                at 0 and ending at total_q / total_k.  The library cannot read
 *                them on the host: offsets outside the tensors are the caller's
 *                error (like any bad pointer).
 *   max_seqlen_q, max_seqlen_k  at least every sequence's query / key count;
 *                rows beyond max_seqlen_q are not computed.
 *   Positions    each sequence's query rows are the last of its keys: row i of a
 *                sequence with Lq queries and Lk keys sits at key position
 *                i + Lk - Lq (with Lq = Lk, position i), as in fa_forward_split.
 *   Mask         causal != 0 hides keys after the row's position; a row that
 *                sees no key (Lk = 0, or position < 0) gets O = 0, LSE = -inf.
 *   Hkv          key/value heads, dividing H, as in fa_forward_split.
 *   dtype        FA_DTYPE_BF16 only; d = 64 or 128.
 *   Sizes        one sequence's rows of q (and of k) at most 2^31 - 1 bytes.
 * Enqueues one kernel on `stream`; allocates nothing.
 */
int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int H,
                      int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                      int d, float scale, int causal, int dtype, void* stream);

/*
 * Attention backward by recomputation ("IO-aware exact attention", section
 * "Backward recomputation"): the gradients dQ, dK, dV of the loss
 * sum(dO * O) for O = fa_forward(q, k, v, ...), rebuilt from the inputs, the
 * forward's output o and its log-sum-exp lse, without storing any N x N
 * matrix.  With P the masked softmax, D_i = dO_i . O_i:
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
 *   q, k, v, o, dout, dq, dk, dv  [B, H, N, d] of `dtype`; lse [B, H, N] fp32 as
 *                written by fa_forward with the same scale, causal and key_len_mask.
 *   Masks        those of fa_forward; padding rows and keys at or beyond L_b get
 *                zero gradients (their dO and lse entries are not read).
 *   dtype        FA_DTYPE_BF16 only; d = 64 or 128 (FA_ERR_HEAD_DIM otherwise).
 *   workspace    device memory, 256-byte aligned, of at least
 *                fa_backward_workspace_bytes(B, H, N, d, dtype) bytes (fp32 D,
 *                [B, H, N]); it and dq, dk, dv overlap no input and no other output.
 * Enqueues two kernels on `stream` (dQ and D, then dK and dV).  Validation,
 * alignment and error conventions are those of fa_forward.
 */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d, int dtype);
int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, const int32_t* key_len_mask, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of fa_forward_dropout's result: the gradients of sum(dO * O) for
 * O = (P * Z / (1 - p)) V with the keep mask Z of the forward ("IO-aware
 * exact attention", section "Why implementations form a family", names
 * dropout among the variants), regenerated from the same Philox4x32-10
 * stream (seed, offset; counter (j/4, i, b*H + h, offset), draw = word j % 4,
 * kept iff draw >= floor(p_drop * 2^32), formed exactly from the double
 * p_drop), never stored:
 *   dV = (P*Z)^T dO / (1-p),  dS = P * (Z * dO V^T / (1-p) - D),  D_i = dO_i . O_i.
 * Arguments as fa_backward plus p_drop, seed and offset, which must be those
 * of the fa_forward_dropout call that produced o and lse; p_drop outside
 * [0, 1) returns FA_ERR_SCALE.  bf16, d = 64 or 128.
 */
int fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                        int H, int N, int d, float scale, int causal,
                        const int32_t* key_len_mask, int dtype, double p_drop, uint64_t seed,
                        uint32_t offset, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of fa_forward_bias's result: the gradients dQ, dK, dV of
 * sum(dO * O) for O = softmax(scale * Q K^T + M) V with the masks of
 * fa_forward, by the recomputation of fa_backward with P rebuilt from the
 * masked scores ("IO-aware exact attention", sections "Move less data" and
 * "Backward recomputation").  M is a constant: no gradient is formed for it.
 * Arguments as fa_backward, plus the mask of the fa_forward_bias call that
 * produced o and lse (bias, bias_stride_b, bias_stride_h, bias_ld, with the
 * layout and checks described there).  bf16, d = 64 or 128.
 */
int fa_backward_bias(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, const float* bias, int B,
                     int H, int N, int d, float scale, int causal, const int32_t* key_len_mask,
                     int dtype, int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_ld,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of fa_forward_split's result (grouped key/value heads, query rows
 * at the end of each sequence's keys), by the recomputation of fa_backward
 * ("IO-aware exact attention", section "Backward recomputation"; grouped
 * heads are among the variants of section "Why implementations form a
 * family").
 *   q, o, dout, dq  [B, H, Nq, d]; k, v, dk, dv [B, Hkv, Nk, d]; lse [B, H, Nq]
 *                fp32 as written by fa_forward_split with the same scale,
 *                causal and key_len_mask.  H % Hkv == 0; query head h reads
 *                key/value head h / (H / Hkv), and dk, dv of a key/value head
 *                are the sums over the H / Hkv query heads that read it.
 *   Positions    as fa_forward_split: row i of sequence b at key position
 *                i + L_b - Nq, L_b = clamp(key_len_mask[b], 0, Nk) (Nk without
 *                a mask).  Keys at or beyond L_b, and rows that see no key,
 *                get zero gradients.
 *   workspace    256-byte aligned, fa_backward_workspace_bytes(B, H, Nq, d,
 *                dtype) bytes (fp32 D in the layout of lse); may be NULL when
 *                B * H * Nq == 0.
 *   Empty cases  Nq == 0 or H == 0 writes dk = dv = 0; Nk == 0 writes dq = 0
 *                (k, v, dk, dv may then be NULL).
 * bf16 only, d = 64 or 128.  Validation, alignment, aliasing and error
 * conventions are those of fa_backward.
 */
int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq,
                    int Nk, int d, float scale, int causal, const int32_t* key_len_mask, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of fa_forward_varlen's result: packed batches, grouped heads.
 *   q, o, dout, dq  [total_q, H, d]; k, v, dk, dv [total_k, Hkv, d]; lse
 *                [total_q, H] fp32 as written by fa_forward_varlen with the
 *                same arguments; cu_seqlens_q / cu_seqlens_k as there (device
 *                [B + 1], non-decreasing from 0 to the totals, each length at
 *                most max_seqlen_q / max_seqlen_k: not checked on the host).
 *   Positions    row i of sequence b at key position i + Lk_b - Lq_b.
 *   workspace    256-byte aligned, fa_backward_workspace_bytes(1, H, total_q,
 *                d, dtype) bytes (fp32 D in the layout of lse); may be NULL
 *                when H * total_q == 0.
 *   Empty cases  a sequence without queries gets dk = dv = 0 for its keys; one
 *                without keys gets dq = 0.
 * bf16 only, d = 64 or 128.  Other conventions as fa_backward.
 */
int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int H,
                       int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                       int d, float scale, int causal, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Stored-state backward: the same gradients as fa_backward, computed the
 * conventional way with the N x N matrices in HBM (S and then P in the first
 * half of the workspace, dP and then dS in the second), by five rocBLAS
 * products and two row passes -- the comparison path of "IO-aware exact
 * attention" (section "Measure stored-state and recomputed attention
 * backward").  P and dS are stored in bf16, so results are slightly less
 * accurate than fa_backward's.  Arguments as fa_backward; dtype
 * FA_DTYPE_BF16; d = 64 or 128; the workspace is fa_naive_workspace_bytes(B, H, N,
 * dtype) bytes, 256-byte aligned (o is validated but not read: D is formed
 * from the stored P and dP).
 */
int fa_naive_backward(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                      int H, int N, int d, float scale, int causal, const int32_t* key_len_mask,
                      int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_forward with dropout on the attention probabilities ("IO-aware exact
 * attention", section "Why implementations form a family", names dropout
 * as a variant): O = (P * Z / (1 - p_drop)) V, LSE of the undropped row.
 * Z_ij (keep = 1) is decided by Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 * SC 2011) with key (seed & 0xffffffff, seed >> 32) and counter
 * (j / 4, i, b * H + h, offset): with u the counter's output word j % 4,
 * Z_ij = 1 iff u >= floor(p_drop * 2^32).  The threshold is formed from the
 * double p_drop exactly (p_drop * 2^32 is exact in binary64), so the rate a
 * caller passes is the rate applied, with no rounding to a narrower type.
 * The same (seed, offset) gives the same mask on every call; vary offset
 * between steps.
 *   p_drop       in [0, 1) (FA_ERR_SCALE otherwise).
 *   dtype        FA_DTYPE_BF16 only.
 * Other arguments and conventions are those of fa_forward.
 */
int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, float scale, int causal,
                       const int32_t* key_len_mask, int dtype, double p_drop, uint64_t seed,
                       uint32_t offset, void* stream);

/*
 * fa_forward with a general additive mask M ("FlashAttention" glossary,
 * section "Move less data": O = softmax(Q K^T / sqrt(d) + M) V):
 * s_ij = scale * q_i . k_j + M_bhij, then the causal and length masks of
 * fa_forward.  M may hold -inf (the pair is hidden); a row whose every score
 * is -inf gets O = 0, LSE = -inf.
 *   bias         device fp32, element (b, h, i, j) at
 *                bias[b * bias_stride_b + h * bias_stride_h + i * bias_ld + j];
 *                a stride of 0 broadcasts over batch or heads.  16-byte aligned;
 *                bias_ld >= N; bias_ld and both strides multiples of 4 (pad the
 *                rows); FA_ERR_SHAPE otherwise.  Rows are read in 16-byte
 *                groups, so each row's elements up to the next multiple of 4
 *                at or above N must be readable (they lie within bias_ld).
 *   dtype        FA_DTYPE_BF16 only.
 * Reading M costs 4 * N * N bytes per (batch, head) it does not broadcast
 * over, on top of the IO-aware traffic.  Other arguments and conventions
 * are those of fa_forward.
 */
int fa_forward_bias(const void* q, const void* k, const void* v, void* o, float* lse,
                    const float* bias, int B, int H, int N, int d, float scale, int causal,
                    const int32_t* key_len_mask, int dtype, int64_t bias_stride_b,
                    int64_t bias_stride_h, int64_t bias_ld, void* stream);

/*
 * fa_forward_split for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  The
 * same computation and kernels as fa_forward_split, with the key ranges' fp32
 * partial results in a scratch area the library holds in device memory
 * (FA_NOALLOC_SCRATCH_BYTES on every device it runs on, until the process
 * ends) instead of a caller workspace.  Allocates nothing.
 *   q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, key_len_mask,
 *   dtype, num_splits, stream: as fa_forward_split.
 * Returns FA_ERR_WORKSPACE, before any HIP call, when the partial results,
 * fa_split_workspace_bytes(B, H, Nq, Nk, d, num_splits) bytes, exceed
 * FA_NOALLOC_SCRATCH_BYTES (num_splits = 1 needs none); other validation and
 * errors as fa_forward_split.  Every call on one device shares that device's
 * scratch: calls that overlap in time on one device (other streams, other
 * host threads) race and must be ordered by the caller.  No scratch content
 * carries over: each call writes every partial row it later reads.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
int fa_forward_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                             const int32_t* key_len_mask, int dtype, int num_splits, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int fa_abi_version(void);

#define FA_ABI_VERSION ((1 << 16) | 10)

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
