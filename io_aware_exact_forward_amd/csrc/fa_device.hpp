// Device-side helpers shared by the gfx950 attention kernels: vector types,
// the 32x32 MFMA wrappers, wave-half exchanges and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Operand layout on a 64-lane wave: lane l holds row (A) / column (B)
// l % 32 and eight consecutive k values starting at 8 * (l / 32).
// Accumulator layout: lane l holds column l % 32; register r holds row
// 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x2, fp32) * B(2x32, fp32); lane l holds k = l / 32.
__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held by register r of a lane in half h.
__device__ __forceinline__ constexpr int acc_row(int r, int h) {
  return 8 * (r >> 2) + 4 * h + (r & 3);
}

// Combine a value with the one held by the lane 32 apart (the other half of
// the wave).  v_permlane32_swap exchanges the two halves between a pair of
// registers; applying it to two copies of x leaves x of lane l%32 in one
// result and x of lane 32 + l%32 in the other, in every lane.
__device__ __forceinline__ float halves_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// x from another lane of the same row of 16, by a DPP control (quad_perm,
// row mirrors): all rows and banks enabled, every lane has a source.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  const int v = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16 bytes per lane from global memory straight into LDS (buffer_load ...
// lds): lane l of the wave writes lds_base + 16*l.  The source is the raw
// buffer [base, base + nbytes); a lane whose offset lies past nbytes reads
// zeros, which are written to LDS like any other data.  The resource is built
// here, in a device-only helper, so that kernels using it keep a host stub.
__device__ __forceinline__ void load_lds_16(const void* base, uint32_t nbytes, void* lds_base,
                                            uint32_t offset) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_base, 16, offset, 0, 0, 0);
}

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): words 0 and 2 are multiplied by
// the round constants, the high halves are mixed with words 1 and 3 and the
// key, and the key advances by the Weyl increments between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    // three-input exclusive or in one instruction (v_bitop3_b32, truth table
    // 0x96 = a ^ b ^ c)
    const uint32_t w0 = (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
    const uint32_t w2 = (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
    c = u32x4{w0, (uint32_t)p1, w2, (uint32_t)p0};
  }
  return c;
}

// 16 bytes per lane from the raw buffer [base, base + nbytes) into registers
// (buffer_load_dwordx4): a lane whose offset lies past nbytes reads zeros,
// so a tile's rows beyond a length need no branch.  nbytes and offsets are
// multiples of 16, so an access is wholly inside or wholly outside.
__device__ __forceinline__ u32x4 load_ranged_16(const void* base, uint32_t nbytes,
                                                uint32_t offset) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, offset, 0, 0));
}

// Transpose read of 4 bf16 (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane r supplies an 8-byte address; lane i receives element i % 4 of
// the chunks addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12, in that
// order.  With lane r pointing at row r/4, columns 4*(r%4) .. +3 of a
// 4 x 16 block, lane i therefore receives column i of rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// The same transpose read issued as an instruction the compiler does not
// track: it inserts no wait for it (in particular no wait for unrelated
// buffer->LDS loads still in flight, which it cannot tell apart), and the
// caller must wait for the result with lds_wait before using it.
template <int OFFSET>
__device__ __forceinline__ bf16x4 lds_read_tr16_async(uint32_t addr) {
  static_assert(OFFSET >= 0 && OFFSET < 65536 && OFFSET % 8 == 0, "ds offset field");
  bf16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET));
  return r;
}

// LDS byte address of a pointer into the workgroup's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// 16-byte LDS read (ds_read_b128) at addr + OFFSET, untracked like the
// transpose read above: wait for it with lds_wait before use.  addr must be
// 16-byte aligned.
template <int OFFSET>
__device__ __forceinline__ bf16x8 lds_read_b128_async(uint32_t addr) {
  static_assert(OFFSET >= 0 && OFFSET < 65536 && OFFSET % 16 == 0, "ds offset field");
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET));
  return r;
}

// Wait until at most N of this wave's LDS operations are outstanding (they
// complete in order).  The values are passed through the wait, so
// everything the compiler schedules after it that uses them sees them
// complete.
template <int N>
__device__ __forceinline__ void lds_wait8(bf16x4 (&v)[8]) {
  static_assert(N >= 0 && N < 16, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7])
               : "i"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait4(bf16x8 (&v)[4]) {
  static_assert(N >= 0 && N < 16, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) : "i"(N));
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so that the
// body can use I as a compile-time constant (for instruction immediates).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier without a memory fence.  The caller makes its own
// memory operations complete (with the waits above) before arriving; the
// fence __syncthreads() adds would also wait for prefetches that are meant
// to stay in flight across the barrier.  The scheduling barriers keep the
// compiler from moving any instruction (MFMAs included, which the memory
// clobber does not hold) across it.
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most N of this wave's vector-memory operations (loads,
// including buffer->LDS loads) are in flight; they complete in issue order.
template <int N>
__device__ __forceinline__ void vmem_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

}  // namespace fa
