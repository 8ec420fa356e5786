// Shared device-side helpers of the gfx950 SSD kernels: vector types, bf16
// conversions, MFMA wrappers and the LDS transpose read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// log2(e) rounded to float32: the cumulative sums are stored in log2 units so
// that every consumer evaluates its decays with the hardware's native 2^x.
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Operand layout (checked on gfx950): lane l holds A row (l & 15) and B
// column (l & 15), with K elements 8*(l >> 4) .. 8*(l >> 4) + 7 in vector
// order; the accumulator lane l holds column (l & 15), rows 4*(l >> 4) + r.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 LDS transpose read.  Within each 16-lane group, lane L supplies the
// address of 4 consecutive 16-bit elements; lane i receives element e from
// the chunk of lane 4*e + i/4, position i%4.  If lane L points at
// M[k0 + L/4][c(L%4) .. c(L%4)+3] of a row-major matrix M, lane i = 4q + s
// receives M[k0 + e][c(q) + s] for e = 0..3: four consecutive rows of one
// column, i.e. an MFMA operand whose K runs along M's rows.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 16-byte direct-to-LDS load (global_load_lds_dwordx4): lane l's 16 bytes from
// `src` land at LDS byte address lds_base + 16 l; lds_base (an LDS byte
// address, see lds_addr) must be uniform across the wave.  Issued through
// inline asm so that the compiler does not see an LDS write it cannot
// disambiguate from later LDS reads of the other buffer (it would then wait
// for the load right away and undo the prefetch).  The caller owns the
// ordering: the issuing waves wait vmcnt(0), then a barrier, before any wave
// reads the destination.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const void* lds_ptr;
  return (uint32_t)(uintptr_t)(lds_ptr)(p);
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations (lgkmcnt 0), leaves its global loads, stores and direct-to-LDS
// loads in flight, then meets the other waves.  __syncthreads() would also
// wait for every outstanding global operation (vmcnt 0), which serialises a
// prefetch issued just before it.  Data brought in by direct-to-LDS loads is
// only safe to read after an explicit vmcnt wait by the issuing wave followed
// by a barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Waits until at most n of this wave's vector memory operations are
// outstanding (and its LDS operations are done).  n is wave-uniform.  Vector
// memory operations retire in issue order, so with n = the number of
// operations issued after a given load, that load has landed.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define M2_W(k) \
  case k: __builtin_amdgcn_s_waitcnt(0x0070 | ((k) & 15) | (((k) >> 4) << 14)); break;
    M2_W(0) M2_W(1) M2_W(2) M2_W(3) M2_W(4) M2_W(5) M2_W(6) M2_W(7) M2_W(8) M2_W(9)
    M2_W(10) M2_W(11) M2_W(12) M2_W(13) M2_W(14) M2_W(15) M2_W(16) M2_W(17) M2_W(18)
    M2_W(19) M2_W(20) M2_W(21) M2_W(22) M2_W(23) M2_W(24) M2_W(25) M2_W(26) M2_W(27)
    M2_W(28) M2_W(29) M2_W(30) M2_W(31) M2_W(32) M2_W(33) M2_W(34) M2_W(35) M2_W(36)
    M2_W(37) M2_W(38) M2_W(39) M2_W(40) M2_W(41) M2_W(42) M2_W(43) M2_W(44) M2_W(45)
    M2_W(46) M2_W(47) M2_W(48) M2_W(49) M2_W(50) M2_W(51) M2_W(52) M2_W(53) M2_W(54)
    M2_W(55) M2_W(56) M2_W(57) M2_W(58) M2_W(59) M2_W(60) M2_W(61) M2_W(62)
#undef M2_W
    default: __builtin_amdgcn_s_waitcnt(0x0070); break;  // vmcnt(0)
  }
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace m2
