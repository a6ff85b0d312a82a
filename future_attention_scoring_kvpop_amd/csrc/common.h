// common.h -- device helpers shared by the libkvpop HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvpop {

typedef uint16_t bf16_t;  // raw bf16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16 contiguous bytes (8 bf16) as an MFMA operand fragment.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void stg16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// 16-byte load with the non-temporal hint, for data that is streamed once
// (a plain read of HBM with it ran at 7.1 TB/s on MI355X against 6.3-6.4
// TB/s without).
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void stg16_nt(void* p, uint4 v) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t t;
  t.x = v.x;
  t.y = v.y;
  t.z = v.z;
  t.w = v.w;
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand fragments: lane l holds
// A[m = l%32][8*(l/32) .. +8) and B[8*(l/32) .. +8)[n = l%32]; the result
// register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Direct global -> LDS loads (no staging registers).  Lane i of the wave
// writes its bytes at lds_base + size * i; lds_base must be wave-uniform.
// Completion is tracked by the wave's vmcnt like any vector memory load.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// Raw buffer resource (gfx9 layout: 48-bit base, stride 0, num_records bytes,
// 32-bit data format) for a wave-uniform range; loads past num_records
// return zero without touching memory.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

}  // namespace kvpop
extern "C" __device__ void kvpop_raw_buffer_load_lds(kvpop::i32x4 rsrc,
                                                     __attribute__((address_space(3))) void* lds,
                                                     int size, int voffset, int soffset, int offset,
                                                     int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
namespace kvpop {

// Direct buffer -> LDS loads: lane i writes its bytes (zero past the
// range) at lds_base + size * i; lds_base must be wave-uniform; voff is the
// lane's byte offset in the range.
__device__ __forceinline__ void bdma16(i32x4 rsrc, uint32_t voff, void* lds_base) {
  kvpop_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_base, 16, (int)voff,
                            0, 0, 0);
}
__device__ __forceinline__ void bdma4(i32x4 rsrc, uint32_t voff, void* lds_base) {
  kvpop_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_base, 4, (int)voff,
                            0, 0, 0);
}

// Wait until at most N vector memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their "no wait" maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this wave's LDS (and scalar memory) operations have completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also drain the wave's in-flight prefetches); callers order LDS traffic
// with explicit waits.  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Blocks are dispatched round-robin over the 8 XCDs (block i runs on XCD
// i % 8).  Renumber so that each XCD receives one contiguous range of
// logical work items: neighbouring items then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = i & 7, j = i >> 3;
  return x * q + (x < r ? x : r) + j;
}

// Order-preserving map of fp32 onto uint32 for ranking: larger key = ranks
// first.  -0.0 and +0.0 share one key; every NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t rank_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace kvpop
