// Device-side helpers shared by the gfx950 kernels of libvdit_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;

// Workgroups are dealt round-robin to the 8 XCDs of an MI355X (block i runs
// on XCD i % 8).  Renumber them so that each XCD receives one contiguous
// range of logical tiles: tiles of one head then share that XCD's L2 while
// they stream the same K/V tiles.  Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int x = bid % kXcd;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  return x * q + min(x, r) + bid / kXcd;
}

__device__ __forceinline__ f32x16 mfma32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32, nearest even
  return __builtin_bit_cast(uint32_t, r);
}

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1))
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ lds_void* lds_ptr(void* p) { return (lds_void*)p; }

// A pointer that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// global_load_lds_dwordx4 written out: 16 bytes per lane from gbase + voff
// to LDS address m0 + 16 * lane.  Issued through asm so that the compiler
// does not track the LDS write (it cannot tell the K/V buffers apart and
// would wait for every DMA before each LDS read); the kernel waits for these
// loads itself (s_waitcnt vmcnt + s_barrier) before any wave reads the
// buffer.  M0 is saved and restored around the load.
__device__ __forceinline__ void dma16(const char* gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(uniform_ptr(gbase))
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)p);
}

// max(a, b, c) as one v_max3_f32.  Written as asm because in IEEE mode the
// compiler first quiets every operand it cannot prove canonical (an MFMA
// result, say) with a v_max of its own; the scores here are never NaN.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// maximum of the 32 values of two 16-register score blocks: 16 v_max3_f32
__device__ __forceinline__ float max_of_32(const f32x16& a, const f32x16& b) {
  float m[12];
#pragma unroll
  for (int i = 0; i < 5; ++i) m[i] = max3_raw(a[3 * i], a[3 * i + 1], a[3 * i + 2]);
  m[5] = max3_raw(a[15], b[0], b[1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) m[6 + i] = max3_raw(b[2 + 3 * i], b[3 + 3 * i], b[4 + 3 * i]);
  m[10] = b[14];
  m[11] = b[15];
  const float r0 = max3_raw(m[0], m[1], m[2]), r1 = max3_raw(m[3], m[4], m[5]);
  const float r2 = max3_raw(m[6], m[7], m[8]), r3 = max3_raw(m[9], m[10], m[11]);
  return max3_raw(max3_raw(r0, r1, r2), r3, r3);
}

// max / sum of the values held by lanes l and l ^ 32
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace vdit
