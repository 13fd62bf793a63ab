// Device-side building blocks shared by the msgl kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msgl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32 by bit manipulation (bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (low half = lo), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 16-byte global load/store through plain vector types (global_load_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16x16x32 bf16 MFMA.  Operand lane layout (l = lane):
//   A (16 x 32): row l % 16, eight k values selected by (l / 16, element)
//   B (32 x 16): col l % 16, the same eight k values for the same (l / 16, e)
//   C (16 x 16): col l % 16, rows 4 * (l / 16) + i for i = 0..3
// Only the A/B agreement on k matters for a contraction, so callers are free
// to choose which physical k each (l / 16, element) pair stands for.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA.  A (32 x 16): row l % 32, eight k values by (l / 32, e);
// B (16 x 32): col l % 32, same k by (l / 32, e);
// C (32 x 32): col l % 32, rows 8 * (i / 4) + 4 * (l / 32) + (i % 4), i = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Cross-lane exchange within a wave via ds_bpermute (LDS crossbar, no LDS
// memory traffic).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  int src = lane ^ mask;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// max(v, v of lane l ^ 32) without the LDS crossbar: v_permlane32_swap of
// (v, v) exchanges the lower half-wave of one copy with the upper half-wave
// of the other, so in every lane the two results are v itself and the value
// of lane l ^ 32 (which of the two comes first depends on the half).
__device__ __forceinline__ float max_xor32(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(v, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// The same over lane pairs l, l ^ 16: v_permlane16_swap exchanges the odd
// 16-lane rows of one copy with the even rows of the other.
__device__ __forceinline__ float max_xor16(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return fmaxf(v, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i
// receives element i % 4 of the 8-byte rows addressed by lanes 4k + i / 4
// (k = 0..3), i.e. a 16x4 block of 16-bit values comes back transposed.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// s_waitcnt with only the vector-memory counter constrained (<= n).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(n) : "memory");
}

// Direct global -> LDS loads, issued from inline assembly so the compiler
// neither tracks them nor inserts waits for them: callers order them with
// explicit vmcnt waits (vector-memory loads complete in order).
// Each wave instruction fills LDS at the wave-uniform base, lane l at
// +size*l.
// (The base must be the same in every lane and known so to the compiler: it
// goes into a scalar register.)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// m0 (the LDS base of these loads) is saved and restored around them, so the
// compiler's view of it never changes.
__device__ __forceinline__ void dma16(const void* src, const void* lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_addr(lds_base)) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, const void* lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_addr(lds_base)) : "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace msgl
