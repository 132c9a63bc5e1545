// Shared device/host helpers of the kvx HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvx.h"

namespace kvx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 bits
// bf16 values are carried as raw uint16 bit patterns outside the MFMA
// operands, so every conversion below is explicit and rounds to nearest even.

__device__ __host__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  // NaN stays NaN (quiet bit set); finite values and infinities round to
  // nearest, ties to even.
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two bf16 of a packed dword (low half = first element).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16_rne(a)) | (static_cast<uint32_t>(f32_to_bf16_rne(b)) << 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = static_cast<_Float16>(f);  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return static_cast<uint32_t>(f32_to_f16_bits(a)) | (static_cast<uint32_t>(f32_to_f16_bits(b)) << 16);
}

// ---------------------------------------------------------------- direct loads, waits

typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer resource over [base, base + bytes) for raw 32-bit loads (word 3 as
// for gfx9 raw buffers); loads past the end return zero without a memory
// access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane from the buffer at voffset + soffset (per-lane and
// uniform byte offsets) straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding:
// vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14).
#define KVX_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | 0x70 | 0xF00)
#define KVX_COMPILER_FENCE() asm volatile("" ::: "memory")
// s_waitcnt lgkmcnt(0): this wave's LDS writes are complete (a barrier alone
// does not wait for them).
#define KVX_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Two fp32 -> packed bf16 (hardware convert, round to nearest even).
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// Two fp32 -> packed fp16 (hardware convert, round to nearest even).
__device__ __forceinline__ uint32_t cvt_f16x2(float a, float b) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), f16x2_t));
}

// Wave index inside the workgroup as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------- launch check

#define KVX_HIP_TRY(expr)                                        \
  do {                                                           \
    hipError_t _e = (expr);                                      \
    if (_e != hipSuccess) return KVX_ERR_HIP;                    \
  } while (0)

#define KVX_LAUNCH_CHECK()                                       \
  do {                                                           \
    hipError_t _e = hipGetLastError();                           \
    if (_e != hipSuccess) return KVX_ERR_HIP;                    \
  } while (0)

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bump allocator over a caller workspace (256-byte aligned slices).
struct Carve {
  char* base;
  size_t used;
  explicit Carve(void* p) : base(static_cast<char*>(p)), used(0) {}
  template <typename T>
  T* take(size_t count) {
    used = align_up(used, 256);
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

}  // namespace kvx
