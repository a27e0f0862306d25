// Device-side helpers shared by the KDA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// bf16 is carried as its raw 16-bit pattern in memory.
struct bf16_t {
  uint16_t bits;
};

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA bf16 operand
typedef __attribute__((ext_vector_type(4))) float f32x4_t;      // 16x16 accumulator
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
__device__ __forceinline__ float to_f32(float x) { return x; }

// Two bf16 packed in one dword -> floats (low half is the lower address).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 (compiles to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = static_cast<__bf16>(lo);
  r[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ bf16_t from(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return bf16_t{__builtin_bit_cast(uint16_t, h)};
  }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float from(float x) { return x; }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// Gate and normalisation prologue constants: the retention factor's lower bound
// e^-5 (log-decay >= -5) and the epsilon inside the L2 norm of q and k.
constexpr float kMinRetention = 0.006737946999085467f;
constexpr float kNormEps = 1e-6f;

}  // namespace kda

namespace kda {

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;

// Raw buffer resource over [base, base + bytes): loads past the end return 0 and
// stores past the end are dropped, which handles ragged tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ uint16_t buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
__device__ __forceinline__ i32x2_t buf_ld64(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
__device__ __forceinline__ i32x4_t buf_ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st32(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(v), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st64(i32x2_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st128(i32x4_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}

// Stores with the non-temporal hint: for data this kernel does not read again
// (streamed past the caches, which keeps HBM writes at full rate).
__device__ __forceinline__ void buf_st64_nt(i32x2_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 2);
}
__device__ __forceinline__ void buf_st128_nt(i32x4_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 2);
}

}  // namespace kda
