// Shared device helpers for the gfx950 kernels of libmhe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhe {

typedef uint16_t bf16_t;  // bfloat16 bits

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Round-to-nearest-even float -> bf16 with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32; bit-identical to RNE on every finite input).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 held in a 16-byte vector into floats.
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// Eight floats times `factor`, clamped to +-448 and converted to E4M3 codes
// (v_cvt_pk_fp8_f32: round to nearest even, OCP "fn" format), as 8 bytes in
// element order. The product is a plain fp32 multiply (no fusion).
__device__ __forceinline__ u32x2 e4m3x8(const float* f, float factor) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(__fmul_rn(f[i], factor), -448.f), 448.f);
  u32x2 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h], y[4 * h + 1], 0, false));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2], y[4 * h + 3], 0, false));
    o[h] = (lo & 0xffffu) | (hi << 16);
  }
  return o;
}

// The same for eight bf16 values held in a 16-byte vector.
__device__ __forceinline__ u32x2 e4m3x8(const u32x4& v, float factor) {
  float f[8];
  unpack8(v, f);
  return e4m3x8(f, factor);
}

// Sum over the 64 lanes of a wavefront (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = WIDTH / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace mhe
