// Shared device helpers for the gfx950 kernels: bf16 packing, MFMA wrappers, wave reductions.
//
// MFMA lane layouts used throughout (wave64, checked on gfx950 with exact integer data):
//   v_mfma_f32_16x16x32_bf16  C[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[l%16][8*(l/16) + e], e = 0..7      (8 bf16 = 4 VGPRs)
//     B: lane l holds B[8*(l/16) + e][l%16], e = 0..7
//     C: lane l holds C[4*(l/16) + e][l%16], e = 0..3
// Any permutation of the reduction index k applied to A and B alike leaves C unchanged; the
// attention kernels use that to feed the probabilities produced in C layout straight back in
// as an operand without moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sala {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // bf16 bits as stored in memory

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// round-to-nearest-even conversion (hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ bf16_t f2bf(float x) {
  __bf16 a = (__bf16)x;
  return __builtin_bit_cast(uint16_t, a);
}

// unpack 8 bf16 held in a uint4 into floats
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]); u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]); u.w = pack_bf16x2(f[6], f[7]);
  return u;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 as_bf16x8(const uint2& a, const uint2& b) {
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// butterfly reductions over lane groups (width = power of two <= 64)
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// logistic function for the output gate
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// sin and cos of 2*pi*rev for rev in [-0.5, 0.5] (hardware v_sin_f32 / v_cos_f32 take revolutions)
__device__ __forceinline__ void sincos_rev(float rev, float* s, float* c) {
  *s = __builtin_amdgcn_sinf(rev);
  *c = __builtin_amdgcn_cosf(rev);
}

// RoPE angle of frequency f (in revolutions per position) at position p, reduced to [-0.5, 0.5]
// revolutions in fp64 so positions up to 2^40 keep full fp32 accuracy after reduction.
__device__ __forceinline__ float rope_rev(double pos, double f) {
  double r = pos * f;
  r -= rint(r);
  return (float)r;
}

// monotone uint32 key of a float score (larger score -> larger key; -0.0 maps like +0.0)
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == 0.0f) s = 0.0f;
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace sala
