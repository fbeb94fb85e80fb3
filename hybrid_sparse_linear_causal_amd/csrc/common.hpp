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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// round-to-nearest-even conversion of a pair: one v_cvt_pk_bf16_f32 on gfx950 (converting the
// two halves separately costs two conversions plus a shift and an OR)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
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

// Sum over aligned groups of 8 lanes with DPP (VALU-speed lane exchange, no LDS round trip):
// swap neighbours, swap pairs, then mirror within the 8-lane half-row.
__device__ __forceinline__ float group_sum8_dpp(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the last lane of row 0 (2) is added to row 1 (3), then lane 31 to rows 2
// and 3. Lanes whose DPP source does not exist receive 0. All 64 lanes must be active.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
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


// ---- LDS tiles of 256-byte rows (64 or 128 bf16): 16-byte chunk c of row r is stored at chunk
// position c ^ (r & 15), so 16 rows read at one column land in 16 different bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + 8 * (chunk ^ (row & 15)); }
// Layout of tiles that are also read transposed: chunk c of row r at position c ^ 2(r & 7). The
// transposing reads of 32 lanes (8 consecutive rows x 2 adjacent chunks) land on 16 different
// positions, and row reads of 16 rows at one chunk stay free of bank conflicts as well
// (measured with the LDS bank-conflict counter on gfx950); swz gives the transposing reads
// two-way conflicts.
__device__ __forceinline__ int swzv(int row, int chunk) { return row * 128 + 8 * (chunk ^ (2 * (row & 7))); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16 lanes, lane i
// supplies the address of 4 consecutive bf16; lane j receives element j%4 of the chunks of
// lanes j/4 + 4e, e = 0..3. With lane i pointing at row k0 + i/4, columns c0 + 4*(i%4), lane j
// receives column c0 + j of rows k0 .. k0+3: four consecutive-k values of one MFMA column.
__device__ __forceinline__ uint2 ds_read_tr(const bf16_t* p) {
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  return __builtin_bit_cast(uint2, r);
}
// MFMA operand "column j = c0 + l16, k = rows k0 + 0..7" of a row-major tile in the swzv
// layout, k0 and c0 multiples of 4: two transposing reads (rows k0..k0+3, then k0+d1..k0+d1+3).
// Free of bank conflicts when the lanes of each 32 cover 8 consecutive rows (k0 = kb + 4 * lq,
// d1 = 16).
__device__ __forceinline__ bf16x8 tr_frag_v(const bf16_t* T, int k0, int d1, int c0, int l16) {
  const int row = k0 + (l16 >> 2), col = c0 + 4 * (l16 & 3);
  const uint2 a = ds_read_tr(T + swzv(row, col >> 3) + (col & 7));
  const uint2 b = ds_read_tr(T + swzv(row + d1, col >> 3) + (col & 7));
  return as_bf16x8(a, b);
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4): lane l's
// chunk lands at LDS byte address lds_addr + 16 * l (lds_addr wave-uniform). Issued from inline
// assembly so that the compiler does not serialise it with unrelated LDS reads; it has no
// register outputs, and completion is awaited with wait_vmcnt before the barrier that
// publishes the data.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr)
               : "memory", "m0");
}
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_u32(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// logistic function from hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

}  // namespace sala
