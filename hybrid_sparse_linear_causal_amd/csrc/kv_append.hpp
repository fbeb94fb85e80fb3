// One block of the sparse-layer KV append (QK-norm of the new keys, cache write, the block's
// pooled key once complete), shared by the append kernel and the fused decode-step selection.
//
// Pages: "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍", section
// "SALA混合架构：黄金配比破解瓶颈" — the sparse layers keep no positional encoding, so cached keys
// are position-free, and the mean key of a block is the representative the selection scores;
// "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" opening summary — QK normalisation in
// every layer.
#pragma once

#include "common.hpp"

namespace sala {
namespace {

// Elements a lane moves per 16-byte access and lanes per head row.
template <typename T, int DD> struct RowGeom {
  static constexpr int EPL = 16 / (int)sizeof(T);
  static constexpr int LPR = DD / EPL;  // lanes per row (<= 64)
  static constexpr int RPP = 256 / LPR; // rows per 256-thread pass
};

template <typename T>
__device__ __forceinline__ void load_row_part(const T* p, float* f);
template <>
__device__ __forceinline__ void load_row_part<bf16_t>(const bf16_t* p, float* f) {
  unpack8(*reinterpret_cast<const uint4*>(p), f);
}
template <>
__device__ __forceinline__ void load_row_part<float>(const float* p, float* f) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
}
template <typename T>
__device__ __forceinline__ void store_row_part(T* p, const float* f);
template <>
__device__ __forceinline__ void store_row_part<bf16_t>(bf16_t* p, const float* f) {
  *reinterpret_cast<uint4*>(p) = pack8(f);
}
template <>
__device__ __forceinline__ void store_row_part<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

// The append of one (sequence b, KV group g) = bg and one 64-token block (the by-th block touched
// by the new tokens), by the 256 threads of a workgroup: QK-norm of the new keys, cache writes of
// keys and values, and the block's mean key once the block is complete. psum: RPP x DD floats of
// LDS. kv_lens (one token per sequence only): each sequence's own cache length, clamped to
// [1, kv_len].
template <typename T, int DD>
__device__ __forceinline__ void append_block(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                             const float* __restrict__ kw, T* __restrict__ k_cache,
                                             T* __restrict__ v_cache, float* __restrict__ k_pool, int n_q, int Hkv,
                                             long kv_len, long cap, float eps, const int64_t* __restrict__ kv_lens,
                                             int bg, int by, float (*psum)[DD]) {
  using G = RowGeom<T, DD>;
  constexpr int EPL = G::EPL, LPR = G::LPR, RPP = G::RPP;
  const int b = bg / Hkv, g = bg % Hkv;
  if (kv_lens) {
    const long kb = kv_lens[b];
    kv_len = kb < 1 ? 1 : (kb > kv_len ? kv_len : kb);
  }
  const long q0 = kv_len - n_q;
  const long blk = q0 / 64 + by;
  const int j = threadIdx.x, r = j / LPR, seg = j % LPR;
  const long row_base = ((long)b * Hkv + g) * cap;  // cache row of (b, g, position 0)
  constexpr int NIT = 64 / RPP;  // rows of the block per thread
  const bool completes = (blk + 1) * 64 <= kv_len;  // the block is full once these tokens are in
  // a block that completes is pooled: its cached rows are all loaded first (the rows that the
  // new tokens replace are read too, in bounds, and overwritten below), so that the loads
  // overlap instead of waiting one by one
  float xs[NIT][EPL];
  if (completes) {
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      load_row_part<T>(k_cache + (row_base + blk * 64 + r + it * RPP) * DD + seg * EPL, xs[it]);
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const long p = blk * 64 + r + it * RPP;
    if (p >= q0 && p < kv_len) {
      const long src = (((long)b * n_q + (p - q0)) * Hkv + g) * DD + seg * EPL;
      float x[EPL], vv[EPL];
      load_row_part<T>(k_new + src, x);
      load_row_part<T>(v_new + src, vv);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
      ss = group_sum<LPR>(ss);
      const float inv = 1.0f / sqrtf(ss / DD + eps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) xs[it][e] = x[e] * inv * (kw ? kw[seg * EPL + e] : 1.0f);
      store_row_part<T>(k_cache + (row_base + p) * DD + seg * EPL, xs[it]);
      store_row_part<T>(v_cache + (row_base + p) * DD + seg * EPL, vv);
    }
  }
  if (!completes) return;  // block still incomplete: nothing to pool (uniform)
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += xs[it][e];
#pragma unroll
  for (int e = 0; e < EPL; ++e) psum[r][seg * EPL + e] = acc[e];
  __syncthreads();
  for (int dd = j; dd < DD; dd += 256) {
    float s = 0.f;
    for (int rr = 0; rr < RPP; ++rr) s += psum[rr][dd];
    k_pool[(((long)b * Hkv + g) * (cap / 64) + blk) * DD + dd] = s * (1.0f / 64.0f);
  }
}


}  // namespace
}  // namespace sala
