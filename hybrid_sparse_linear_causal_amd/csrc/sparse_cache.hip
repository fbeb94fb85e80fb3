// Sparse-layer KV cache maintenance: append (QK-norm of the new keys, cache write) and block
// pooling (mean key of each complete 64-token block).
//
// Pages: "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍", section
// "SALA混合架构：黄金配比破解瓶颈" — the sparse layers (InfLLM-V2) select key blocks per query
// and keep no positional encoding, so cached keys are position-free; "MiniCPM-SALA：融合稀疏与线性
// 注意力实现高效长上下文建模" §1 — sparse attention still keeps the full KV cache. The pooled
// (mean) key per block is the block representative the selection scores against.
#include "common.hpp"
#include "kv_append.hpp"
#include "launch.hpp"

namespace sala {

SparseGeom sparse_geom(const sala_sparse_desc& d) {
  SparseGeom g;
  g.q0 = d.kv_len - d.n_q;
  g.qb0 = g.q0 / 64;
  g.nqb = (d.kv_len - 1) / 64 - g.qb0 + 1;
  g.nblk_cap = d.kv_capacity / 64;
  g.scale = d.scale > 0.f ? d.scale : (float)(1.0 / sqrt((double)d.head_dim));
  return g;
}

namespace {

// grid (B*Hkv, blocks touched by the new tokens); 256 threads
template <typename T, int DD>
__global__ void __launch_bounds__(256)
kv_append_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                 const float* __restrict__ kw, T* __restrict__ k_cache, T* __restrict__ v_cache,
                 float* __restrict__ k_pool, int n_q, int Hkv, long kv_len, long cap, float eps,
                 const int64_t* __restrict__ kv_lens) {
  __shared__ float psum[RowGeom<T, DD>::RPP][DD];
  append_block<T, DD>(k_new, v_new, kw, k_cache, v_cache, k_pool, n_q, Hkv, kv_len, cap, eps, kv_lens, blockIdx.x,
                      blockIdx.y, psum);
}

// grid (B*Hkv, blk_end - blk_begin); mean of the 64 cached keys of each block
template <typename T, int DD>
__global__ void __launch_bounds__(256)
kv_pool_kernel(const T* __restrict__ k_cache, float* __restrict__ k_pool, int Hkv, long cap,
               long blk_begin) {
  using G = RowGeom<T, DD>;
  constexpr int EPL = G::EPL, LPR = G::LPR, RPP = G::RPP;
  __shared__ float psum[RPP][DD];
  const int bg = blockIdx.x;
  const long blk = blk_begin + blockIdx.y;
  const int j = threadIdx.x, r = j / LPR, seg = j % LPR;
  const long row_base = (long)bg * cap;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int t = r; t < 64; t += RPP) {
    float x[EPL];
    load_row_part<T>(k_cache + (row_base + blk * 64 + t) * DD + seg * EPL, x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) psum[r][seg * EPL + e] = acc[e];
  __syncthreads();
  for (int dd = j; dd < DD; dd += 256) {
    float s = 0.f;
    for (int rr = 0; rr < RPP; ++rr) s += psum[rr][dd];
    k_pool[((long)bg * (cap / 64) + blk) * DD + dd] = s * (1.0f / 64.0f);
  }
}

}  // namespace

hipError_t launch_kv_append(const sala_sparse_desc& d, const void* k_new, const void* v_new,
                            const float* kw, void* k_cache, void* v_cache, float* k_pool,
                            hipStream_t st, const int64_t* kv_lens) {
  const long q0 = d.kv_len - d.n_q;
  const long nblk = (d.kv_len - 1) / 64 - q0 / 64 + 1;
  const dim3 grid(d.batch * d.n_kv_heads, (unsigned)nblk);
#define SALA_APPEND(T, DD)                                                                        \
  hipLaunchKernelGGL((kv_append_kernel<T, DD>), grid, dim3(256), 0, st, (const T*)k_new,          \
                     (const T*)v_new, kw, (T*)k_cache, (T*)v_cache, k_pool, d.n_q, d.n_kv_heads,  \
                     (long)d.kv_len, (long)d.kv_capacity, d.norm_eps, kv_lens)
  if (d.dtype == SALA_BF16) {
    if (d.head_dim == 128) SALA_APPEND(bf16_t, 128); else SALA_APPEND(bf16_t, 64);
  } else {
    if (d.head_dim == 128) SALA_APPEND(float, 128); else SALA_APPEND(float, 64);
  }
#undef SALA_APPEND
  return hipGetLastError();
}

hipError_t launch_kv_pool(const sala_sparse_desc& d, const void* k_cache, float* k_pool,
                          int64_t blk_begin, int64_t blk_end, hipStream_t st) {
  if (blk_end <= blk_begin) return hipSuccess;
  const dim3 grid(d.batch * d.n_kv_heads, (unsigned)(blk_end - blk_begin));
#define SALA_POOL(T, DD)                                                                          \
  hipLaunchKernelGGL((kv_pool_kernel<T, DD>), grid, dim3(256), 0, st, (const T*)k_cache, k_pool,  \
                     d.n_kv_heads, (long)d.kv_capacity, (long)blk_begin)
  if (d.dtype == SALA_BF16) {
    if (d.head_dim == 128) SALA_POOL(bf16_t, 128); else SALA_POOL(bf16_t, 64);
  } else {
    if (d.head_dim == 128) SALA_POOL(float, 128); else SALA_POOL(float, 64);
  }
#undef SALA_POOL
  return hipGetLastError();
}

}  // namespace sala
