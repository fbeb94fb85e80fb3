// Internal launcher declarations shared by the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sala.h"

namespace sala {

typedef uint16_t bf16_t;

// RoPE frequencies in revolutions per position, f_i = base^(-2i/d) / (2 pi), i < d/2,
// computed on the host in double precision and passed by value to the kernels.
// c64/s64: cos and sin of the rotation by 64 positions (64 * theta_i), used to advance a
// table of angles from one 64-token chunk to the next.
struct RopeFreqs {
  double f[64];
  float c64[64], s64[64];
};

inline RopeFreqs make_rope_freqs(int d, float base) {
  RopeFreqs r;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < 64; ++i) {
    const double theta = (i < d / 2) ? pow((double)base, -2.0 * i / d) : 0.0;
    r.f[i] = theta / two_pi;
    r.c64[i] = (float)cos(fmod(64.0 * theta, two_pi));
    r.s64[i] = (float)sin(fmod(64.0 * theta, two_pi));
  }
  return r;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// ---- linear layer
// linear segment length (forward and backward): B*H*N / target_wgs rounded up to a power of two
// in [64, max_seg]
int linear_segment_len(const sala_linear_desc& d, int target_wgs = 512, int max_seg = 8192);
size_t linear_prefill_workspace(const sala_linear_desc& d);
hipError_t launch_linear_prefill(const sala_linear_desc& d, const void* q, const void* k,
                                 const void* v, const void* g, const float* qw, const float* kw,
                                 const float* state_in, float* state_out, void* out, void* ws,
                                 hipStream_t st);
size_t linear_prefill_varlen_workspace(const sala_linear_desc& d, const int32_t* cu_seqlens);
hipError_t launch_linear_prefill_varlen(const sala_linear_desc& d, const int32_t* cu_seqlens, const int64_t* pos0,
                                        const void* q, const void* k, const void* v, const void* g,
                                        const float* qw, const float* kw, const float* state_in,
                                        float* state_out, void* out, void* ws, hipStream_t st);
hipError_t launch_linear_decode(const sala_linear_desc& d, const void* q, const void* k,
                                const void* v, const void* g, const float* qw, const float* kw,
                                float* state, void* out, const int64_t* pos_b, hipStream_t st);
size_t linear_backward_workspace(const sala_linear_desc& d);
hipError_t launch_linear_backward(const sala_linear_desc& d, const void* q, const void* k, const void* v,
                                  const void* g, const float* qw, const float* kw, const float* state_in,
                                  const void* dout, const float* dstate_out, float* dq, float* dk, float* dv,
                                  float* dg, float* dqw, float* dkw, float* dstate_in, void* ws, hipStream_t st);

// ---- sparse layer
struct SparseGeom {
  int64_t q0;       // position of the first query token
  int64_t qb0;      // first query block
  int64_t nqb;      // query blocks covered by the call
  int64_t nblk_cap; // pooled-key rows per (b, g) = kv_capacity / 64
  float scale;      // resolved softmax scale
};
SparseGeom sparse_geom(const sala_sparse_desc& d);

// kv_lens (device, [B], one appended token per sequence): per-sequence cache lengths
hipError_t launch_kv_append(const sala_sparse_desc& d, const void* k_new, const void* v_new,
                            const float* kw, void* k_cache, void* v_cache, float* k_pool,
                            hipStream_t st, const int64_t* kv_lens = nullptr);
hipError_t launch_kv_pool(const sala_sparse_desc& d, const void* k_cache, float* k_pool,
                          int64_t blk_begin, int64_t blk_end, hipStream_t st);
size_t block_select_workspace(const sala_sparse_desc& d);
hipError_t launch_block_select(const sala_sparse_desc& d, const void* q, const float* qw,
                               const float* k_pool, int32_t* sel, float* sel_sc, void* ws, hipStream_t st);
size_t sparse_attn_workspace(const sala_sparse_desc& d);
// decode with each sequence at its own cache length (kv_lens: device [B] int64)
size_t block_select_decode_at_workspace(const sala_sparse_desc& d);  // SIZE_MAX: context too long
// the one-token append that the decode step runs inside the selection's first kernel
struct DecodeAppendPtrs {
  const void* k_new;
  const void* v_new;
  const float* kw;
  void* k_cache;
  void* v_cache;
  float* k_pool;
};
// app: also append (bf16, d = 128)
hipError_t launch_block_select_decode_at(const sala_sparse_desc& d, const int64_t* kv_lens, const void* q,
                                         const float* qw, const float* k_pool, int32_t* sel, void* ws,
                                         hipStream_t st, const DecodeAppendPtrs* app = nullptr);
size_t sparse_decode_at_workspace(const sala_sparse_desc& d);
hipError_t launch_sparse_decode_at(const sala_sparse_desc& d, const int64_t* kv_lens, const void* q, const float* qw,
                                   const void* k_cache, const void* v_cache, const void* g, const int32_t* sel,
                                   void* out, void* ws, hipStream_t st);
// packed variable-length batches (desc.batch = sequences, cu_seqlens / pos0 on the host)
int64_t varlen_query_blocks(int nseq, const int32_t* cu_seqlens);
size_t block_select_varlen_workspace(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0);
hipError_t launch_kv_append_varlen(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0,
                                   const void* k_new, const void* v_new, const float* kw, void* k_cache,
                                   void* v_cache, float* k_pool, hipStream_t st);
hipError_t launch_block_select_varlen(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0,
                                      const void* q, const float* qw, const float* k_pool, int32_t* sel, void* ws,
                                      hipStream_t st);
hipError_t launch_sparse_attn_varlen(const sala_sparse_desc& d, const int32_t* cu_seqlens, const int64_t* pos0,
                                     const void* q, const float* qw, const void* k_cache, const void* v_cache,
                                     const void* g, const int32_t* sel, void* out, hipStream_t st);
hipError_t launch_sparse_attn(const sala_sparse_desc& d, const void* q, const float* qw,
                              const void* k_cache, const void* v_cache, const void* g,
                              const int32_t* sel, void* out, float* lse, void* ws, hipStream_t st);
size_t sparse_attn_backward_workspace(const sala_sparse_desc& d);
hipError_t launch_sparse_attn_backward(const sala_sparse_desc& d, const void* q, const float* qw, const void* k_cache,
                                       const void* v_cache, const void* g, const int32_t* sel, const void* dout,
                                       const void* out, const float* lse, float* dq, float* dk_cache, float* dv_cache,
                                       float* dg, float* dqw, void* ws, hipStream_t st);
size_t kv_norm_backward_workspace(const sala_sparse_desc& d);
hipError_t launch_kv_norm_backward(const sala_sparse_desc& d, const void* k_new, const float* kw,
                                   const float* dk_cache, float* dk_new, float* dkw, void* ws, hipStream_t st);
// dense causal attention over every cached block up to the query's own (no selection)
hipError_t launch_dense_attn(const sala_sparse_desc& d, const void* q, const float* qw,
                             const void* k_cache, const void* v_cache, const void* g, void* out,
                             void* ws, hipStream_t st);

}  // namespace sala
