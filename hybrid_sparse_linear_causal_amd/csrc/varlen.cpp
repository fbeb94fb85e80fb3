// Packed variable-length batches for the KV append and the block selection: the calls run
// sequence by sequence on the stream (each a one-sequence call with the sequence's own cache
// row, cache length and query blocks), with one shared workspace. These two steps are a few
// percent of the sparse layer; the attention and the linear prefill, where the time goes, run
// every sequence in one launch (sparse_attn.hip, linear.hip).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.hpp"

namespace sala {

namespace {

size_t elem_bytes(const sala_sparse_desc& d) { return d.dtype == SALA_BF16 ? 2 : 4; }

// the one-sequence shape of sequence s: its tokens are the queries, its cache holds pos0 + n
sala_sparse_desc seq_desc(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0, int s) {
  sala_sparse_desc x = d;
  x.batch = 1;
  x.n_q = cu[s + 1] - cu[s];
  x.kv_len = pos0[s] + x.n_q;
  return x;
}

}  // namespace

size_t block_select_varlen_workspace(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0) {
  size_t need = 0;
  for (int s = 0; s < d.batch; ++s)
    if (cu[s + 1] > cu[s]) need = std::max(need, block_select_workspace(seq_desc(d, cu, pos0, s)));
  return need;
}

hipError_t launch_kv_append_varlen(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0,
                                   const void* k_new, const void* v_new, const float* kw, void* k_cache,
                                   void* v_cache, float* k_pool, hipStream_t st) {
  const size_t eb = elem_bytes(d), row = (size_t)d.n_kv_heads * d.head_dim;
  const size_t cache_seq = row * d.kv_capacity, pool_seq = row * (d.kv_capacity / 64);
  for (int s = 0; s < d.batch; ++s) {
    if (cu[s + 1] == cu[s]) continue;
    const size_t tok = (size_t)cu[s] * row * eb;
    const hipError_t e = launch_kv_append(
        seq_desc(d, cu, pos0, s), static_cast<const char*>(k_new) + tok, static_cast<const char*>(v_new) + tok, kw,
        static_cast<char*>(k_cache) + s * cache_seq * eb, static_cast<char*>(v_cache) + s * cache_seq * eb,
        k_pool + s * pool_seq, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_block_select_varlen(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0,
                                      const void* q, const float* qw, const float* k_pool, int32_t* sel, void* ws,
                                      hipStream_t st) {
  const size_t eb = elem_bytes(d), qrow = (size_t)d.n_heads * d.head_dim;
  const size_t pool_seq = (size_t)d.n_kv_heads * d.head_dim * (d.kv_capacity / 64);
  int64_t qb_row = 0;  // query blocks of the earlier sequences
  for (int s = 0; s < d.batch; ++s) {
    const int n = cu[s + 1] - cu[s];
    if (n == 0) continue;
    const hipError_t e =
        launch_block_select(seq_desc(d, cu, pos0, s), static_cast<const char*>(q) + (size_t)cu[s] * qrow * eb, qw,
                            k_pool + s * pool_seq, sel + qb_row * d.n_kv_heads * d.topk, nullptr, ws, st);
    if (e != hipSuccess) return e;
    qb_row += (n + 63) / 64;
  }
  return hipSuccess;
}

}  // namespace sala
