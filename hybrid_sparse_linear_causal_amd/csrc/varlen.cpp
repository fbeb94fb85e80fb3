// Packed variable-length batches for the KV append: the calls run sequence by sequence on the
// stream (each a one-sequence call with the sequence's own cache row and cache length). The
// append is a few percent of the sparse layer; the selection (block_select.hip), the attention
// and the linear prefill run the sequences' heavy passes in single launches.
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

}  // namespace sala
