// C ABI of libsala: argument validation (nothing is enqueued unless every check passes),
// workspace sizing and dispatch to the gfx950 kernels. The method, layouts and error rules of
// each entry point are documented in sala.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "launch.hpp"
#include "sala.h"

// Scratch memory of sala_sparse_decode_step_noalloc: one copy per device the library runs on,
// held until the process ends. Host code never uses this name as an address (on the host it is
// a stand-in symbol); it uses the device address looked up per device below.
static __device__ __align__(256) unsigned char scratch[SALA_NOALLOC_SCRATCH_BYTES];

namespace {

// per-device address of `scratch`, looked up once per device with that device current
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sala_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SALA_OK;
  g_last_hip_error = (int)e;
  return SALA_ERR_HIP;
}

sala_status check_linear(const sala_linear_desc* d) {
  if (!d) return SALA_ERR_NULL;
  if (d->batch < 1 || d->seq_len < 0 || d->n_heads < 1 || d->n_kv_heads < 1 || d->pos0 < 0)
    return SALA_ERR_INVALID;
  if (d->head_dim != 64 && d->head_dim != 128) return SALA_ERR_UNSUPPORTED;
  if (d->dtype != SALA_F32 && d->dtype != SALA_BF16) return SALA_ERR_INVALID;
  if (!(d->rope_base > 0.f) || !isfinite(d->rope_base)) return SALA_ERR_INVALID;
  if (!(d->norm_eps >= 0.f) || !isfinite(d->norm_eps)) return SALA_ERR_INVALID;
  if (d->n_heads % d->n_kv_heads != 0 || d->reserved_ != 0) return SALA_ERR_INVALID;
  if (d->n_heads / d->n_kv_heads > 64) return SALA_ERR_UNSUPPORTED;
  // the chunked evaluation is built for 64-token chunks; 128 and 256 are chunk sizes of the
  // method that are not built here
  if (d->chunk != 0 && d->chunk != 64) return (d->chunk == 128 || d->chunk == 256) ? SALA_ERR_UNSUPPORTED : SALA_ERR_INVALID;
  // sizes must stay within 64-bit element offsets and 32-bit grid dimensions
  const double elems = (double)d->batch * d->seq_len * d->n_heads * d->head_dim;
  if (elems > 9.0e15 || (double)d->batch * d->seq_len * d->n_heads > 2.0e9) return SALA_ERR_INVALID;
  return SALA_OK;
}

// with_sel: the call uses topk / n_local (selection, sparse attention); dense attention does not
sala_status check_sparse(const sala_sparse_desc* d, bool with_sel = true) {
  if (!d) return SALA_ERR_NULL;
  if (d->batch < 1 || d->n_q < 1 || d->n_heads < 1 || d->n_kv_heads < 1) return SALA_ERR_INVALID;
  if (d->n_heads % d->n_kv_heads != 0) return SALA_ERR_INVALID;
  if (d->head_dim != 64 && d->head_dim != 128) return SALA_ERR_UNSUPPORTED;
  if (d->dtype != SALA_F32 && d->dtype != SALA_BF16) return SALA_ERR_INVALID;
  if (d->block != 64) return SALA_ERR_UNSUPPORTED;
  if (with_sel && d->n_local != 1 && d->n_local != 2) return SALA_ERR_UNSUPPORTED;
  if (with_sel && (d->topk < 1 + d->n_local || d->topk > 256)) return SALA_ERR_INVALID;
  if (!(d->norm_eps >= 0.f) || !isfinite(d->norm_eps)) return SALA_ERR_INVALID;
  if (!(d->scale >= 0.f) || !isfinite(d->scale)) return SALA_ERR_INVALID;
  if (d->kv_len < d->n_q || d->kv_capacity < d->kv_len || d->kv_capacity % 64 != 0)
    return SALA_ERR_INVALID;
  if (d->n_q > 1 && (d->kv_len - d->n_q) % 64 != 0) return SALA_ERR_INVALID;
  if (d->n_heads > 64) return SALA_ERR_UNSUPPORTED;
  if ((double)d->batch * d->n_kv_heads * (d->kv_capacity / 64) > 2.0e9) return SALA_ERR_INVALID;
  return SALA_OK;
}

// a packed batch: nseq = desc batch sequences, cu_seqlens[0] = 0, nondecreasing, ending at the
// packed token count; positions >= 0 (and multiples of 64 with the cache row within capacity
// for the sparse layer)
sala_status check_varlen(int nseq, int64_t total, const int32_t* cu, const int64_t* pos0, int64_t cap) {
  if (!cu || !pos0) return SALA_ERR_NULL;
  if (nseq < 1) return SALA_ERR_INVALID;
  if (nseq > SALA_VARLEN_MAX_SEQS) return SALA_ERR_UNSUPPORTED;
  if (cu[0] != 0 || cu[nseq] != total) return SALA_ERR_INVALID;
  for (int s = 0; s < nseq; ++s) {
    if (cu[s + 1] < cu[s] || pos0[s] < 0) return SALA_ERR_INVALID;
    if (cap >= 0 && (pos0[s] % 64 != 0 || pos0[s] + (cu[s + 1] - cu[s]) > cap)) return SALA_ERR_INVALID;
  }
  return SALA_OK;
}

// the sparse shape fields of a packed batch: as check_sparse, with n_q = packed token count and
// kv_len unused (each sequence's cache holds pos0 + its token count)
sala_status check_sparse_varlen(const sala_sparse_desc* d, const int32_t* cu, const int64_t* pos0) {
  if (!d) return SALA_ERR_NULL;
  sala_sparse_desc x = *d;
  x.batch = 1;
  x.n_q = 1;
  x.kv_len = 1;
  const sala_status s = check_sparse(&x);
  if (s != SALA_OK) return s;
  if (d->n_q < 0) return SALA_ERR_INVALID;
  if (d->dtype != SALA_BF16 || d->head_dim != 128) return SALA_ERR_UNSUPPORTED;
  return check_varlen(d->batch, d->n_q, cu, pos0, d->kv_capacity);
}

sala_status check_linear_varlen(const sala_linear_desc* d, const int32_t* cu, const int64_t* pos0) {
  const sala_status s = check_linear(d);
  if (s != SALA_OK) return s;
  if (d->dtype != SALA_BF16 || d->head_dim != 128) return SALA_ERR_UNSUPPORTED;
  return check_varlen(d->batch, d->seq_len, cu, pos0, -1);
}

// the decode step of the sparse layer with per-sequence cache lengths: bf16, d = 128, one query
// token per sequence, group <= 16, contexts within the two-level selection range
sala_status check_sparse_decode_at(const sala_sparse_desc* d) {
  const sala_status s = check_sparse(d);
  if (s != SALA_OK) return s;
  if (d->n_q != 1) return SALA_ERR_INVALID;
  if (d->dtype != SALA_BF16 || d->head_dim != 128 || d->n_heads / d->n_kv_heads > 16) return SALA_ERR_UNSUPPORTED;
  if (sala::block_select_decode_at_workspace(*d) == SIZE_MAX) return SALA_ERR_UNSUPPORTED;
  return SALA_OK;
}

// the decode step's workspace: the selection's, then the attention's partials
size_t step_select_bytes(const sala_sparse_desc& d) {
  return (sala::block_select_decode_at_workspace(d) + 255) & ~(size_t)255;
}
size_t sparse_decode_step_workspace(const sala_sparse_desc& d) {
  return step_select_bytes(d) + sala::sparse_decode_at_workspace(d);
}

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}

}  // namespace

extern "C" {

int sala_abi_version(void) { return SALA_ABI_VERSION; }

int sala_last_hip_error(void) { return g_last_hip_error; }

const char* sala_status_str(sala_status s) {
  switch (s) {
    case SALA_OK: return "ok";
    case SALA_ERR_NULL: return "a required pointer is NULL";
    case SALA_ERR_INVALID: return "invalid sizes, parameters or alignment";
    case SALA_ERR_UNSUPPORTED: return "shape or dtype not supported by this library";
    case SALA_ERR_WORKSPACE: return "workspace missing or too small";
    case SALA_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

size_t sala_workspace_bytes(int op, const void* desc) {
  switch (op) {
    case SALA_OP_LINEAR_PREFILL: {
      const sala_linear_desc* d = static_cast<const sala_linear_desc*>(desc);
      if (check_linear(d) != SALA_OK) return SIZE_MAX;
      return sala::linear_prefill_workspace(*d);
    }
    case SALA_OP_BLOCK_SELECT: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse(d) != SALA_OK) return SIZE_MAX;
      return sala::block_select_workspace(*d);
    }
    case SALA_OP_SPARSE_ATTN: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse(d) != SALA_OK) return SIZE_MAX;
      return sala::sparse_attn_workspace(*d);
    }
    case SALA_OP_DENSE_ATTN: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse(d, false) != SALA_OK) return SIZE_MAX;
      return sala::sparse_attn_workspace(*d);
    }
    case SALA_OP_SPARSE_ATTN_BACKWARD: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse(d) != SALA_OK || d->dtype != SALA_BF16 || d->head_dim != 128 || d->n_q < 2)
        return SIZE_MAX;
      return sala::sparse_attn_backward_workspace(*d);
    }
    case SALA_OP_KV_NORM_BACKWARD: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse(d, false) != SALA_OK || d->dtype != SALA_BF16 || d->head_dim != 128) return SIZE_MAX;
      return sala::kv_norm_backward_workspace(*d);
    }
    case SALA_OP_SPARSE_DECODE_STEP: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse_decode_at(d) != SALA_OK) return SIZE_MAX;
      return sparse_decode_step_workspace(*d);
    }
    case SALA_OP_LINEAR_BACKWARD: {
      const sala_linear_desc* d = static_cast<const sala_linear_desc*>(desc);
      if (check_linear(d) != SALA_OK || d->dtype != SALA_BF16 || d->head_dim != 128 || d->n_kv_heads != d->n_heads)
        return SIZE_MAX;
      return sala::linear_backward_workspace(*d);
    }
    default: return SIZE_MAX;
  }
}

sala_status sala_linear_prefill(const sala_linear_desc* desc, const void* q, const void* k,
                                const void* v, const void* gate, const float* q_norm_w,
                                const float* k_norm_w, const float* state_in, float* state_out,
                                void* out, void* workspace, size_t workspace_bytes, void* stream) {
  sala_status s = check_linear(desc);
  if (s != SALA_OK) return s;
  const sala_linear_desc& d = *desc;
  if (d.dtype == SALA_BF16 && d.head_dim != 128) return SALA_ERR_UNSUPPORTED;
  if (d.seq_len > 0 && (!q || !k || !v || !gate || !out)) return SALA_ERR_NULL;
  if (!all_aligned({q, k, v, gate, out, q_norm_w, k_norm_w, state_in, state_out, workspace}))
    return SALA_ERR_INVALID;
  const size_t need = sala::linear_prefill_workspace(d);
  if (d.seq_len > 0 && need > 0 && (!workspace || workspace_bytes < need)) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_linear_prefill(d, q, k, v, gate, q_norm_w, k_norm_w, state_in,
                                                state_out, out, workspace, (hipStream_t)stream));
}

sala_status sala_linear_backward(const sala_linear_desc* desc, const void* q, const void* k,
                                 const void* v, const void* gate, const float* q_norm_w,
                                 const float* k_norm_w, const float* state_in, const void* dout,
                                 const float* dstate_out, float* dq, float* dk, float* dv,
                                 float* dg, float* dq_norm_w, float* dk_norm_w, float* dstate_in,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  sala_status s = check_linear(desc);
  if (s != SALA_OK) return s;
  const sala_linear_desc& d = *desc;
  if (d.dtype != SALA_BF16 || d.head_dim != 128 || d.n_kv_heads != d.n_heads) return SALA_ERR_UNSUPPORTED;
  if (d.seq_len > 0 && (!q || !k || !v || !gate || !dout || !dq || !dk || !dv || !dg)) return SALA_ERR_NULL;
  if (!all_aligned({q, k, v, gate, q_norm_w, k_norm_w, state_in, dout, dstate_out, dq, dk, dv, dg, dq_norm_w,
                    dk_norm_w, dstate_in, workspace}))
    return SALA_ERR_INVALID;
  const size_t need = sala::linear_backward_workspace(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_linear_backward(d, q, k, v, gate, q_norm_w, k_norm_w, state_in, dout,
                                                 dstate_out, dq, dk, dv, dg, dq_norm_w, dk_norm_w, dstate_in,
                                                 workspace, (hipStream_t)stream));
}

sala_status sala_linear_decode_step(const sala_linear_desc* desc, const void* q, const void* k,
                                    const void* v, const void* gate, const float* q_norm_w,
                                    const float* k_norm_w, float* state, void* out, void* stream) {
  sala_status s = check_linear(desc);
  if (s != SALA_OK) return s;
  if (desc->seq_len != 1) return SALA_ERR_INVALID;
  if (!q || !k || !v || !gate || !state || !out) return SALA_ERR_NULL;
  if (!all_aligned({q, k, v, gate, out, q_norm_w, k_norm_w, state})) return SALA_ERR_INVALID;
  return hip_status(sala::launch_linear_decode(*desc, q, k, v, gate, q_norm_w, k_norm_w, state, out, nullptr,
                                               (hipStream_t)stream));
}

sala_status sala_linear_decode_step_at(const sala_linear_desc* desc, const int64_t* pos, const void* q,
                                       const void* k, const void* v, const void* gate, const float* q_norm_w,
                                       const float* k_norm_w, float* state, void* out, void* stream) {
  sala_status s = check_linear(desc);
  if (s != SALA_OK) return s;
  if (desc->seq_len != 1) return SALA_ERR_INVALID;
  if (!pos || !q || !k || !v || !gate || !state || !out) return SALA_ERR_NULL;
  if (!all_aligned({q, k, v, gate, out, q_norm_w, k_norm_w, state}) || (reinterpret_cast<uintptr_t>(pos) & 7u))
    return SALA_ERR_INVALID;
  return hip_status(sala::launch_linear_decode(*desc, q, k, v, gate, q_norm_w, k_norm_w, state, out, pos,
                                               (hipStream_t)stream));
}

sala_status sala_sparse_decode_step(const sala_sparse_desc* desc, const int64_t* kv_lens, const void* q,
                                    const float* q_norm_w, const void* k_new, const void* v_new,
                                    const float* k_norm_w, const void* gate, void* k_cache, void* v_cache,
                                    float* k_pool, int32_t* sel, void* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const sala_status s = check_sparse_decode_at(desc);
  if (s != SALA_OK) return s;
  if (!kv_lens || !q || !k_new || !v_new || !gate || !k_cache || !v_cache || !k_pool || !sel || !out)
    return SALA_ERR_NULL;
  if (!all_aligned({q, q_norm_w, k_new, v_new, k_norm_w, gate, k_cache, v_cache, k_pool, sel, out, workspace}) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 7u))
    return SALA_ERR_INVALID;
  const size_t need = sparse_decode_step_workspace(*desc);
  if (!workspace || workspace_bytes < need) return SALA_ERR_WORKSPACE;
  const sala_sparse_desc& d = *desc;
  const hipStream_t st = (hipStream_t)stream;
  // the append rides in the selection's first kernel: it writes only the query's own block
  // (cache rows and pooled key), which is never a candidate
  char* ws = static_cast<char*>(workspace);
  const sala::DecodeAppendPtrs app{k_new, v_new, k_norm_w, k_cache, v_cache, k_pool};
  hipError_t e = sala::launch_block_select_decode_at(d, kv_lens, q, q_norm_w, k_pool, sel, ws, st, &app);
  if (e == hipSuccess)
    e = sala::launch_sparse_decode_at(d, kv_lens, q, q_norm_w, k_cache, v_cache, gate, sel, out,
                                      ws + step_select_bytes(d), st);
  return hip_status(e);
}

sala_status sala_sparse_decode_step_noalloc(const sala_sparse_desc* desc, const int64_t* kv_lens, const void* q,
                                            const float* q_norm_w, const void* k_new, const void* v_new,
                                            const float* k_norm_w, const void* gate, void* k_cache, void* v_cache,
                                            float* k_pool, int32_t* sel, void* out, void* stream) {
  const sala_status s = check_sparse_decode_at(desc);
  if (s != SALA_OK) return s;
  if (!kv_lens || !q || !k_new || !v_new || !gate || !k_cache || !v_cache || !k_pool || !sel || !out)
    return SALA_ERR_NULL;
  if (!all_aligned({q, q_norm_w, k_new, v_new, k_norm_w, gate, k_cache, v_cache, k_pool, sel, out}) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 7u))
    return SALA_ERR_INVALID;
  if (sparse_decode_step_workspace(*desc) > SALA_NOALLOC_SCRATCH_BYTES) return SALA_ERR_WORKSPACE;
  // the scratch copy of the device the work runs on: the stream's, which must be current
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return hip_status(e);
    if (sdev != dev) return SALA_ERR_INVALID;
  }
  void* ws = nullptr;
  e = scratch_address(dev, &ws);
  if (e != hipSuccess) return hip_status(e);
  return sala_sparse_decode_step(desc, kv_lens, q, q_norm_w, k_new, v_new, k_norm_w, gate, k_cache, v_cache, k_pool,
                                 sel, out, ws, SALA_NOALLOC_SCRATCH_BYTES, stream);
}

sala_status sala_kv_append(const sala_sparse_desc* desc, const void* k_new, const void* v_new,
                           const float* k_norm_w, void* k_cache, void* v_cache, float* k_pool,
                           void* stream) {
  sala_status s = check_sparse(desc);
  if (s != SALA_OK) return s;
  if (!k_new || !v_new || !k_cache || !v_cache || !k_pool) return SALA_ERR_NULL;
  if (!all_aligned({k_new, v_new, k_norm_w, k_cache, v_cache, k_pool})) return SALA_ERR_INVALID;
  return hip_status(sala::launch_kv_append(*desc, k_new, v_new, k_norm_w, k_cache, v_cache, k_pool,
                                           (hipStream_t)stream));
}

sala_status sala_linear_prefill_varlen(const sala_linear_desc* desc, const int32_t* cu_seqlens,
                                       const int64_t* pos0, const void* q, const void* k, const void* v,
                                       const void* gate, const float* q_norm_w, const float* k_norm_w,
                                       const float* state_in, float* state_out, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const sala_status s = check_linear_varlen(desc, cu_seqlens, pos0);
  if (s != SALA_OK) return s;
  const sala_linear_desc& d = *desc;
  if (d.seq_len > 0 && (!q || !k || !v || !gate || !out)) return SALA_ERR_NULL;
  if (!all_aligned({q, k, v, gate, out, q_norm_w, k_norm_w, state_in, state_out, workspace})) return SALA_ERR_INVALID;
  const size_t need = sala::linear_prefill_varlen_workspace(d, cu_seqlens);
  if (d.seq_len > 0 && need > 0 && (!workspace || workspace_bytes < need)) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_linear_prefill_varlen(d, cu_seqlens, pos0, q, k, v, gate, q_norm_w, k_norm_w,
                                                       state_in, state_out, out, workspace, (hipStream_t)stream));
}

sala_status sala_kv_append_varlen(const sala_sparse_desc* desc, const int32_t* cu_seqlens, const int64_t* pos0,
                                  const void* k_new, const void* v_new, const float* k_norm_w, void* k_cache,
                                  void* v_cache, float* k_pool, void* stream) {
  const sala_status s = check_sparse_varlen(desc, cu_seqlens, pos0);
  if (s != SALA_OK) return s;
  if (!k_cache || !v_cache || !k_pool || (desc->n_q > 0 && (!k_new || !v_new))) return SALA_ERR_NULL;
  if (!all_aligned({k_new, v_new, k_norm_w, k_cache, v_cache, k_pool})) return SALA_ERR_INVALID;
  return hip_status(sala::launch_kv_append_varlen(*desc, cu_seqlens, pos0, k_new, v_new, k_norm_w, k_cache, v_cache,
                                                  k_pool, (hipStream_t)stream));
}

sala_status sala_block_select_varlen(const sala_sparse_desc* desc, const int32_t* cu_seqlens, const int64_t* pos0,
                                     const void* q, const float* q_norm_w, const float* k_pool, int32_t* sel,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  const sala_status s = check_sparse_varlen(desc, cu_seqlens, pos0);
  if (s != SALA_OK) return s;
  if (!k_pool || (desc->n_q > 0 && (!q || !sel))) return SALA_ERR_NULL;
  if (!all_aligned({q, q_norm_w, k_pool, sel, workspace})) return SALA_ERR_INVALID;
  const size_t need = sala::block_select_varlen_workspace(*desc, cu_seqlens, pos0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_block_select_varlen(*desc, cu_seqlens, pos0, q, q_norm_w, k_pool, sel, workspace,
                                                     (hipStream_t)stream));
}

sala_status sala_sparse_attn_varlen(const sala_sparse_desc* desc, const int32_t* cu_seqlens, const int64_t* pos0,
                                    const void* q, const float* q_norm_w, const void* k_cache, const void* v_cache,
                                    const void* gate, const int32_t* sel, void* out, void* stream) {
  const sala_status s = check_sparse_varlen(desc, cu_seqlens, pos0);
  if (s != SALA_OK) return s;
  if (!k_cache || !v_cache || (desc->n_q > 0 && (!q || !gate || !sel || !out))) return SALA_ERR_NULL;
  if (!all_aligned({q, q_norm_w, k_cache, v_cache, gate, sel, out})) return SALA_ERR_INVALID;
  return hip_status(sala::launch_sparse_attn_varlen(*desc, cu_seqlens, pos0, q, q_norm_w, k_cache, v_cache, gate, sel,
                                                    out, (hipStream_t)stream));
}

int64_t sala_varlen_query_blocks(int32_t nseq, const int32_t* cu_seqlens) {
  if (!cu_seqlens || nseq < 1 || nseq > SALA_VARLEN_MAX_SEQS) return -1;
  return sala::varlen_query_blocks(nseq, cu_seqlens);
}

size_t sala_varlen_workspace_bytes(int op, const void* desc, const int32_t* cu_seqlens, const int64_t* pos0) {
  switch (op) {
    case SALA_OP_LINEAR_PREFILL: {
      const sala_linear_desc* d = static_cast<const sala_linear_desc*>(desc);
      if (check_linear_varlen(d, cu_seqlens, pos0) != SALA_OK) return SIZE_MAX;
      return sala::linear_prefill_varlen_workspace(*d, cu_seqlens);
    }
    case SALA_OP_BLOCK_SELECT: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse_varlen(d, cu_seqlens, pos0) != SALA_OK) return SIZE_MAX;
      return sala::block_select_varlen_workspace(*d, cu_seqlens, pos0);
    }
    case SALA_OP_SPARSE_ATTN: {
      const sala_sparse_desc* d = static_cast<const sala_sparse_desc*>(desc);
      if (check_sparse_varlen(d, cu_seqlens, pos0) != SALA_OK) return SIZE_MAX;
      return 0;
    }
    default: return SIZE_MAX;
  }
}

sala_status sala_kv_pool(const sala_sparse_desc* desc, const void* k_cache, float* k_pool,
                         int64_t block_begin, int64_t block_end, void* stream) {
  sala_status s = check_sparse(desc);
  if (s != SALA_OK) return s;
  if (!k_cache || !k_pool) return SALA_ERR_NULL;
  if (block_begin < 0 || block_end < block_begin || block_end * 64 > desc->kv_len ||
      block_end - block_begin > 2000000000LL)
    return SALA_ERR_INVALID;
  if (!all_aligned({k_cache, k_pool})) return SALA_ERR_INVALID;
  return hip_status(sala::launch_kv_pool(*desc, k_cache, k_pool, block_begin, block_end,
                                         (hipStream_t)stream));
}

sala_status sala_block_select(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                              const float* k_pool, int32_t* sel, float* sel_scores, void* workspace,
                              size_t workspace_bytes, void* stream) {
  sala_status s = check_sparse(desc);
  if (s != SALA_OK) return s;
  if (!q || !k_pool || !sel) return SALA_ERR_NULL;
  if (!all_aligned({q, q_norm_w, k_pool, sel, sel_scores, workspace})) return SALA_ERR_INVALID;
  const size_t need = sala::block_select_workspace(*desc);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_block_select(*desc, q, q_norm_w, k_pool, sel, sel_scores, workspace,
                                              (hipStream_t)stream));
}

sala_status sala_sparse_attn(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                             const void* k_cache, const void* v_cache, const void* gate,
                             const int32_t* sel, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  sala_status s = check_sparse(desc);
  if (s != SALA_OK) return s;
  const sala_sparse_desc& d = *desc;
  if (d.dtype == SALA_BF16 && d.head_dim != 128) return SALA_ERR_UNSUPPORTED;
  if (d.dtype == SALA_BF16 && d.n_q == 1 && d.n_heads / d.n_kv_heads > 16) return SALA_ERR_UNSUPPORTED;
  if (lse && (d.dtype != SALA_BF16 || d.n_q < 2)) return SALA_ERR_UNSUPPORTED;  // bf16 prefill only
  if (!q || !k_cache || !v_cache || !gate || !sel || !out) return SALA_ERR_NULL;
  if (!all_aligned({q, q_norm_w, k_cache, v_cache, gate, sel, out, lse, workspace})) return SALA_ERR_INVALID;
  const size_t need = sala::sparse_attn_workspace(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_sparse_attn(d, q, q_norm_w, k_cache, v_cache, gate, sel, out, lse,
                                             workspace, (hipStream_t)stream));
}

sala_status sala_dense_attn(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                            const void* k_cache, const void* v_cache, const void* gate, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  sala_status s = check_sparse(desc, false);
  if (s != SALA_OK) return s;
  const sala_sparse_desc& d = *desc;
  if (d.dtype == SALA_BF16 && d.head_dim != 128) return SALA_ERR_UNSUPPORTED;
  if (d.dtype == SALA_BF16 && d.n_q == 1 && d.n_heads / d.n_kv_heads > 16) return SALA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !gate || !out) return SALA_ERR_NULL;
  if (!all_aligned({q, q_norm_w, k_cache, v_cache, gate, out, workspace})) return SALA_ERR_INVALID;
  const size_t need = sala::sparse_attn_workspace(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_dense_attn(d, q, q_norm_w, k_cache, v_cache, gate, out, workspace,
                                            (hipStream_t)stream));
}

sala_status sala_sparse_attn_backward(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                                      const void* k_cache, const void* v_cache, const void* gate,
                                      const int32_t* sel, const void* dout, const void* out, const float* lse,
                                      float* dq, float* dk_cache, float* dv_cache, float* dg, float* dq_norm_w,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  sala_status s = check_sparse(desc);
  if (s != SALA_OK) return s;
  const sala_sparse_desc& d = *desc;
  if (d.dtype != SALA_BF16 || d.head_dim != 128 || d.n_q < 2) return SALA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !gate || !sel || !dout || !dq || !dk_cache || !dv_cache || !dg)
    return SALA_ERR_NULL;
  if ((out == nullptr) != (lse == nullptr)) return SALA_ERR_NULL;  // the saved forward state: both or neither
  if (!all_aligned({q, q_norm_w, k_cache, v_cache, gate, sel, dout, out, lse, dq, dk_cache, dv_cache, dg, dq_norm_w,
                    workspace}))
    return SALA_ERR_INVALID;
  const size_t need = sala::sparse_attn_backward_workspace(d);
  if (!workspace || workspace_bytes < need) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_sparse_attn_backward(d, q, q_norm_w, k_cache, v_cache, gate, sel, dout, out, lse,
                                                      dq, dk_cache, dv_cache, dg, dq_norm_w, workspace,
                                                      (hipStream_t)stream));
}

sala_status sala_kv_norm_backward(const sala_sparse_desc* desc, const void* k_new, const float* k_norm_w,
                                  const float* dk_cache, float* dk_new, float* dk_norm_w, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  sala_status s = check_sparse(desc, false);
  if (s != SALA_OK) return s;
  const sala_sparse_desc& d = *desc;
  if (d.dtype != SALA_BF16 || d.head_dim != 128) return SALA_ERR_UNSUPPORTED;
  if (!k_new || !dk_cache || !dk_new) return SALA_ERR_NULL;
  if (!all_aligned({k_new, k_norm_w, dk_cache, dk_new, dk_norm_w, workspace})) return SALA_ERR_INVALID;
  const size_t need = sala::kv_norm_backward_workspace(d);
  if (!workspace || workspace_bytes < need) return SALA_ERR_WORKSPACE;
  return hip_status(sala::launch_kv_norm_backward(d, k_new, k_norm_w, dk_cache, dk_new, dk_norm_w, workspace,
                                                  (hipStream_t)stream));
}

int sala_sparse_layer_uses_dense(const sala_sparse_desc* desc) {
  if (check_sparse(desc) != SALA_OK) return -1;
  return desc->kv_len <= (int64_t)desc->topk * 64 ? 1 : 0;
}

}  // extern "C"
