/*
 * libsala — the SALA hybrid attention hot path (linear layers + block-sparse layers) for
 * AMD MI355X (gfx950). C ABI: plain pointers and sizes, no framework types.
 *
 * The method: a hybrid decoder whose attention layers are 75% linear attention (Lightning
 * style) and 25% block-sparse softmax attention (InfLLM-V2 style); QK normalisation in every
 * layer; RoPE only in the linear layers (the sparse layers use no positional encoding, so
 * their KV cache is position-free); an output gate after every attention block.
 * Pages: "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" (opening summary; §1
 * Introduction; §2.1 Model architecture) and "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧
 * 跑通百万上下文，速度飙升3.5倍" (section "SALA混合架构：黄金配比破解瓶颈").
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Memory: every tensor pointer is DEVICE memory owned by the caller; the library never
 *   allocates, frees or synchronises. Scratch memory, where needed, is a caller-provided
 *   device `workspace` of at least sala_workspace_bytes(op, desc) bytes. Pointers must be
 *   16-byte aligned; tensors are dense and contiguous in the layouts stated below.
 * - dtype: SALA_BF16 tensors hold bf16 bit patterns (uint16); SALA_F32 tensors hold float.
 *   The linear state, norm weights and pooled keys are always float32.
 * - Stream: `stream` is a hipStream_t (NULL = the default stream). Work is enqueued in
 *   stream order and runs asynchronously; results are valid once the stream is synchronised.
 * - Errors: arguments are checked before anything is enqueued. On any non-OK status nothing
 *   has been enqueued, except SALA_ERR_HIP, which reports a failed launch (the HIP error code
 *   is kept per thread, see sala_last_hip_error). Device faults surface at the caller's next
 *   synchronisation. No C++ exception crosses this interface.
 * - Aliasing: outputs must not overlap inputs, except where an entry point says otherwise.
 */
#ifndef SALA_H_
#define SALA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SALA_ABI_VERSION 6

/* sequences per call of the packed variable-length (varlen) entry points */
#define SALA_VARLEN_MAX_SEQS 64

typedef enum {
  SALA_OK = 0,
  SALA_ERR_NULL = 1,        /* a required pointer is NULL */
  SALA_ERR_INVALID = 2,     /* inconsistent or out-of-range sizes / parameters / alignment */
  SALA_ERR_UNSUPPORTED = 3, /* valid, but not a shape or dtype this library implements */
  SALA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than sala_workspace_bytes() */
  SALA_ERR_HIP = 5          /* a kernel launch failed */
} sala_status;

typedef enum { SALA_F32 = 0, SALA_BF16 = 1 } sala_dtype;

typedef enum {
  SALA_OP_LINEAR_PREFILL = 1,
  SALA_OP_BLOCK_SELECT = 2,
  SALA_OP_SPARSE_ATTN = 3,
  SALA_OP_DENSE_ATTN = 4,
  SALA_OP_LINEAR_BACKWARD = 5,
  SALA_OP_SPARSE_ATTN_BACKWARD = 6,
  SALA_OP_KV_NORM_BACKWARD = 7,
  SALA_OP_SPARSE_DECODE_STEP = 8
} sala_op;

/* Linear-attention layer shape.
 *   batch      B >= 1
 *   seq_len    N tokens in this call (prefill: N >= 0; decode: must be 1)
 *   n_heads    H query heads
 *   n_kv_heads Hkv key/value heads, dividing H (at most 64 query heads per KV head): query head h
 *              reads the state of KV head h / (H / Hkv); the state is per KV head. Hkv = H is
 *              plain multi-head linear attention
 *   head_dim   d: 64 or 128 (bf16 prefill needs 128)
 *   dtype      sala_dtype of q, k, v, gate and out
 *   pos0       position of the first token of the call (>= 0); RoPE uses p = pos0 + t
 *   rope_base  RoPE base (theta_i = rope_base^(-2i/d)), > 0
 *   norm_eps   QK-norm epsilon, >= 0
 *   chunk      tokens per chunk of the chunked evaluation: 64 (0 selects 64). The result does not
 *              depend on it in exact arithmetic (the chunked form equals the recurrence); 128
 *              and 256 are valid chunk sizes that this library does not build
 *              (SALA_ERR_UNSUPPORTED); other values are SALA_ERR_INVALID
 *   reserved_  must be 0 */
typedef struct {
  int32_t batch;
  int32_t seq_len;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int64_t pos0;
  float rope_base;
  float norm_eps;
  int32_t chunk;
  int32_t reserved_;
} sala_linear_desc;

/* Block-sparse layer shape.
 *   batch       B >= 1
 *   n_q         query tokens in this call (prefill: >= 1; decode: 1). The queries are the
 *               tokens at positions [kv_len - n_q, kv_len); when n_q > 1 the first of them
 *               must start a block ((kv_len - n_q) % block == 0).
 *   n_heads     Hq query heads; n_kv_heads Hkv divides Hq (GQA group = Hq / Hkv heads)
 *   head_dim    d: 64 or 128 (bf16 needs 128)
 *   dtype       sala_dtype of q, gate, out, k/v caches and new k/v
 *   block       tokens per key block and per query block: must be 64
 *   topk        blocks kept per query block, forced blocks included: 1 + n_local .. 256
 *   n_local     local blocks forced (the query's own block, and block i-1 when 2): 1 or 2
 *   norm_eps    QK-norm epsilon, >= 0
 *   scale       softmax scale; 0 selects 1/sqrt(d)
 *   kv_len      tokens in the cache once this call's tokens are in it (>= n_q)
 *   kv_capacity token capacity of each cache row: >= kv_len, multiple of 64 */
typedef struct {
  int32_t batch;
  int32_t n_q;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t block;
  int32_t topk;
  int32_t n_local;
  float norm_eps;
  float scale;
  int32_t reserved_;
  int64_t kv_len;
  int64_t kv_capacity;
} sala_sparse_desc;

/* Linear layer prefill: causal linear attention over the N tokens of the call, carrying the
 * per-head d x d state (pages: "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" §1 and
 * §2.1 — O(N) recurrent linear attention with constant per-token memory; opening summary —
 * QK-norm, RoPE and output gate). Per token t at position p = pos0 + t:
 *   q^ = RoPE_p(RMSNorm(q_t) * q_norm_w), k^ = RoPE_p(RMSNorm(k_t) * k_norm_w)
 *   S  <- S + k^^T v_t           (S[i][j] += k^[i] v[j])
 *   out_t = (q^ S) * sigmoid(g_t)
 * Inputs  q, gate, out: [B, N, H, d]; k, v: [B, N, Hkv, d] (token-major, dtype);
 *         q_norm_w, k_norm_w: [d] float or NULL (= all ones);
 *         state_in: [B, Hkv, d, d] float (S[i][j], row i = key dim) or NULL (= zeros).
 * Outputs out: [B, N, H, d]; state_out: [B, Hkv, d, d] float, or NULL to skip. state_out may
 *         alias state_in. The bf16 path evaluates the recurrence in 64-token chunks on MFMA
 *         (bf16 operands, fp32 accumulation, fp32 state); the f32 path is a plain fp32 scan.
 * Workspace: sala_workspace_bytes(SALA_OP_LINEAR_PREFILL, desc) bytes (may be 0). */
sala_status sala_linear_prefill(const sala_linear_desc* desc, const void* q, const void* k,
                                const void* v, const void* gate, const float* q_norm_w,
                                const float* k_norm_w, const float* state_in, float* state_out,
                                void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Linear layer decode step: one token per sequence at position desc->pos0 (same pages).
 * desc->seq_len must be 1. q, gate, out: [B, H, d]; k, v: [B, Hkv, d]; state: [B, Hkv, d, d]
 * float, updated in place (S <- S + k^^T v once per KV head, then out = (q^ S) * sigmoid(g) for
 * each query head of its group). */
sala_status sala_linear_decode_step(const sala_linear_desc* desc, const void* q, const void* k,
                                    const void* v, const void* gate, const float* q_norm_w,
                                    const float* k_norm_w, float* state, void* out, void* stream);

/* Linear layer backward (pages: as sala_linear_prefill; "面壁智能发布MiniCPM-SALA：稀疏-线性混合
 * 架构，9B模型端侧跑通百万上下文，速度飙升3.5倍" section "高效训练范式：以25%的成本完成转换" — the
 * linear layers are trained first, all parameters later). Given dout = dL/d out and, optionally,
 * dstate_out = dL/d state_out, returns the gradients of L through sala_linear_prefill with the
 * same desc and inputs:
 *   dq, dk, dv, dg: [B, N, H, d] float (required);
 *   dq_norm_w, dk_norm_w: [d] float, or NULL to skip (computed as if the weight were all ones
 *   when the matching input weight is NULL);
 *   dstate_in: [B, H, d, d] float, or NULL to skip.
 * Inputs q, k, v, gate, dout: [B, N, H, d] bf16 (desc->dtype must be SALA_BF16, head_dim 128,
 * n_kv_heads = n_heads: grouped heads are SALA_ERR_UNSUPPORTED here);
 * q_norm_w, k_norm_w, state_in, dstate_out as in sala_linear_prefill (NULL = ones / zeros).
 * The gradients are chunked causal linear attentions over the normalised, rotated q and k (two
 * of them in reverse token order) on MFMA with bf16 operands and fp32 accumulation; the norm,
 * RoPE and gate transposes run in fp32. Deterministic (no atomics). Nothing may alias.
 * Workspace: sala_workspace_bytes(SALA_OP_LINEAR_BACKWARD, desc) bytes. */
sala_status sala_linear_backward(const sala_linear_desc* desc, const void* q, const void* k,
                                 const void* v, const void* gate, const float* q_norm_w,
                                 const float* k_norm_w, const float* state_in, const void* dout,
                                 const float* dstate_out, float* dq, float* dk, float* dv,
                                 float* dg, float* dq_norm_w, float* dk_norm_w, float* dstate_in,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Sparse layer KV append (pages: "面壁智能发布MiniCPM-SALA…" section "SALA混合架构…" — the sparse
 * layers keep the full KV cache without positional encoding; the block-selection mechanism
 * works on whole key blocks). Writes the n_q new tokens at positions [kv_len - n_q, kv_len):
 *   k_cache[b, g, p, :] = RMSNorm(k_new[b, t, g, :]) * k_norm_w   (bf16/f32 as dtype)
 *   v_cache[b, g, p, :] = v_new[b, t, g, :]
 * and, for every key block that this call completes, the pooled key
 *   k_pool[b, g, j, :] = mean of the block's 64 normalised keys (float; new keys contribute
 *   their float value before rounding to the cache dtype, keys already cached their stored
 *   value).
 * k_new, v_new: [B, n_q, Hkv, d]; k_cache, v_cache: [B, Hkv, kv_capacity, d];
 * k_pool: [B, Hkv, kv_capacity / 64, d] float; k_norm_w: [d] float or NULL. */
sala_status sala_kv_append(const sala_sparse_desc* desc, const void* k_new, const void* v_new,
                           const float* k_norm_w, void* k_cache, void* v_cache, float* k_pool,
                           void* stream);

/* Rebuild pooled keys from the cache contents: k_pool[b, g, j, :] = mean over the block's 64
 * cached keys, for blocks j in [block_begin, block_end), all of which must be complete
 * (block_end * 64 <= kv_len). For caches filled outside sala_kv_append (restored state). */
sala_status sala_kv_pool(const sala_sparse_desc* desc, const void* k_cache, float* k_pool,
                         int64_t block_begin, int64_t block_end, void* stream);

/* Linear layer decode step with each sequence at its own position (same pages): as
 * sala_linear_decode_step, with token b at position pos[b] (pos: DEVICE array [B] int64, read
 * by the kernel, so a captured graph can replay with updated positions; negative values read as
 * 0); desc->pos0 is ignored. */
sala_status sala_linear_decode_step_at(const sala_linear_desc* desc, const int64_t* pos, const void* q,
                                       const void* k, const void* v, const void* gate, const float* q_norm_w,
                                       const float* k_norm_w, float* state, void* out, void* stream);

/* Block selection for the sparse layer (same pages; sliding-window and global-anchor patterns
 * from "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" §1). For each query block i covered by
 * the call (decode: the block of the single query) and KV group g:
 *   q~[g, i] = sum over the group's heads h of mean over the block's query tokens of
 *              RMSNorm(q[t, h]) * q_norm_w          (decode: the single token, no mean)
 *   score[j] = q~[g, i] . k_pool[g, j] for candidate blocks j in [1, i - n_local]
 *   forced   = {0} U {i - n_local + 1 .. i}; keep the topk - |forced| best candidates,
 *              ranked by score descending then block index ascending (ties: lowest index).
 * Output sel: [B, Hkv, nqb, topk] int32, ascending block indices, padded with -1, where
 * nqb = (kv_len - 1) / 64 - (kv_len - n_q) / 64 + 1 (row r is query block
 * (kv_len - n_q) / 64 + r). Scores are fp32. q: [B, n_q, Hq, d]; k_pool as in sala_kv_append.
 * sel_scores: NULL, or [B, Hkv, nqb, topk] float receiving, beside each entry of sel, the score
 * of a chosen candidate block, +INFINITY for a forced block and -INFINITY for padding.
 * Workspace: sala_workspace_bytes(SALA_OP_BLOCK_SELECT, desc). */
sala_status sala_block_select(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                              const float* k_pool, int32_t* sel, float* sel_scores, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Block-sparse softmax attention with output gate (same pages). For each query token t (at
 * position p) and head h in KV group g, with i = p / 64:
 *   keys    = tokens s <= p of the blocks listed in sel[b, g, i - first_block, :] (-1 ignored)
 *   out[t,h] = softmax_s(scale * q^ . k_cache[s]) . v_cache[s] * sigmoid(gate[t, h])
 * where q^ = RMSNorm(q) * q_norm_w and the cache holds already-normalised keys. The bf16 path
 * uses MFMA (bf16 operands, fp32 accumulation and fp32 online softmax).
 * q, gate, out: [B, n_q, Hq, d]; caches as in sala_kv_append; sel as from sala_block_select:
 *   ascending block indices of 0 .. i ending with i, then -1. Other contents are not checked on
 *   the device: they give unspecified outputs, but every read stays inside the caches (indices
 *   are clamped to the cache rows that exist).
 * lse: NULL, or [B, n_q, Hq] float receiving each row's log2-sum-exp2 of its scaled scores,
 *   log2 sum_s exp2(scale * log2(e) * q^ . k_cache[s]) (the state a backward pass can reuse,
 *   see sala_sparse_attn_backward); bf16 prefill (n_q > 1) only, else SALA_ERR_UNSUPPORTED.
 * Workspace: sala_workspace_bytes(SALA_OP_SPARSE_ATTN, desc). */
sala_status sala_sparse_attn(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                             const void* k_cache, const void* v_cache, const void* gate,
                             const int32_t* sel, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Dense mode of the sparse layer ("MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" §2.1: the
 * sparse attention module switches between a dense and a sparse mode with the same weights).
 * As sala_sparse_attn with every block 0 .. i attended (plain causal softmax attention over
 * the cache, QK-norm on q, no positional encoding, output gate); no selection is read.
 * desc->topk and desc->n_local are ignored. Same layouts, ownership and errors as
 * sala_sparse_attn. Workspace: sala_workspace_bytes(SALA_OP_DENSE_ATTN, desc). */
sala_status sala_dense_attn(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                            const void* k_cache, const void* v_cache, const void* gate, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Sparse layer attention backward (pages: as sala_sparse_attn; "面壁智能发布MiniCPM-SALA…" section
 * "高效训练范式：以25%的成本完成转换" — sparse attention is on in the later training stages, which
 * train every parameter). Given dout = dL/d out of a bf16 prefill sala_sparse_attn call (n_q > 1)
 * with the same desc and inputs, returns, with the selection held fixed (a discrete choice):
 *   dq, dg: [B, n_q, Hq, d] float (required);
 *   dk_cache, dv_cache: [B, Hkv, kv_capacity, d] float (required): the gradients with respect to
 *     the cache contents (the normalised keys k^ and the values); every row is written, 0 for
 *     rows no query attends;
 *   dq_norm_w: [d] float or NULL to skip (computed as if all ones when q_norm_w is NULL).
 * out, lse: the forward call's out and lse (both, or both NULL). Given, the softmax statistics
 * come from them (lse as saved; D = rowsum(dout * out)); NULL, they are recomputed by rerunning
 * the forward. Products run on MFMA with bf16
 * operands (q^ scale log2 e, dO = dout sigmoid(gate), P and dS) and fp32 accumulation. The
 * key/value gradients are accumulated key-block by key-block over the query blocks that chose
 * each block, in a fixed order: the result is deterministic. Nothing may alias.
 * Workspace: sala_workspace_bytes(SALA_OP_SPARSE_ATTN_BACKWARD, desc) bytes. */
sala_status sala_sparse_attn_backward(const sala_sparse_desc* desc, const void* q, const float* q_norm_w,
                                      const void* k_cache, const void* v_cache, const void* gate,
                                      const int32_t* sel, const void* dout, const void* out, const float* lse,
                                      float* dq, float* dk_cache, float* dv_cache, float* dg, float* dq_norm_w,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Backward of the key normalisation sala_kv_append applies to the n_q appended tokens (k^ =
 * RMSNorm(k_new) * k_norm_w, written at cache positions [kv_len - n_q, kv_len)). dk_cache is the
 * cache gradient from sala_sparse_attn_backward; returns dk_new [B, n_q, Hkv, d] float and, unless
 * NULL, dk_norm_w [d] float. The value gradient of the appended tokens is the dv_cache rows of
 * those positions (the append copies v unchanged). k_new: bf16 [B, n_q, Hkv, d].
 * Workspace: sala_workspace_bytes(SALA_OP_KV_NORM_BACKWARD, desc) bytes. */
sala_status sala_kv_norm_backward(const sala_sparse_desc* desc, const void* k_new, const float* k_norm_w,
                                  const float* dk_cache, float* dk_new, float* dk_norm_w, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Decode step of the sparse layer with each sequence at its own cache length (the pages'
 * decoding against a cache that grows per sequence; "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模"
 * §1 and the sections cited at sala_kv_append / sala_block_select / sala_sparse_attn). One call
 * runs, for every sequence b with L_b = kv_lens[b] (DEVICE array [B] int64, clamped to
 * [1, desc->kv_len]): sala_kv_append of its token at position L_b - 1 (pooling the block it
 * completes), sala_block_select for its query block (L_b - 1) / 64, and sala_sparse_attn
 * over the cache's first L_b tokens. desc: n_q = 1, kv_len = the largest L_b (sizes the grids;
 * contexts up to 16,384 candidate blocks, else UNSUPPORTED), bf16, d = 128, at most 16 query
 * heads per KV head. q, gate, out: [B, Hq, d]; k_new, v_new: [B, Hkv, d]; caches and pool as in
 * sala_kv_append; sel: [B, Hkv, topk] int32 receives the selection.
 * Workspace: sala_workspace_bytes(SALA_OP_SPARSE_DECODE_STEP, desc). */
sala_status sala_sparse_decode_step(const sala_sparse_desc* desc, const int64_t* kv_lens, const void* q,
                                    const float* q_norm_w, const void* k_new, const void* v_new,
                                    const float* k_norm_w, const void* gate, void* k_cache, void* v_cache,
                                    float* k_pool, int32_t* sel, void* out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Scratch bytes of sala_sparse_decode_step_noalloc (a static device array per device). */
#define SALA_NOALLOC_SCRATCH_BYTES (8u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc): sala_sparse_decode_step with its scratch memory taken
 * from a static device array of SALA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each
 * device it runs on until the process ends, instead of a caller workspace. The library allocates
 * nothing during the call. Arguments, layouts and results are those of sala_sparse_decode_step
 * without the workspace. The work runs on the current device; a non-NULL stream must belong to
 * it (else SALA_ERR_INVALID). SALA_ERR_WORKSPACE: the call needs more than
 * SALA_NOALLOC_SCRATCH_BYTES (sala_workspace_bytes(SALA_OP_SPARSE_DECODE_STEP, desc) bytes;
 * 2.4 MB for batch 8, 2 KV heads and a 1M-token context). Every call on a device shares its array
 * and leaves it holding that call's partial results; the kernels write every scratch byte they
 * read, so nothing carries over, but calls that overlap in time on one device (other streams,
 * other threads) race on it and must be serialised by the caller. */
sala_status sala_sparse_decode_step_noalloc(const sala_sparse_desc* desc, const int64_t* kv_lens, const void* q,
                                            const float* q_norm_w, const void* k_new, const void* v_new,
                                            const float* k_norm_w, const void* gate, void* k_cache, void* v_cache,
                                            float* k_pool, int32_t* sel, void* out, void* stream);

/* The switch between the two modes (same section; the pages give no length, so the rule is the
 * one under which both modes give the same result): 1 when every query of the call would
 * select all of its causal blocks (kv_len <= topk * 64, so sala_dense_attn equals block
 * selection + sala_sparse_attn and the selection can be skipped), 0 when the sparse path must
 * run, -1 for an invalid descriptor. Host-side, no device work. */
int sala_sparse_layer_uses_dense(const sala_sparse_desc* desc);

/* ---- Packed variable-length batches ("varlen"). The pages advise sizing the batch to the
 * context length ("MiniCPM-SALA：混合注意力机制突破LLM长文本处理瓶颈" §5.1 部署建议), so a serving
 * batch mixes prompts of different lengths. These entry points prefill nseq = desc->batch
 * sequences (1 .. SALA_VARLEN_MAX_SEQS) whose new tokens are stored back to back along the token
 * dimension, with the same per-sequence results as one call per sequence.
 *   cu_seqlens  HOST array [nseq + 1] int32: cu_seqlens[0] = 0, nondecreasing, ending at the
 *               packed token count (desc->seq_len, resp. desc->n_q); sequence s owns packed
 *               tokens [cu_seqlens[s], cu_seqlens[s + 1]) (an empty sequence is allowed)
 *   pos0        HOST array [nseq] int64 >= 0: position of sequence s's first token of the call
 *               (the number of its tokens processed by earlier calls)
 * Both arrays are read during the call only. bf16 and d = 128 only (else UNSUPPORTED); more than
 * SALA_VARLEN_MAX_SEQS sequences: UNSUPPORTED. Activations are [T, H, d]; per-sequence state,
 * cache and pool tensors are indexed by the sequence (batch) index s.
 * Workspace: sala_varlen_workspace_bytes(op, desc, cu_seqlens, pos0). */

/* Linear layer prefill of a packed batch: sala_linear_prefill on each sequence, its tokens at
 * positions pos0[s] + t (desc->pos0 is ignored). desc->batch = nseq, desc->seq_len = T.
 * q, k, v, gate, out: [T, H, d] bf16; state_in / state_out: [nseq, H, d, d] float (NULL: zeros /
 * not written; may alias). All sequences run in one launch per kernel. */
sala_status sala_linear_prefill_varlen(const sala_linear_desc* desc, const int32_t* cu_seqlens,
                                       const int64_t* pos0, const void* q, const void* k, const void* v,
                                       const void* gate, const float* q_norm_w, const float* k_norm_w,
                                       const float* state_in, float* state_out, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Sparse layer of a packed batch. desc: batch = nseq, n_q = T, kv_capacity = capacity of each
 * sequence's cache row; kv_len is ignored: sequence s's cache holds pos0[s] + n_s tokens once its
 * n_s new tokens are in it. pos0[s] must be a multiple of 64 and pos0[s] + n_s <= kv_capacity.
 * k_cache, v_cache: [nseq, Hkv, kv_capacity, d]; k_pool: [nseq, Hkv, kv_capacity / 64, d] float.
 * sel: the per-sequence selections [Hkv, nqb_s, topk] (nqb_s = ceil(n_s / 64); row r is query
 * block pos0[s] / 64 + r) stored one after another in sequence order,
 * sala_varlen_query_blocks() * Hkv rows of topk int32 in all.
 *   sala_kv_append_varlen:    sala_kv_append per sequence (new k, v: [T, Hkv, d]).
 *   sala_block_select_varlen: sala_block_select per sequence (q: [T, Hq, d]); one workspace is
 *                             shared by the sequences, which run one after another.
 *   sala_sparse_attn_varlen:  sala_sparse_attn per sequence (q, gate, out: [T, Hq, d]), all
 *                             sequences in one launch; no workspace. */
sala_status sala_kv_append_varlen(const sala_sparse_desc* desc, const int32_t* cu_seqlens, const int64_t* pos0,
                                  const void* k_new, const void* v_new, const float* k_norm_w, void* k_cache,
                                  void* v_cache, float* k_pool, void* stream);
sala_status sala_block_select_varlen(const sala_sparse_desc* desc, const int32_t* cu_seqlens, const int64_t* pos0,
                                     const void* q, const float* q_norm_w, const float* k_pool, int32_t* sel,
                                     void* workspace, size_t workspace_bytes, void* stream);
sala_status sala_sparse_attn_varlen(const sala_sparse_desc* desc, const int32_t* cu_seqlens, const int64_t* pos0,
                                    const void* q, const float* q_norm_w, const void* k_cache, const void* v_cache,
                                    const void* gate, const int32_t* sel, void* out, void* stream);

/* Query blocks of a packed batch: the sum over the sequences of ceil(n_s / 64) (-1 for invalid
 * arguments). Host-side. */
int64_t sala_varlen_query_blocks(int32_t nseq, const int32_t* cu_seqlens);

/* Workspace bytes of a varlen operation (SALA_OP_LINEAR_PREFILL, SALA_OP_BLOCK_SELECT or
 * SALA_OP_SPARSE_ATTN, which needs none) for this batch; SIZE_MAX if the arguments are invalid. */
size_t sala_varlen_workspace_bytes(int op, const void* desc, const int32_t* cu_seqlens, const int64_t* pos0);

/* Workspace bytes an operation needs for this descriptor (0 if none; SIZE_MAX if the
 * descriptor is invalid). `desc` points to a sala_linear_desc for SALA_OP_LINEAR_PREFILL and
 * to a sala_sparse_desc otherwise. */
size_t sala_workspace_bytes(int op, const void* desc);

const char* sala_status_str(sala_status status);
int sala_abi_version(void);
/* hipError_t of the last SALA_ERR_HIP on the calling thread (0 if none). */
int sala_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SALA_H_ */
