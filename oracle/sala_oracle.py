"""CPU oracle for the SALA hybrid attention hot path.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The product path (the
HIP library and its Python binding) never imports, calls or links anything here, and this
module imports nothing from the product path.

Everything is plain numpy in float64, written for a reader to check against the pages by eye:
no blocking, fusion or reordering beyond what each definition states. Inputs may arrive as
float32 arrays that hold bf16-representable values; they are upcast exactly to float64.

Sources (the pages this follows; cited by title and section):

* [SALA-zh] "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" (Chinese rendering of
  the MiniCPM-SALA paper): the opening summary (hybrid of 1 sparse : 3 linear layers, QK
  normalisation in every layer, RoPE only in the linear layers, an output gate after every
  attention block), §1 Introduction (sparse attention computes only the most significant part
  of the attention matrix, e.g. a sliding window or global anchors, yet keeps the full KV
  cache; linear attention reaches O(N) through a recurrent formulation), §2.1 Model
  architecture (linear layers have constant per-token compute and memory).
* [SALA-news] "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍",
  section "SALA混合架构：黄金配比破解瓶颈" (Lightning Attention for the linear layers; a fine
  block-selection mechanism lets each query process only a small set of key/value pairs in
  the InfLLM-V2 sparse layers; HyPE: RoPE kept in the linear layers, no positional encoding
  in the sparse layers so the KV cache carries no position information).
* [SALA-blog] "MiniCPM-SALA：混合注意力机制突破LLM长文本处理瓶颈", §2.2 混合位置编码（HyPE）, and
  §5.1 部署建议 (batch size chosen against context length: the packed variable-length batches
  of the *_varlen functions).

Where the pages are silent the reading taken is stated at the function (the pages give no
formula at all): no decay, no normaliser and no scale in the linear layer; an inclusive causal
mask; half-split RoPE with theta_i = base^(-2i/d); per-head RMS QK-norm with eps and an
optional weight; elementwise sigmoid gate; block score = (query-block mean of q-hat, summed
over the GQA group) . (mean of k-hat over the key block); forced blocks = block 0 and the
n_local most recent blocks; ties to the lowest block index; softmax scale 1/sqrt(d).

Parity status: every function below is pinned by the CPU tests (closed forms, a worked
example under tests/golden/, library special cases, brute force and invariants). The RoPE
*convention* (half-split vs interleaved pairs) is not fixed by the pages: the pins fix the
convention chosen here, and that choice itself is "parity unpinned" against the pages.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "qk_norm",
    "rope_inv_freq",
    "rope",
    "sigmoid",
    "linear_prefill",
    "linear_decode",
    "pool_keys",
    "query_block_tilde",
    "block_scores",
    "select_row",
    "select_blocks",
    "sparse_attention",
    "dense_attention",
    "sparse_prefill",
    "sparse_decode",
    "linear_prefill_varlen",
    "sparse_prefill_varlen",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------------------
# Shared per-layer steps: QK-norm, RoPE, output gate ([SALA-zh] opening summary).
# --------------------------------------------------------------------------------------


def qk_norm(x, weight=None, eps=1e-6):
    """Per-head RMS normalisation over the last (head) dimension.

    x_hat = x / sqrt(mean_d(x^2) + eps) * weight. The pages only say QK normalisation is applied
    in every layer ([SALA-zh] opening summary); the RMS form, eps and the unit default weight
    are the reading taken.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if weight is not None:
        y = y * _f64(weight)
    return y


def rope_inv_freq(d, base=10000.0):
    """theta_i = base^(-2i/d) for i in [0, d/2), in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope(x, positions, base=10000.0):
    """Rotary position encoding, half-split ("rotate-half") convention.

    For each pair (x_i, x_{i+d/2}) and angle a = p * theta_i:
        x_i'       = x_i cos a - x_{i+d/2} sin a
        x_{i+d/2}' = x_i sin a + x_{i+d/2} cos a
    x has shape [..., N, H, d] with positions of shape [N] (or a scalar for one token, with
    x of shape [..., H, d]). RoPE is used only in the linear layers ([SALA-news] HyPE;
    [SALA-blog] §2.2); the pair convention is the reading taken.
    """
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    theta = rope_inv_freq(d, base)
    pos = _f64(positions)
    if pos.ndim == 0:
        ang = pos * theta  # [d/2], broadcast over [..., H, d/2]
    else:
        ang = pos[:, None, None] * theta[None, None, :]  # [N, 1, d/2] over [..., N, H, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def sigmoid(x):
    """Logistic function 1 / (1 + exp(-x)), the output gate nonlinearity (reading taken)."""
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------------------
# Linear-attention layer (Lightning-style; [SALA-zh] §1, §2.1; [SALA-news] SALA section).
# --------------------------------------------------------------------------------------


def linear_prefill(q, k, v, g, *, pos0=0, rope_base=10000.0, eps=1e-6, state_in=None,
                   q_norm_w=None, k_norm_w=None):
    """Causal linear attention over a prompt, by its token-by-token recurrence.

    Shapes: q, g [B, N, H, d]; k, v [B, N, Hkv, d] with Hkv dividing H (query head h reads
    the state of KV head h // (H // Hkv)); state_in [B, Hkv, d, d] or None (zeros).

    Steps, for each token t at position p = pos0 + t:
      1. q_hat, k_hat = QK-norm(q_t), QK-norm(k_t); then RoPE at p on both.
      2. S <- S + k_t^T v_t          (outer product, S[i][j] += k[i] v[j])
      3. o_t = q_t S                 (o[j] = sum_i q[i] S[i][j]; read after the update, so the
                                      token attends to itself: inclusive causal mask)
      4. out_t = o_t * sigmoid(g_t)
    Returns (out [B, N, H, d], S_N [B, Hkv, d, d]).

    The recurrence is the definition: the pages describe the linear layer only as an O(N)
    recurrent formulation with constant per-token memory ([SALA-zh] §1, §2.1). No decay,
    no normaliser and no 1/sqrt(d) scale are applied (reading taken).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    assert H % Hkv == 0
    group = H // Hkv
    pos = pos0 + np.arange(N, dtype=np.float64)
    qt = rope(qk_norm(q, q_norm_w, eps), pos, rope_base)
    kt = rope(qk_norm(k, k_norm_w, eps), pos, rope_base)
    S = np.zeros((B, Hkv, d, d)) if state_in is None else _f64(state_in).copy()
    o = np.empty((B, N, H, d))
    kv_head = np.arange(H) // group
    for t in range(N):
        S += kt[:, t, :, :, None] * v[:, t, :, None, :]
        o[:, t] = np.einsum("bhi,bhij->bhj", qt[:, t], S[:, kv_head])
    return o * sigmoid(g), S


def linear_decode(q, k, v, g, state, pos, *, rope_base=10000.0, eps=1e-6, q_norm_w=None,
                  k_norm_w=None):
    """One decode step of the linear layer at position ``pos`` (the same four steps as
    ``linear_prefill`` for a single token). q, g [B, H, d]; k, v [B, Hkv, d];
    state [B, Hkv, d, d]. Returns (out [B, H, d], new state)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, d = q.shape
    Hkv = k.shape[1]
    kv_head = np.arange(H) // (H // Hkv)
    qt = rope(qk_norm(q, q_norm_w, eps), float(pos), rope_base)
    kt = rope(qk_norm(k, k_norm_w, eps), float(pos), rope_base)
    S = _f64(state) + kt[:, :, :, None] * v[:, :, None, :]
    o = np.einsum("bhi,bhij->bhj", qt, S[:, kv_head])
    return o * sigmoid(g), S


# --------------------------------------------------------------------------------------
# Sparse (InfLLM-V2-style) layer: block pooling, block scores, forced + top-k selection,
# softmax attention over the selected blocks ([SALA-zh] §1, §2.1; [SALA-news] SALA section).
# No positional encoding in this layer ([SALA-news] HyPE; [SALA-blog] §2.2).
# --------------------------------------------------------------------------------------


def pool_keys(k_hat, block, n_blocks=None):
    """Mean of the normalised keys over each complete key block.

    k_hat [B, L, Hkv, d] (token-major) -> k_bar [B, Hkv, n_blocks, d]. Only blocks whose
    ``block`` tokens are all present are pooled (n_blocks defaults to L // block).
    """
    k_hat = _f64(k_hat)
    B, L, Hkv, d = k_hat.shape
    nb = L // block if n_blocks is None else n_blocks
    kb = k_hat[:, : nb * block].reshape(B, nb, block, Hkv, d).mean(axis=2)
    return kb.transpose(0, 2, 1, 3)


def query_block_tilde(q_hat, block, n_kv_heads):
    """Per query block i: mean of q_hat over the block's tokens (a ragged last block averages
    only the tokens it has), then summed over the query heads of each GQA group.

    q_hat [B, N, H, d] -> q_tilde [B, Hkv, ceil(N/block), d]. Query head h belongs to group
    h // (H // Hkv).
    """
    q_hat = _f64(q_hat)
    B, N, H, d = q_hat.shape
    nqb = -(-N // block)
    group = H // n_kv_heads
    qt = np.zeros((B, n_kv_heads, nqb, d))
    for i in range(nqb):
        qbar = q_hat[:, i * block: min(N, (i + 1) * block)].mean(axis=1)  # [B, H, d]
        qt[:, :, i] = qbar.reshape(B, n_kv_heads, group, d).sum(axis=2)
    return qt


def block_scores(q_tilde_row, k_bar_rows):
    """Score of each key block j for one query block: q_tilde . k_bar_j (no scale)."""
    return _f64(k_bar_rows) @ _f64(q_tilde_row)


def select_row(scores, i, topk, n_local):
    """Forced + top-k block selection for query block i.

    Forced set F = {0} union {max(0, i - n_local + 1), ..., i} (the first block as a global
    anchor, the n_local most recent blocks as the local window: the sliding-window / global
    anchor patterns of [SALA-zh] §1). Candidates are the remaining causal blocks
    j in [1, i - n_local]; ``scores[j]`` is their score. The r = topk - |F| best candidates are
    kept, ordered by score descending then block index ascending (ties go to the lowest
    index). Returns the selected block indices ascending, padded with -1 to length topk.
    """
    forced = {0} | set(range(max(0, i - n_local + 1), i + 1))
    cands = list(range(1, i - n_local + 1))
    r = topk - len(forced)
    assert r >= 0, "topk must cover the forced blocks"
    if len(cands) <= r:
        chosen = cands
    else:
        chosen = sorted(cands, key=lambda j: (-float(scores[j]), j))[:r]
    sel = sorted(forced | set(chosen))
    return np.array(sel + [-1] * (topk - len(sel)), dtype=np.int64)


def select_blocks(q_tilde, k_bar, topk, n_local):
    """Selection for every (b, kv head, query block). q_tilde [B, Hkv, nqb, d];
    k_bar [B, Hkv, >= nqb - n_local + 1, d]. Returns sel [B, Hkv, nqb, topk] (int64)."""
    q_tilde, k_bar = _f64(q_tilde), _f64(k_bar)
    B, Hkv, nqb, _ = q_tilde.shape
    sel = np.empty((B, Hkv, nqb, topk), dtype=np.int64)
    for b in range(B):
        for gh in range(Hkv):
            for i in range(nqb):
                ncand_end = max(0, i - n_local + 1)  # blocks [0, i - n_local] have scores
                sc = np.full(max(ncand_end, 1), -np.inf)
                if ncand_end > 0:
                    sc[:ncand_end] = block_scores(q_tilde[b, gh, i], k_bar[b, gh, :ncand_end])
                sel[b, gh, i] = select_row(sc, i, topk, n_local)
    return sel


def sparse_attention(q_hat, k_hat, v, sel, block, scale, q_positions=None):
    """Softmax attention of every query over the keys of its query block's selected blocks,
    causal at token level (key position s <= query position t).

    q_hat [B, Nq, H, d] at positions q_positions (default 0..Nq-1); k_hat, v [B, L, Hkv, d]
    (token-major, positions 0..L-1); sel [B, Hkv, nqb, topk] indexed by query block
    t // block. Returns o [B, Nq, H, d].
    """
    q_hat, k_hat, v = _f64(q_hat), _f64(k_hat), _f64(v)
    B, Nq, H, d = q_hat.shape
    L, Hkv = k_hat.shape[1], k_hat.shape[2]
    group = H // Hkv
    qpos = np.arange(Nq) if q_positions is None else np.asarray(q_positions)
    o = np.empty((B, Nq, H, d))
    blocks_of_q = qpos // block
    for b in range(B):
        for i in np.unique(blocks_of_q):
            rows = np.nonzero(blocks_of_q == i)[0]
            for gh in range(Hkv):
                blks = [int(j) for j in sel[b, gh, i] if j >= 0]
                keys = np.concatenate([np.arange(j * block, min(L, (j + 1) * block)) for j in blks])
                K = k_hat[b, keys, gh]  # [nk, d]
                V = v[b, keys, gh]
                allowed = keys[None, :] <= qpos[rows][:, None]  # [nrows, nk]
                for h in range(gh * group, (gh + 1) * group):
                    s = (q_hat[b, rows, h] @ K.T) * scale
                    s = np.where(allowed, s, -np.inf)
                    s = s - s.max(axis=1, keepdims=True)
                    p = np.exp(s)
                    p = p / p.sum(axis=1, keepdims=True)
                    o[b, rows, h] = p @ V
    return o


def dense_attention(q_hat, k_hat, v, scale, q_positions=None):
    """Dense mode of the sparse layer ([SALA-zh] §2.1: the sparse module can run in a dense
    mode with the same weights): causal softmax attention of every query over all keys at
    positions s <= its own position t, by definition (no blocks).

    q_hat [B, Nq, H, d] at positions q_positions (default 0..Nq-1); k_hat, v [B, L, Hkv, d].
    Returns o [B, Nq, H, d].
    """
    q_hat, k_hat, v = _f64(q_hat), _f64(k_hat), _f64(v)
    B, Nq, H, d = q_hat.shape
    L, Hkv = k_hat.shape[1], k_hat.shape[2]
    group = H // Hkv
    qpos = np.arange(Nq) if q_positions is None else np.asarray(q_positions)
    allowed = np.arange(L)[None, :] <= qpos[:, None]  # [Nq, L]
    o = np.empty((B, Nq, H, d))
    for b in range(B):
        for h in range(H):
            s = (q_hat[b, :, h] @ k_hat[b, :, h // group].T) * scale
            s = np.where(allowed, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o[b, :, h] = (p / p.sum(axis=1, keepdims=True)) @ v[b, :, h // group]
    return o


def sparse_prefill(q, k, v, g, *, block=64, topk=64, n_local=2, eps=1e-6, scale=None,
                   q_norm_w=None, k_norm_w=None):
    """The sparse layer over a prompt starting at position 0.

    Shapes: q, g [B, N, H, d]; k, v [B, N, Hkv, d]. Steps: QK-norm on q and k (no RoPE);
    pool complete key blocks; per query block the GQA-summed block mean of q_hat; scores and
    forced + top-k selection; softmax attention (scale 1/sqrt(d) by default) over the
    selected blocks with a token-level causal mask; sigmoid output gate.
    Returns dict(out, sel, q_tilde, k_bar, k_hat).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_hat = qk_norm(q, q_norm_w, eps)
    k_hat = qk_norm(k, k_norm_w, eps)
    k_bar = pool_keys(k_hat, block)
    q_tilde = query_block_tilde(q_hat, block, Hkv)
    sel = select_blocks(q_tilde, k_bar, topk, n_local)
    o = sparse_attention(q_hat, k_hat, v, sel, block, scale)
    return dict(out=o * sigmoid(g), sel=sel, q_tilde=q_tilde, k_bar=k_bar, k_hat=k_hat)


def sparse_decode(q, k_new, v_new, g, k_cache_hat, v_cache, kv_len, *, block=64, topk=64,
                  n_local=2, eps=1e-6, scale=None, q_norm_w=None, k_norm_w=None, k_bar=None):
    """One decode step of the sparse layer for the token at position p = kv_len - 1.

    q, g [B, H, d]; k_new, v_new [B, Hkv, d]; k_cache_hat, v_cache [B, Hkv, >= kv_len - 1, d]
    hold the (already normalised) keys and the values of positions 0..kv_len-2 (cache layout
    [B, Hkv, L, d]). The new key is normalised and appended at p. The query "block" is the
    single current token: q_tilde = sum over the group's heads of q_hat. Candidates are the
    complete blocks [1, i - n_local] with i = p // block. ``k_bar`` may pass precomputed
    pooled keys [B, Hkv, >= i - n_local + 1, d] of the cache (else they are computed here).
    Returns dict(out [B, H, d], sel [B, Hkv, topk]).
    """
    q, g = _f64(q), _f64(g)
    B, H, d = q.shape
    Hkv = k_new.shape[1]
    group = H // Hkv
    p = kv_len - 1
    i = p // block
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_hat = qk_norm(q, q_norm_w, eps)
    k_hat_new = qk_norm(k_new, k_norm_w, eps)
    out = np.empty((B, H, d))
    sel = np.empty((B, Hkv, topk), dtype=np.int64)
    n_cand_blocks = max(0, i - n_local + 1)  # blocks 0 .. i - n_local need pooled keys
    for b in range(B):
        for gh in range(Hkv):
            K = np.concatenate([_f64(k_cache_hat[b, gh, :p]), k_hat_new[b, gh][None]], axis=0)
            V = np.concatenate([_f64(v_cache[b, gh, :p]), _f64(v_new[b, gh])[None]], axis=0)
            qt = q_hat[b, gh * group:(gh + 1) * group].sum(axis=0)
            sc = np.full(max(n_cand_blocks, 1), -np.inf)
            if n_cand_blocks > 0:
                if k_bar is None:
                    kb = K[: n_cand_blocks * block].reshape(n_cand_blocks, block, d).mean(axis=1)
                else:
                    kb = _f64(k_bar[b, gh, :n_cand_blocks])
                sc[:n_cand_blocks] = block_scores(qt, kb)
            row = select_row(sc, i, topk, n_local)
            sel[b, gh] = row
            keys = np.concatenate([np.arange(j * block, min(kv_len, (j + 1) * block))
                                   for j in row if j >= 0])
            Ks, Vs = K[keys], V[keys]
            for h in range(gh * group, (gh + 1) * group):
                s = (Ks @ q_hat[b, h]) * scale
                s = s - s.max()
                w = np.exp(s)
                out[b, h] = (w / w.sum()) @ Vs
    return dict(out=out * sigmoid(g), sel=sel)


# ---------------------------------------------------------------- packed variable-length batches


def _cu(seqlens):
    cu = np.zeros(len(seqlens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(seqlens)
    return cu


def linear_prefill_varlen(q, k, v, g, seqlens, pos0=None, *, rope_base=10000.0, eps=1e-6, state_in=None,
                          q_norm_w=None, k_norm_w=None):
    """A packed batch of independent sequences through the linear layer ([SALA-blog] §5.1: the
    batch is sized to the context, so one batch holds prompts of different lengths).

    q, k, v, g [T, H, d] hold the sequences back to back (sequence s owns rows
    cu[s] .. cu[s+1] - 1, cu = prefix sums of seqlens); pos0[s] is the position of its first
    token; state_in [nseq, H, d, d] or None. Each sequence is ``linear_prefill`` on its own
    rows with its own state: no state or position crosses sequences.
    Returns (out [T, H, d], states [nseq, H, d, d]).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    T, H, d = q.shape
    Hkv = k.shape[1]
    cu = _cu(seqlens)
    assert cu[-1] == T
    pos0 = [0] * len(seqlens) if pos0 is None else list(pos0)
    out = np.empty((T, H, d))
    states = np.empty((len(seqlens), Hkv, d, d))
    for s in range(len(seqlens)):
        a, b = cu[s], cu[s + 1]
        o, S = linear_prefill(q[None, a:b], k[None, a:b], v[None, a:b], g[None, a:b], pos0=pos0[s],
                              rope_base=rope_base, eps=eps,
                              state_in=None if state_in is None else _f64(state_in)[s:s + 1],
                              q_norm_w=q_norm_w, k_norm_w=k_norm_w)
        out[a:b] = o[0]
        states[s] = S[0]
    return out, states


def sparse_prefill_varlen(q, k, v, g, seqlens, *, block=64, topk=64, n_local=2, eps=1e-6, scale=None,
                          q_norm_w=None, k_norm_w=None):
    """A packed batch of prompts through the sparse layer, each prompt from position 0 with
    its own KV cache, pooled keys and selection. q, g [T, Hq, d]; k, v [T, Hkv, d], sequences
    back to back as in ``linear_prefill_varlen``. Each sequence is ``sparse_prefill`` on its own
    rows. Returns dict(out [T, Hq, d], sel: list of [Hkv, nqb_s, topk] per sequence).
    (The queries of a prompt continued after a cached prefix give the outputs of the whole
    prompt's last tokens, as when one prompt is prefilled in consecutive calls.)
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    T, Hq, d = q.shape
    cu = _cu(seqlens)
    assert cu[-1] == T
    out = np.empty((T, Hq, d))
    sels = []
    for s in range(len(seqlens)):
        a, b = cu[s], cu[s + 1]
        if b == a:
            sels.append(np.zeros((k.shape[1], 0, topk), dtype=np.int64))
            continue
        r = sparse_prefill(q[None, a:b], k[None, a:b], v[None, a:b], g[None, a:b], block=block, topk=topk,
                           n_local=n_local, eps=eps, scale=scale, q_norm_w=q_norm_w, k_norm_w=k_norm_w)
        out[a:b] = r["out"][0]
        sels.append(r["sel"][0])
    return dict(out=out, sel=sels)
