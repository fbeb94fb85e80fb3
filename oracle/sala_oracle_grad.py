"""Gradient oracle for the SALA attention layers (backward of the hot path).

TEST INFRASTRUCTURE ONLY, like ``sala_oracle``: only the test suite, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg may import or call it; the product path never does.

The forward steps of ``sala_oracle`` are re-expressed one for one in float64 PyTorch on the CPU
(same order, same readings of the pages), and their gradients are taken by autograd. No
gradient formula is written by hand here. The pages convert a model by training its linear
layers first, with sparse attention off, and later train all parameters with sparse attention
on ([SALA-news] section "高效训练范式：以25%的成本完成转换"), which is what a backward pass of both
layers serves; the pages give no gradient formulas of their own.

* ``linear_layer``: the linear-attention layer (QK-norm, RoPE, the token recurrence with an
  inclusive causal read-out, sigmoid output gate), returning (out, final state).
* ``sparse_attention_layer``: the sparse layer's attention step for a fixed block selection:
  QK-norm of q, softmax over the keys of the selected blocks (causal at token level, scale
  1/sqrt(d)), sigmoid output gate. The keys arrive already normalised (the cache holds
  k_hat); ``key_norm`` is the normalisation the cache append applies. The selection is a
  discrete choice and carries no gradient.

Parity status: pinned by tests/test_oracle_grad_pins.py: the torch forward equals the numpy
oracle forward, and every gradient matches central finite differences of the numpy oracle.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from . import sala_oracle as npo

__all__ = [
    "linear_layer",
    "linear_layer_grads",
    "sparse_attention_layer",
    "sparse_attention_grads",
    "key_norm",
    "key_norm_grads",
]


def _t(x, grad=False):
    if x is None:
        return None
    return torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64, requires_grad=grad)


def _qk_norm(x, w, eps):
    """x / sqrt(mean_d x^2 + eps) * w over the last dimension (sala_oracle.qk_norm)."""
    y = x / torch.sqrt(torch.mean(x * x, dim=-1, keepdim=True) + eps)
    return y if w is None else y * w


def _rope(x, positions, base):
    """Half-split rotation by p * theta_i (sala_oracle.rope), positions [N] over x [B, N, H, d]."""
    d = x.shape[-1]
    half = d // 2
    theta = torch.tensor(npo.rope_inv_freq(d, base), dtype=torch.float64)
    ang = torch.tensor(np.asarray(positions, np.float64), dtype=torch.float64)[:, None, None] * theta
    c, s = torch.cos(ang), torch.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], dim=-1)


def linear_layer(q, k, v, g, *, pos0=0, rope_base=10000.0, eps=1e-6, state_in=None, q_norm_w=None,
                 k_norm_w=None):
    """sala_oracle.linear_prefill in torch: the same four steps per token. Tensors in, tensors
    out (out [B, N, H, d], final state [B, Hkv, d, d])."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    group = H // Hkv
    pos = pos0 + np.arange(N, dtype=np.float64)
    qt = _rope(_qk_norm(q, q_norm_w, eps), pos, rope_base)
    kt = _rope(_qk_norm(k, k_norm_w, eps), pos, rope_base)
    S = torch.zeros((B, Hkv, d, d), dtype=torch.float64) if state_in is None else state_in
    kv_head = torch.arange(H) // group
    outs = []
    for t in range(N):
        S = S + kt[:, t, :, :, None] * v[:, t, :, None, :]
        outs.append(torch.einsum("bhi,bhij->bhj", qt[:, t], S[:, kv_head]))
    o = torch.stack(outs, dim=1)
    return o * torch.sigmoid(g), S


def linear_layer_grads(q, k, v, g, dout, *, dstate_out=None, pos0=0, rope_base=10000.0, eps=1e-6,
                       state_in=None, q_norm_w=None, k_norm_w=None):
    """Gradients of <out, dout> + <final state, dstate_out> with respect to every input of the
    linear layer. Returns dict(dq, dk, dv, dg, dstate_in, dq_norm_w, dk_norm_w) as float64
    numpy arrays (the last three are None when the input was None)."""
    tq, tk, tv, tg = _t(q, True), _t(k, True), _t(v, True), _t(g, True)
    ts, tqw, tkw = _t(state_in, True), _t(q_norm_w, True), _t(k_norm_w, True)
    out, S = linear_layer(tq, tk, tv, tg, pos0=pos0, rope_base=rope_base, eps=eps, state_in=ts,
                          q_norm_w=tqw, k_norm_w=tkw)
    loss = (out * _t(dout)).sum()
    if dstate_out is not None:
        loss = loss + (S * _t(dstate_out)).sum()
    loss.backward()

    def grad(x):
        return None if x is None else x.grad.numpy().copy()

    return dict(dq=grad(tq), dk=grad(tk), dv=grad(tv), dg=grad(tg), dstate_in=grad(ts),
                dq_norm_w=grad(tqw), dk_norm_w=grad(tkw))


def sparse_attention_layer(q, k_hat, v, g, sel, *, block=64, scale=None, eps=1e-6, q_norm_w=None,
                           q_positions=None):
    """The sparse layer's attention step for a fixed selection (sala_oracle.sparse_attention on
    q_hat = qk_norm(q), then the sigmoid gate). q, g [B, N, H, d] at positions q_positions
    (default 0..N-1); k_hat, v [B, L, Hkv, d]; sel [B, Hkv, nqb, topk] of block indices (-1
    ignored), indexed by the query's block position // block."""
    B, N, H, d = q.shape
    L, Hkv = k_hat.shape[1], k_hat.shape[2]
    group = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_hat = _qk_norm(q, q_norm_w, eps)
    qpos = np.arange(N) if q_positions is None else np.asarray(q_positions)
    o = torch.zeros((B, N, H, d), dtype=torch.float64)
    blocks_of_q = qpos // block
    for b in range(B):
        for i in np.unique(blocks_of_q):
            rows = torch.as_tensor(np.nonzero(blocks_of_q == i)[0])
            for gh in range(Hkv):
                blks = [int(j) for j in np.asarray(sel)[b, gh, i] if j >= 0]
                keys = np.concatenate([np.arange(j * block, min(L, (j + 1) * block)) for j in blks])
                K = k_hat[b, torch.as_tensor(keys), gh]  # [nk, d]
                V = v[b, torch.as_tensor(keys), gh]
                allowed = torch.as_tensor(keys[None, :] <= qpos[rows.numpy()][:, None])
                for h in range(gh * group, (gh + 1) * group):
                    s = (q_hat[b, rows, h] @ K.T) * scale
                    s = torch.where(allowed, s, torch.tensor(-math.inf, dtype=torch.float64))
                    o[b, rows, h] = torch.softmax(s, dim=1) @ V
    return o * torch.sigmoid(g)


def sparse_attention_grads(q, k_hat, v, g, sel, dout, *, block=64, scale=None, eps=1e-6,
                           q_norm_w=None, q_positions=None):
    """Gradients of <out, dout> for the sparse layer's attention step with a fixed selection.
    Returns dict(dq, dk_hat, dv, dg, dq_norm_w) as float64 numpy arrays (dq_norm_w None when
    no weight was given)."""
    tq, tk, tv, tg, tw = _t(q, True), _t(k_hat, True), _t(v, True), _t(g, True), _t(q_norm_w, True)
    out = sparse_attention_layer(tq, tk, tv, tg, sel, block=block, scale=scale, eps=eps, q_norm_w=tw,
                                 q_positions=q_positions)
    (out * _t(dout)).sum().backward()
    return dict(dq=tq.grad.numpy().copy(), dk_hat=tk.grad.numpy().copy(), dv=tv.grad.numpy().copy(),
                dg=tg.grad.numpy().copy(), dq_norm_w=None if tw is None else tw.grad.numpy().copy())


def key_norm(k, k_norm_w=None, eps=1e-6):
    """k_hat = qk_norm(k, k_norm_w): the normalisation the cache append applies (no RoPE in the
    sparse layer)."""
    return _qk_norm(k, k_norm_w, eps)


def key_norm_grads(k, dk_hat, k_norm_w=None, eps=1e-6):
    """Gradients of <key_norm(k), dk_hat>: dict(dk, dk_norm_w)."""
    tk, tw = _t(k, True), _t(k_norm_w, True)
    (key_norm(tk, tw, eps) * _t(dk_hat)).sum().backward()
    return dict(dk=tk.grad.numpy().copy(), dk_norm_w=None if tw is None else tw.grad.numpy().copy())
