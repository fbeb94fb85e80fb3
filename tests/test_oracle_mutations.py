"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check that the pins
in test_oracle_pins.py catch each one. This shows the pins are sensitive, not just passing."""

import numpy as np
import pytest

import oracle.sala_oracle as M
import test_oracle_pins as P


def _rope_wrong_sign(x, positions, base=10000.0):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    th = M.rope_inv_freq(d, base)
    pos = np.asarray(positions, np.float64)
    ang = pos * th if pos.ndim == 0 else pos[:, None, None] * th[None, None, :]
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., :h] * s + x[..., h:] * c], -1)


def _rope_interleaved(x, positions, base=10000.0):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    th = M.rope_inv_freq(d, base)
    pos = np.asarray(positions, np.float64)
    ang = pos * th if pos.ndim == 0 else pos[:, None, None] * th[None, None, :]
    c, s = np.cos(ang), np.sin(ang)
    y = x.copy()
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return y


def _linear_prefill_exclusive(q, k, v, g, *, pos0=0, rope_base=10000.0, eps=1e-6, state_in=None,
                              q_norm_w=None, k_norm_w=None):
    q, k, v, g = (np.asarray(a, np.float64) for a in (q, k, v, g))
    B, N, H, d = q.shape
    pos = pos0 + np.arange(N)
    qt = M.rope(M.qk_norm(q, eps=eps), pos, rope_base)
    kt = M.rope(M.qk_norm(k, eps=eps), pos, rope_base)
    S = np.zeros((B, H, d, d)) if state_in is None else np.array(state_in, np.float64)
    o = np.empty((B, N, H, d))
    for t in range(N):  # readout before the update: drops the diagonal term
        o[:, t] = np.einsum("bhi,bhij->bhj", qt[:, t], S)
        S += kt[:, t, :, :, None] * v[:, t, :, None, :]
    return o * M.sigmoid(g), S


def _linear_prefill_transposed(q, k, v, g, *, pos0=0, rope_base=10000.0, eps=1e-6, state_in=None,
                               q_norm_w=None, k_norm_w=None):
    q, k, v, g = (np.asarray(a, np.float64) for a in (q, k, v, g))
    B, N, H, d = q.shape
    pos = pos0 + np.arange(N)
    qt = M.rope(M.qk_norm(q, eps=eps), pos, rope_base)
    kt = M.rope(M.qk_norm(k, eps=eps), pos, rope_base)
    S = np.zeros((B, H, d, d)) if state_in is None else np.array(state_in, np.float64)
    o = np.empty((B, N, H, d))
    for t in range(N):
        S += kt[:, t, :, :, None] * v[:, t, :, None, :]
        o[:, t] = np.einsum("bhj,bhij->bhi", qt[:, t], S)  # q S^T
    return o * M.sigmoid(g), S


def _pool_sum(k_hat, block, n_blocks=None):
    return M.__dict__["_orig_pool"](k_hat, block, n_blocks) * block


def _select_row_high_ties(scores, i, topk, n_local):
    forced = {0} | set(range(max(0, i - n_local + 1), i + 1))
    cands = list(range(1, i - n_local + 1))
    r = topk - len(forced)
    chosen = cands if len(cands) <= r else sorted(cands, key=lambda j: (-scores[j], -j))[:r]
    sel = sorted(forced | set(chosen))
    return np.array(sel + [-1] * (topk - len(sel)))


def _sparse_attention_no_mask(q_hat, k_hat, v, sel, block, scale, q_positions=None):
    # causal mask inside the diagonal block dropped: every key of a selected block is used
    q_hat, k_hat, v = (np.asarray(a, np.float64) for a in (q_hat, k_hat, v))
    B, Nq, H, d = q_hat.shape
    L, Hkv = k_hat.shape[1], k_hat.shape[2]
    grp = H // Hkv
    o = np.empty((B, Nq, H, d))
    for b in range(B):
        for t in range(Nq):
            for h in range(H):
                gh = h // grp
                keys = np.concatenate([np.arange(j * block, min(L, (j + 1) * block))
                                       for j in sel[b, gh, t // block] if j >= 0])
                s = k_hat[b, keys, gh] @ q_hat[b, t, h] * scale
                w = np.exp(s - s.max())
                o[b, t, h] = (w / w.sum()) @ v[b, keys, gh]
    return o


def _qk_norm_l2(x, weight=None, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _sigmoid_missing(x):
    return np.ones_like(np.asarray(x, np.float64))


CASES = [
    ("rope", _rope_wrong_sign, [P.test_linear_worked_example, P.test_rope_invariants]),
    ("rope", _rope_interleaved, [P.test_rope_matches_complex_rotation]),
    ("linear_prefill", _linear_prefill_exclusive, [P.test_linear_worked_example]),
    ("linear_prefill", _linear_prefill_transposed, [P.test_linear_worked_example]),
    ("pool_keys", _pool_sum, [P.test_sparse_worked_example]),
    ("select_row", _select_row_high_ties, [lambda: P.test_selection_brute_force_with_ties(0)]),
    ("sparse_attention", _sparse_attention_no_mask, [P.test_sparse_worked_example]),
    ("qk_norm", _qk_norm_l2, [P.test_linear_worked_example, P.test_qk_norm_rms_one_and_scale_invariance]),
    ("sigmoid", _sigmoid_missing, [P.test_linear_worked_example, P.test_sigmoid_special_values]),
]


@pytest.mark.parametrize("name,mutant,pins", CASES, ids=[f"{c[0]}:{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setitem(M.__dict__, "_orig_pool", M.pool_keys)
    monkeypatch.setitem(M.__dict__, "_orig_attn", M.sparse_attention)
    monkeypatch.setattr(M, name, mutant)
    monkeypatch.setattr(P.O, name, mutant, raising=False)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
