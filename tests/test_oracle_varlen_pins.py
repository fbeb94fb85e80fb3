"""Pins of the packed variable-length (varlen) oracle functions. CPU only.

The varlen functions run each packed sequence through the single-sequence oracle. What could
go wrong is the packing: rows of one sequence read by another, a state or position carried
across sequences, a wrong offset. The pins check, against the batched form of the oracle (a
different code path: numpy over the batch dimension) and against invariants:
- equal lengths: the packed batch equals the [B, N] batch call;
- independence: changing one sequence's inputs leaves every other sequence's outputs
  bit-identical, and reordering the sequences reorders the outputs;
- positions: a sequence starting at pos0 = p with the state of its first p tokens equals the
  last tokens of the whole sequence (the linear recurrence read in two calls);
- empty sequences pass their state through.
"""

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(77)


def rnd(*shape):
    return RNG.standard_normal(shape)


def _lin_inputs(T, H=2, d=8):
    return rnd(T, H, d), rnd(T, H, d), rnd(T, H, d), rnd(T, H, d)


def test_linear_varlen_equal_lengths_equals_batched():
    B, N, H, d = 3, 7, 2, 8
    q, k, v, g = _lin_inputs(B * N, H, d)
    s_in = rnd(B, H, d, d)
    out, S = O.linear_prefill_varlen(q, k, v, g, [N] * B, [5] * B, state_in=s_in)
    ref, Sr = O.linear_prefill(q.reshape(B, N, H, d), k.reshape(B, N, H, d), v.reshape(B, N, H, d),
                               g.reshape(B, N, H, d), pos0=5, state_in=s_in)
    np.testing.assert_allclose(out, ref.reshape(B * N, H, d), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, Sr, rtol=0, atol=1e-12)


def test_linear_varlen_sequences_independent_and_reorderable():
    lens, pos = [5, 0, 9, 3], [0, 4, 17, 2]
    q, k, v, g = _lin_inputs(sum(lens))
    s_in = rnd(4, 2, 8, 8)
    out, S = O.linear_prefill_varlen(q, k, v, g, lens, pos, state_in=s_in)
    # perturb sequence 2 (rows 5..13): the others are bit-identical
    q2 = q.copy()
    q2[5:14] += 1.0
    k2 = k.copy()
    k2[5:14] *= -1.0
    out2, S2 = O.linear_prefill_varlen(q2, k2, v, g, lens, pos, state_in=s_in)
    assert np.array_equal(out2[:5], out[:5]) and np.array_equal(out2[14:], out[14:])
    assert np.array_equal(S2[[0, 1, 3]], S[[0, 1, 3]])
    assert not np.array_equal(out2[5:14], out[5:14])
    # the empty sequence keeps its state
    assert np.array_equal(S[1], s_in[1])
    # reversed order of the sequences: outputs and states follow
    order = [3, 2, 1, 0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    out3, S3 = O.linear_prefill_varlen(q[rows], k[rows], v[rows], g[rows], [lens[s] for s in order],
                                       [pos[s] for s in order], state_in=s_in[order])
    np.testing.assert_allclose(out3, out[rows], rtol=0, atol=0)
    np.testing.assert_allclose(S3, S[order], rtol=0, atol=0)


def test_linear_varlen_pos0_continues_the_sequence():
    """Sequence 1 holds the last 6 tokens of a 10-token prompt, at pos0 = 4 with the state of
    the first 4 tokens: it equals the whole prompt's last 6 outputs."""
    q, k, v, g = _lin_inputs(10)
    full, S_full = O.linear_prefill(q[None], k[None], v[None], g[None], pos0=0)
    _, S4 = O.linear_prefill(q[None, :4], k[None, :4], v[None, :4], g[None, :4], pos0=0)
    qa, ka, va, ga = _lin_inputs(3)
    s_in = np.concatenate([np.zeros((1, 2, 8, 8)), S4], axis=0)
    out, S = O.linear_prefill_varlen(np.concatenate([qa, q[4:]]), np.concatenate([ka, k[4:]]),
                                     np.concatenate([va, v[4:]]), np.concatenate([ga, g[4:]]), [3, 6], [0, 4],
                                     state_in=s_in)
    np.testing.assert_allclose(out[3:], full[0, 4:], rtol=0, atol=1e-10)
    np.testing.assert_allclose(S[1], S_full[0], rtol=0, atol=1e-10)


def _sp_inputs(T, Hq=4, Hkv=2, d=8):
    return rnd(T, Hq, d), rnd(T, Hkv, d), rnd(T, Hkv, d), rnd(T, Hq, d)


def test_sparse_varlen_equal_lengths_equals_batched():
    B, N, Hq, Hkv, d, blk = 2, 20, 4, 2, 8, 4
    q, k, v, g = _sp_inputs(B * N, Hq, Hkv, d)
    r = O.sparse_prefill_varlen(q, k, v, g, [N] * B, block=blk, topk=3, n_local=2)
    ref = O.sparse_prefill(q.reshape(B, N, Hq, d), k.reshape(B, N, Hkv, d), v.reshape(B, N, Hkv, d),
                           g.reshape(B, N, Hq, d), block=blk, topk=3, n_local=2)
    np.testing.assert_allclose(r["out"], ref["out"].reshape(B * N, Hq, d), rtol=0, atol=1e-12)
    for s in range(B):
        assert np.array_equal(r["sel"][s], ref["sel"][s])


def test_sparse_varlen_sequences_independent():
    lens, blk = [9, 0, 16, 5], 4
    q, k, v, g = _sp_inputs(sum(lens))
    r = O.sparse_prefill_varlen(q, k, v, g, lens, block=blk, topk=3, n_local=2)
    k2 = k.copy()
    k2[9:25] += 2.0  # sequence 2's keys
    r2 = O.sparse_prefill_varlen(q, k2, v, g, lens, block=blk, topk=3, n_local=2)
    assert np.array_equal(r2["out"][:9], r["out"][:9]) and np.array_equal(r2["out"][25:], r["out"][25:])
    assert not np.array_equal(r2["out"][9:25], r["out"][9:25])
    assert r["sel"][1].shape == (2, 0, 3)
    # a sequence alone gives the same rows as inside the batch
    alone = O.sparse_prefill(q[None, 9:25], k[None, 9:25], v[None, 9:25], g[None, 9:25], block=blk, topk=3,
                             n_local=2)
    np.testing.assert_allclose(r["out"][9:25], alone["out"][0], rtol=0, atol=0)
