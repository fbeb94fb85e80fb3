"""Pins of the CPU oracle to things other than itself: hand-derived worked examples, closed
forms, library special cases, brute force and invariants. CPU only.

Each pin is chosen so that a plausible slip in the oracle (dropped term, wrong sign or index,
transposed operand, missing scale or mask, wrong tie rule) fails at least one of them;
test_oracle_mutations.py plants such slips in the oracle and checks that they are caught.
"""

import itertools
import math

import numpy as np
import pytest

import oracle as O
from conftest import load_golden

RNG = np.random.default_rng(12345)


def rnd(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------ helpers (independent forms)


def closed_form_linear(qt, kt, v, S_in):
    """(Q K^T (.) M) V + Q S_in with M_ts = 1[s <= t], per (b, h): the masked-quadratic form."""
    B, N, H, d = qt.shape
    Hkv = kt.shape[2]
    grp = H // Hkv
    o = np.zeros((B, N, H, d))
    M = np.tril(np.ones((N, N)))
    for b in range(B):
        for h in range(H):
            gh = h // grp
            A = (qt[b, :, h] @ kt[b, :, gh].T) * M
            o[b, :, h] = A @ v[b, :, gh] + qt[b, :, h] @ S_in[b, gh]
    return o


def chunked_linear(qt, kt, v, S_in, C):
    """Chunked form: intra-chunk masked product plus inter-chunk running d x d state."""
    B, N, H, d = qt.shape
    o = np.zeros((B, N, H, d))
    S = S_in.copy()
    for c0 in range(0, N, C):
        c1 = min(N, c0 + C)
        M = np.tril(np.ones((c1 - c0, c1 - c0)))
        for b in range(B):
            for h in range(H):
                Qc, Kc, Vc = qt[b, c0:c1, h], kt[b, c0:c1, h], v[b, c0:c1, h]
                o[b, c0:c1, h] = ((Qc @ Kc.T) * M) @ Vc + Qc @ S[b, h]
        for b in range(B):
            for h in range(H):
                S[b, h] += kt[b, c0:c1, h].T @ v[b, c0:c1, h]
    return o, S


def prep(q, k, pos, base=10000.0, eps=1e-6):
    return O.rope(O.qk_norm(q, eps=eps), pos, base), O.rope(O.qk_norm(k, eps=eps), pos, base)


# ------------------------------------------------------------------ worked examples (golden)


def test_linear_worked_example():
    gx = load_golden("linear_worked_example.txt")
    q = np.array(gx["q"], float)[None, :, None, :]
    k = np.array(gx["k"], float)[None, :, None, :]
    v = np.array(gx["v"], float)[None, :, None, :]
    g = np.array(gx["g"], float)[None, :, None, :]
    out, S = O.linear_prefill(q, k, v, g, pos0=gx["pos0"], eps=gx["eps"])
    np.testing.assert_allclose(out[0, :, 0], np.array(gx["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], np.array(gx["state"]), rtol=0, atol=1e-14)


def test_sparse_worked_example():
    gx = load_golden("sparse_worked_example.txt")
    q = np.stack([np.array(gx["q_head0"], float), np.array(gx["q_head1"], float)], axis=1)[None]
    k = np.array(gx["k"], float)[None, :, None, :]
    v = np.array(gx["v"], float)[None, :, None, :]
    g = np.zeros_like(q)
    r = O.sparse_prefill(q, k, v, g, block=gx["block"], topk=gx["topk"], n_local=gx["n_local"],
                         eps=gx["eps"])
    np.testing.assert_allclose(r["k_bar"][0, 0], np.array(gx["k_bar"]), atol=1e-15)
    np.testing.assert_allclose(r["q_tilde"][0, 0, 3], np.array(gx["q_tilde_block3"]), atol=1e-15)
    assert r["sel"][0, 0].tolist() == gx["sel"]
    out = r["out"][0]
    np.testing.assert_allclose(out[7, 0], gx["out_t7_h0"], atol=1e-14)
    np.testing.assert_allclose(out[6, 0], gx["out_t6_h0"], atol=1e-14)
    np.testing.assert_allclose(out[7, 1], gx["out_t7_h1"], atol=1e-14)
    np.testing.assert_allclose(out[5, 0], gx["out_t5_h0"], atol=1e-14)


# ------------------------------------------------------------------ shared steps


def test_qk_norm_rms_one_and_scale_invariance():
    x = rnd(3, 5, 4, 64)
    y = O.qk_norm(x, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.qk_norm(7.5 * x, eps=0.0), y, rtol=1e-13)
    w = rnd(64)
    np.testing.assert_allclose(O.qk_norm(x, weight=w, eps=0.0), y * w, rtol=1e-13)
    # eps only matters at tiny magnitudes: x = 0 -> 0, and the 1e-6 default shifts N(0,1)
    # rows by ~5e-7 relative
    assert np.all(O.qk_norm(np.zeros((2, 8))) == 0)
    np.testing.assert_allclose(O.qk_norm(x), y, rtol=1e-5)


def test_rope_matches_complex_rotation():
    # Half-split RoPE is multiplication of z_i = x_i + i x_{i+d/2} by exp(i p theta_i).
    d, N = 16, 7
    x = rnd(N, 3, d)
    pos = np.arange(N) * 37 + 5
    theta = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(O.rope(x, pos), ref, atol=1e-12)


def test_rope_invariants():
    d = 128
    x = rnd(5, 2, d)
    y = rnd(5, 2, d)
    # p = 0 is the identity
    np.testing.assert_allclose(O.rope(x, np.zeros(5)), x, atol=0)
    # norm preserved
    pos = np.array([1, 10, 1000, 2 ** 20 - 1, 123456])
    np.testing.assert_allclose(np.linalg.norm(O.rope(x, pos), axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-12)
    # <R_m q, R_n k> depends on m - n only
    a = np.sum(O.rope(x, np.full(5, 17.0)) * O.rope(y, np.full(5, 5.0)), axis=-1)
    b = np.sum(O.rope(x, np.full(5, 1012.0)) * O.rope(y, np.full(5, 1000.0)), axis=-1)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)
    # theta_0 = 1 and theta_{d/2-1} = base^(-(d-2)/d)
    th = O.rope_inv_freq(d)
    assert th[0] == 1.0
    assert math.isclose(th[-1], 10000.0 ** (-(d - 2) / d), rel_tol=1e-15)


def test_sigmoid_special_values():
    from scipy.special import expit

    x = np.linspace(-30, 30, 101)
    np.testing.assert_allclose(O.sigmoid(x), expit(x), rtol=1e-14)
    assert O.sigmoid(0.0) == 0.5
    np.testing.assert_allclose(O.sigmoid(x) + O.sigmoid(-x), 1.0, rtol=1e-15)


# ------------------------------------------------------------------ linear layer


@pytest.mark.parametrize("B,N,H,Hkv,d", [(1, 9, 1, 1, 4), (2, 33, 3, 3, 8), (1, 40, 4, 2, 16)])
def test_linear_recurrence_equals_masked_quadratic(B, N, H, Hkv, d):
    q, k, v, g = rnd(B, N, H, d), rnd(B, N, Hkv, d), rnd(B, N, Hkv, d), rnd(B, N, H, d)
    S_in = rnd(B, Hkv, d, d)
    out, S = O.linear_prefill(q, k, v, g, pos0=3, state_in=S_in)
    qt, kt = prep(q, k, 3 + np.arange(N))
    ref = closed_form_linear(qt, kt, v, S_in)
    np.testing.assert_allclose(out / O.sigmoid(g), ref, rtol=1e-11, atol=1e-11)
    # final state = S_in + sum_t k_t^T v_t
    S_ref = S_in + np.einsum("bnhi,bnhj->bhij", kt, v)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C", [1, 16, 64, 100])
def test_linear_chunk_size_invariance(C):
    B, N, H, d = 1, 100, 2, 8
    q, k, v, g = rnd(B, N, H, d), rnd(B, N, H, d), rnd(B, N, H, d), rnd(B, N, H, d)
    S_in = rnd(B, H, d, d)
    out, S = O.linear_prefill(q, k, v, g, state_in=S_in)
    qt, kt = prep(q, k, np.arange(N))
    oc, Sc = chunked_linear(qt, kt, v, S_in, C)
    np.testing.assert_allclose(out / O.sigmoid(g), oc, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(S, Sc, rtol=1e-12, atol=1e-12)


def test_linear_prefill_then_decode_equals_longer_prefill():
    B, N, H, d = 2, 21, 3, 8
    q, k, v, g = rnd(B, N + 1, H, d), rnd(B, N + 1, H, d), rnd(B, N + 1, H, d), rnd(B, N + 1, H, d)
    full, S_full = O.linear_prefill(q, k, v, g)
    part, S_part = O.linear_prefill(q[:, :N], k[:, :N], v[:, :N], g[:, :N])
    dec, S_dec = O.linear_decode(q[:, N], k[:, N], v[:, N], g[:, N], S_part, N)
    np.testing.assert_allclose(dec, full[:, N], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_dec, S_full, rtol=1e-12, atol=1e-12)


def test_linear_split_prefill_resume():
    B, N, H, d = 1, 50, 2, 8
    q, k, v, g = rnd(B, N, H, d), rnd(B, N, H, d), rnd(B, N, H, d), rnd(B, N, H, d)
    full, S_full = O.linear_prefill(q, k, v, g)
    a, Sa = O.linear_prefill(q[:, :32], k[:, :32], v[:, :32], g[:, :32])
    b, Sb = O.linear_prefill(q[:, 32:], k[:, 32:], v[:, 32:], g[:, 32:], pos0=32, state_in=Sa)
    np.testing.assert_allclose(np.concatenate([a, b], axis=1), full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sb, S_full, rtol=1e-12, atol=1e-12)


def test_linear_is_linear_in_v():
    B, N, H, d = 1, 12, 1, 4
    q, k, g = rnd(B, N, H, d), rnd(B, N, H, d), rnd(B, N, H, d)
    v1, v2 = rnd(B, N, H, d), rnd(B, N, H, d)
    o1, _ = O.linear_prefill(q, k, v1, g)
    o2, _ = O.linear_prefill(q, k, v2, g)
    o3, _ = O.linear_prefill(q, k, 2 * v1 - 3 * v2, g)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------------ sparse layer


def repeat_kv(x, group):
    return np.repeat(x, group, axis=2)


@pytest.mark.parametrize("N,H,Hkv,d,block", [(64, 2, 1, 8, 8), (70, 4, 2, 16, 16), (37, 2, 2, 8, 4)])
def test_sparse_full_coverage_equals_dense_causal_sdpa(N, H, Hkv, d, block):
    import torch

    q, k, v, g = rnd(1, N, H, d), rnd(1, N, Hkv, d), rnd(1, N, Hkv, d), rnd(1, N, H, d)
    nqb = -(-N // block)
    r = O.sparse_prefill(q, k, v, g, block=block, topk=nqb, n_local=1)
    qh, kh = O.qk_norm(q), O.qk_norm(k)
    grp = H // Hkv
    Q = torch.from_numpy(qh[0].transpose(1, 0, 2).copy())  # [H, N, d]
    K = torch.from_numpy(repeat_kv(kh, grp)[0].transpose(1, 0, 2).copy())
    V = torch.from_numpy(repeat_kv(v, grp)[0].transpose(1, 0, 2).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True).numpy()
    ref = ref.transpose(1, 0, 2)[None] * O.sigmoid(g)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)
    # every causal block is selected
    for i in range(nqb):
        assert sorted(j for j in r["sel"][0, 0, i] if j >= 0) == list(range(i + 1))


@pytest.mark.parametrize("N,H,Hkv,d,q0", [(50, 2, 1, 8, 0), (70, 4, 2, 16, 0), (40, 4, 2, 8, 33), (65, 2, 2, 8, 64)])
def test_dense_attention_equals_torch_sdpa(N, H, Hkv, d, q0):
    """The dense-mode definition against torch's scaled_dot_product_attention: causal for a
    prompt (q0 = 0), an explicit position mask for queries at positions q0 .. N-1 of a longer
    cache; and equal to block attention with every causal block selected."""
    import torch

    q, k, v = rnd(1, N - q0, H, d), rnd(1, N, Hkv, d), rnd(1, N, Hkv, d)
    qh, kh = O.qk_norm(q), O.qk_norm(k)
    pos = np.arange(q0, N)
    o = O.dense_attention(qh, kh, v, 1.0 / np.sqrt(d), q_positions=pos)
    grp = H // Hkv
    Q = torch.from_numpy(qh[0].transpose(1, 0, 2).copy())
    K = torch.from_numpy(repeat_kv(kh, grp)[0].transpose(1, 0, 2).copy())
    V = torch.from_numpy(repeat_kv(v, grp)[0].transpose(1, 0, 2).copy())
    mask = torch.from_numpy(np.arange(N)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask).numpy()
    np.testing.assert_allclose(o, ref.transpose(1, 0, 2)[None], rtol=1e-11, atol=1e-12)
    block = 8
    nqb = -(-N // block)
    sel = np.full((1, Hkv, nqb, nqb), -1)
    for i in range(nqb):
        sel[0, :, i, : i + 1] = np.arange(i + 1)
    ob = O.sparse_attention(qh, kh, v, sel, block, 1.0 / np.sqrt(d), q_positions=pos)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)


def test_pooled_score_equals_mean_of_pair_products():
    beta, d, H, Hkv = 8, 16, 4, 2
    q = rnd(1, 4 * beta, H, d)
    k = rnd(1, 4 * beta, Hkv, d)
    qh, kh = O.qk_norm(q), O.qk_norm(k)
    kb = O.pool_keys(kh, beta)
    qt = O.query_block_tilde(qh, beta, Hkv)
    for gh in range(Hkv):
        for i in range(4):
            for j in range(4):
                heads = range(gh * 2, gh * 2 + 2)
                pairs = sum(qh[0, i * beta + t, h] @ kh[0, j * beta + s, gh]
                            for h in heads for t in range(beta) for s in range(beta))
                assert math.isclose(O.block_scores(qt[0, gh, i], kb[0, gh, j:j + 1])[0],
                                    pairs / beta ** 2, rel_tol=1e-11, abs_tol=1e-12)


def test_query_block_tilde_ragged_last_block():
    q = rnd(1, 20, 2, 4)
    qt = O.query_block_tilde(q, 8, 1)
    np.testing.assert_allclose(qt[0, 0, 2], q[0, 16:20].mean(axis=0).sum(axis=0), rtol=1e-14)


def brute_force_selection(scores, i, topk, n_local):
    """Largest-sum subset of the candidates of size r; among subsets of equal sum, the one
    whose sorted index list is lexicographically smallest (= lowest indices win ties)."""
    forced = {0} | set(range(max(0, i - n_local + 1), i + 1))
    cands = list(range(1, i - n_local + 1))
    r = topk - len(forced)
    if len(cands) <= r:
        best = tuple(cands)
    else:
        best, best_sum = None, -np.inf
        for sub in itertools.combinations(cands, r):  # lexicographic order
            ssum = sum(scores[j] for j in sub)
            if ssum > best_sum:
                best, best_sum = sub, ssum
    sel = sorted(forced | set(best))
    return sel + [-1] * (topk - len(sel))


def iterative_argmax_selection(scores, i, topk, n_local):
    forced = {0} | set(range(max(0, i - n_local + 1), i + 1))
    s = np.array([scores[j] if 1 <= j <= i - n_local else -np.inf for j in range(i + 1)])
    chosen = []
    for _ in range(topk - len(forced)):
        j = int(np.argmax(s))  # first maximum: lowest index on ties
        if s[j] == -np.inf:
            break
        chosen.append(j)
        s[j] = -np.inf
    sel = sorted(forced | set(chosen))
    return sel + [-1] * (topk - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    for i in range(0, 11):
        for topk, n_local in [(3, 1), (4, 2), (5, 1), (6, 2)]:
            if topk < 1 + min(n_local, i):
                continue
            # coarse integer scores create many exact ties; -0.0 and +0.0 must tie too
            sc = rng.integers(-3, 4, size=i + 1).astype(float)
            sc[sc == 0] = rng.choice([0.0, -0.0])
            got = O.select_row(sc, i, topk, n_local).tolist()
            assert got == brute_force_selection(sc, i, topk, n_local)
            assert got == iterative_argmax_selection(sc, i, topk, n_local)


def test_selection_invariants_and_planted_needles():
    rng = np.random.default_rng(7)
    beta, d, H, Hkv, nb = 4, 16, 2, 1, 40
    N = nb * beta
    q = rng.standard_normal((1, N, H, d)) * 0.1
    k = rng.standard_normal((1, N, Hkv, d)) * 0.1
    # plant: every query block points at direction e0; blocks 7, 19, 23 (keys) align with e0
    q[..., 0] += 5.0
    for j in (7, 19, 23):
        k[0, j * beta:(j + 1) * beta, 0, 0] += 5.0
    qh, kh = O.qk_norm(q), O.qk_norm(k)
    sel = O.select_blocks(O.query_block_tilde(qh, beta, Hkv), O.pool_keys(kh, beta), 6, 2)
    for i in range(nb):
        row = [j for j in sel[0, 0, i] if j >= 0]
        assert row == sorted(set(row)) and all(0 <= j <= i for j in row)
        assert 0 in row and i in row and (i == 0 or i - 1 in row)
        assert len(row) == min(6, i + 1)
        for j in (7, 19, 23):
            if j <= i - 2:
                assert j in row
    # duplicated key blocks tie exactly: the lower index wins
    k2 = kh.copy()
    k2[0, 9 * beta:10 * beta] = k2[0, 7 * beta:8 * beta]
    sel2 = O.select_blocks(O.query_block_tilde(qh, beta, Hkv), O.pool_keys(k2, beta), 3, 1)
    assert 7 in sel2[0, 0, 30] and 9 not in sel2[0, 0, 30]


def test_sparse_attention_ignores_order_of_selected_blocks():
    N, H, d, beta = 48, 2, 8, 8
    q, k, v = rnd(1, N, H, d), rnd(1, N, 1, d), rnd(1, N, 1, d)
    qh, kh = O.qk_norm(q), O.qk_norm(k)
    sel = O.select_blocks(O.query_block_tilde(qh, beta, 1), O.pool_keys(kh, beta), 3, 1)
    a = O.sparse_attention(qh, kh, v, sel, beta, 0.3)
    sel_rev = sel.copy()
    sel_rev[..., :] = sel[..., ::-1]
    b = O.sparse_attention(qh, kh, v, sel_rev, beta, 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_sparse_decode_equals_prefill_last_row_when_dense():
    # with top-k covering every block, selection is irrelevant and decode at p = N must equal
    # the last row of a prefill over N + 1 tokens
    N, H, Hkv, d, beta = 45, 4, 2, 8, 8
    q, k, v, g = rnd(1, N + 1, H, d), rnd(1, N + 1, Hkv, d), rnd(1, N + 1, Hkv, d), rnd(1, N + 1, H, d)
    nqb = -(-(N + 1) // beta)
    full = O.sparse_prefill(q, k, v, g, block=beta, topk=nqb, n_local=1)["out"]
    kh = O.qk_norm(k)
    kc = kh.transpose(0, 2, 1, 3)  # cache layout [B, Hkv, L, d]
    vc = v.transpose(0, 2, 1, 3)
    dec = O.sparse_decode(q[:, N], k[:, N], v[:, N], g[:, N], kc[:, :, :N], vc[:, :, :N], N + 1,
                          block=beta, topk=nqb, n_local=1)
    np.testing.assert_allclose(dec["out"], full[:, N], rtol=1e-12, atol=1e-13)


def test_sparse_decode_selection_matches_brute_force():
    rng = np.random.default_rng(3)
    beta, d, H, Hkv, L = 4, 8, 4, 2, 4 * 13 + 3
    q, g = rng.standard_normal((2, H, d)), np.zeros((2, H, d))
    kn, vn = rng.standard_normal((2, Hkv, d)), rng.standard_normal((2, Hkv, d))
    kc = O.qk_norm(rng.standard_normal((2, Hkv, L, d)))
    vc = rng.standard_normal((2, Hkv, L, d))
    r = O.sparse_decode(q, kn, vn, g, kc, vc, L, block=beta, topk=5, n_local=2)
    p = L - 1
    i = p // beta
    qh = O.qk_norm(q)
    for b in range(2):
        for gh in range(Hkv):
            qt = qh[b, gh * 2:(gh + 1) * 2].sum(axis=0)
            kb = kc[b, gh, : (i - 1) * beta].reshape(i - 1, beta, d).mean(axis=1)
            sc = list(kb @ qt) + [0.0, 0.0]
            assert r["sel"][b, gh].tolist() == brute_force_selection(sc, i, 5, 2)
