"""GPU parity of the block-selection paths that the workload-shaped tests do not reach, against
the oracle on the same seeded inputs:

* a short continuation inside one query block after a cached prefix (2, 10 or 64 query tokens
  at position 640, batch 2): the selection ranks candidates by the block mean of those
  queries, not by a single token's query;
* decode selections past the two-level range (the score row plus one exact radix select per
  row): top-256 at a 300K-token context, and a context of more than 16,384 candidate blocks.

Selections are bit-exact up to the margin rule; outputs within 1e-2 * max|ref| of the oracle's
attention on the GPU's selection."""

import math

import numpy as np
import pytest

import oracle as O
from hybrid_sparse_linear_causal_amd.inputs import host_normal
from sala_testutil import assert_rel, check_selection, dev, host, oracle_decode_on_selection

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


@pytest.mark.parametrize("n_q,topk", [(2, 6), (10, 6), (64, 6), (10, 4)])
def test_continuation_in_one_block(S, n_q, topk):
    """Prefix of 640 tokens appended first, then n_q tokens appended, selected and attended;
    against the oracle's prefill of the whole prompt (its last query block)."""
    import torch

    B, Hq, Hkv, d, n_local, P = 2, 8, 2, 128, 2, 640
    N = P + n_q
    print(f"continuation n_q={n_q} topk={topk}", flush=True)
    q = host_normal(900 + n_q, 0, (B, N, Hq, d))
    k = host_normal(900 + n_q, 1, (B, N, Hkv, d))
    v = host_normal(900 + n_q, 2, (B, N, Hkv, d))
    g = host_normal(900 + n_q, 3, (B, N, Hq, d))
    ref = O.sparse_prefill(q, k, v, g, block=64, topk=topk, n_local=n_local)
    cap = ((N + 63) // 64) * 64
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append(dev(k[:, :P], "bf16"), dev(v[:, :P], "bf16"), kc, vc, kp, P, n_heads=Hq)
    S.kv_append(dev(k[:, P:], "bf16"), dev(v[:, P:], "bf16"), kc, vc, kp, N, n_heads=Hq)
    Q = dev(q[:, P:], "bf16")
    sel = S.block_select(Q, kp, N, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local)
    out = S.sparse_attn(Q, kc, vc, dev(g[:, P:], "bf16"), sel, N, n_local=n_local)
    gsel = sel.cpu().numpy()
    i = P // 64
    assert gsel.shape == (B, Hkv, 1, topk)
    qt, kb = ref["q_tilde"], ref["k_bar"]
    nm = check_selection(gsel, ref["sel"][:, :, i:i + 1],
                         lambda b, gg, ii: {j: float(qt[b, gg, ii] @ kb[b, gg, j]) for j in range(ii - 1)},
                         topk, n_local, first_block=i)
    sel_full = ref["sel"].copy()
    sel_full[:, :, i:i + 1] = gsel
    o_ref = O.sparse_attention(O.qk_norm(q), ref["k_hat"], v, sel_full, 64, 1.0 / math.sqrt(d)) * O.sigmoid(g)
    e = assert_rel(host(out), o_ref[:, P:], 1e-2, "out")
    print(f"  margin rows {nm}, rel err {e:.2e}", flush=True)


@pytest.mark.parametrize("L,topk", [(64 * 4700 + 21, 256),          # 253 slots over 10 slices
                                    (64 * 16500 + 5, 64)])          # more than 16,384 candidates
def test_decode_select_beyond_two_level(S, L, topk):
    """Decode at p = L - 1 over a seeded cache of already-normalised keys, B = 1, one KV
    group of 4 heads: selection and output against the oracle's decode."""
    import torch

    B, Hq, Hkv, d, n_local = 1, 4, 1, 128, 2
    print(f"decode select L={L} topk={topk}", flush=True)
    cap = ((L + 63) // 64) * 64
    kc_h = host_normal(950 + topk, 5, (B, Hkv, L - 1, d))
    vc_h = host_normal(950 + topk, 6, (B, Hkv, L - 1, d))
    q = host_normal(950 + topk, 0, (B, 1, Hq, d))
    kn = host_normal(950 + topk, 1, (B, 1, Hkv, d))
    vn = host_normal(950 + topk, 2, (B, 1, Hkv, d))
    g = host_normal(950 + topk, 3, (B, 1, Hq, d))
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :, :L - 1] = dev(kc_h, "bf16")
    vc[:, :, :L - 1] = dev(vc_h, "bf16")
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_pool(kc, kp, L - 1, 0, (L - 1) // 64)
    S.kv_append(dev(kn, "bf16"), dev(vn, "bf16"), kc, vc, kp, L, n_heads=Hq)
    Q = dev(q, "bf16")
    sel = S.block_select(Q, kp, L, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local)
    out = S.sparse_attn(Q, kc, vc, dev(g, "bf16"), sel, L, n_local=n_local)
    gsel = sel.cpu().numpy()
    i = (L - 1) // 64
    kb = O.pool_keys(kc_h.transpose(0, 2, 1, 3), 64)  # the cache holds normalised keys already
    ref = O.sparse_decode(q[:, 0], kn[:, 0], vn[:, 0], g[:, 0], kc_h, vc_h, L, block=64, topk=topk,
                          n_local=n_local, k_bar=kb)
    qh = O.qk_norm(q[0, 0])
    sc = kb[0, 0, : i - 1] @ qh.sum(axis=0)
    nm = check_selection(gsel, ref["sel"][:, :, None],
                         lambda bb, gg, ii: {j: float(sc[j]) for j in range(len(sc))}, topk, n_local,
                         first_block=i)
    o2 = oracle_decode_on_selection(qh, kc_h[0, 0], vc_h[0, 0], O.qk_norm(kn[0, 0, 0]), vn[0, 0, 0],
                                    gsel[0, 0, 0], 1.0 / math.sqrt(d))
    e = assert_rel(host(out)[0, 0], o2 * O.sigmoid(g[0, 0]), 1e-2, "decode out on the gpu selection")
    print(f"  margin rows {nm}, rel err {e:.2e}", flush=True)


def _check_scores(sel, scores, ref_score, first_block, n_local, what):
    """sel_scores beside sel: +inf for forced blocks, -inf for padding, and the candidate's score
    (fp32, against the oracle's float64 q~ . k_bar) for chosen candidates."""
    B, G, R, K = sel.shape
    errs = []
    for b in range(B):
        for g in range(G):
            for r in range(R):
                i = first_block + r
                forced = {0} | set(range(max(0, i - n_local + 1), i + 1))
                row_ref = []
                for x in range(K):
                    j = int(sel[b, g, r, x])
                    if j < 0:
                        assert scores[b, g, r, x] == -np.inf, (what, b, g, i, x)
                    elif j in forced:
                        assert scores[b, g, r, x] == np.inf, (what, b, g, i, x)
                    else:
                        row_ref.append((scores[b, g, r, x], ref_score(b, g, i, j)))
                if row_ref:
                    got, want = np.array(row_ref).T
                    errs.append(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))
    assert errs and max(errs) <= 1e-4, (what, max(errs) if errs else None)
    return max(errs)


def test_selection_scores(S):
    """The optional scores output on the selection paths: prefill rows (score tiles and the
    per-row radix select), decode rows inside the two-level range (slice winners merged by lane
    networks, and by radix thresholds), and a decode row past it (score row and the long-row
    select)."""
    import torch

    d, n_local = 128, 2
    # prefill: 40 query blocks, 2 KV groups of 4 heads, top-6
    B, N, Hq, Hkv, topk = 1, 64 * 40 + 17, 8, 2, 6
    q = host_normal(970, 0, (B, N, Hq, d))
    k = host_normal(970, 1, (B, N, Hkv, d))
    cap = ((N + 63) // 64) * 64
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append(dev(k, "bf16"), dev(k, "bf16"), kc, vc, kp, N, n_heads=Hq)
    nqb = (N + 63) // 64
    scores = torch.empty((B, Hkv, nqb, topk), dtype=torch.float32, device="cuda")
    sel = S.block_select(dev(q, "bf16"), kp, N, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local, sel_scores=scores)
    qt = O.query_block_tilde(O.qk_norm(q), 64, Hkv)
    kb = O.pool_keys(O.qk_norm(k), 64)
    e = _check_scores(sel.cpu().numpy(), scores.cpu().numpy(), lambda b, g, i, j: float(qt[b, g, i] @ kb[b, g, j]), 0,
                      n_local, "prefill")
    print(f"  prefill rel err {e:.2e}", flush=True)
    # decode rows: two-level with the lane-network levels (4,000 blocks, top-16) and with the radix
    # levels (3,000 blocks, top-100), and beyond the two-level range (5,000 blocks, top-256)
    for L, topk in ((64 * 4000 + 9, 16), (64 * 3000 + 9, 100), (64 * 5000 + 9, 256)):
        B, Hq, Hkv = 2, 8, 2
        kc_h = host_normal(971, 5, (B, Hkv, L, d))
        qd = host_normal(971, 0, (B, 1, Hq, d))
        kc = torch.zeros((B, Hkv, cap := ((L + 63) // 64) * 64, d), dtype=torch.bfloat16, device="cuda")
        kc[:, :, :L] = dev(kc_h, "bf16")
        kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
        S.kv_pool(kc, kp, L, 0, (L - 1) // 64)
        scores = torch.empty((B, Hkv, 1, topk), dtype=torch.float32, device="cuda")
        sel = S.block_select(dev(qd, "bf16"), kp, L, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local,
                             sel_scores=scores)
        qh = O.qk_norm(qd[:, 0])
        G = Hq // Hkv
        kbd = O.pool_keys(kc_h.transpose(0, 2, 1, 3), 64)
        e = _check_scores(sel.cpu().numpy(), scores.cpu().numpy(),
                          lambda b, g, i, j: float(qh[b, g * G:(g + 1) * G].sum(axis=0) @ kbd[b, g, j]),
                          (L - 1) // 64, n_local, f"decode L={L}")
        print(f"  decode L={L} top-{topk} rel err {e:.2e}", flush=True)
