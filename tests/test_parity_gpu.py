"""GPU parity: every libsala entry point against the CPU oracle on the same seeded inputs, at
sizes the oracle finishes in seconds that still span several tiles, segments and a ragged
tail. Tolerances: max|gpu - ref| <= 1e-2 * max|ref| (bf16 inputs), 1e-4 * max|ref| (f32);
block selections bit-exact up to the margin rule."""

import numpy as np
import pytest

import oracle as O
from hybrid_sparse_linear_causal_amd.inputs import host_normal
from sala_testutil import assert_rel, check_selection, dev, host, oracle_decode_on_selection

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


def lin_inputs(seed, B, N, H, d, dtype):
    return [host_normal(seed, tid, (B, N, H, d), dtype) for tid in range(4)]


# ---------------------------------------------------------------- linear layer prefill


@pytest.mark.parametrize("B,N,H,d,dtype,pos0,with_state,with_w", [
    (1, 512, 2, 64, "f32", 0, False, False),        # tiny workload shape
    (1, 333, 3, 128, "f32", 17, True, True),
    (1, 1000, 2, 128, "bf16", 0, False, False),     # 16 segments, ragged last chunk
    (2, 777, 3, 128, "bf16", 123, True, True),
    (1, 4096, 4, 128, "bf16", 0, True, False),
    (1, 64, 1, 128, "bf16", 5, False, False),       # exactly one chunk
    (1, 1, 2, 128, "bf16", 9, True, False),         # a single token
])
def test_linear_prefill(S, B, N, H, d, dtype, pos0, with_state, with_w):
    print(f"linear_prefill B={B} N={N} H={H} d={d} {dtype}", flush=True)
    q, k, v, g = lin_inputs(7 + N, B, N, H, d, dtype)
    s_in = host_normal(99, 4, (B, H, d, d), "f32", std=8.0) if with_state else None
    qw = (1.0 + 0.25 * host_normal(5, 8, (d,), "f32")) if with_w else None
    kw = (1.0 + 0.25 * host_normal(5, 9, (d,), "f32")) if with_w else None
    ref, S_ref = O.linear_prefill(q, k, v, g, pos0=pos0, state_in=s_in, q_norm_w=qw, k_norm_w=kw)
    out, st = S.linear_prefill(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g, dtype), pos0=pos0,
                               state_in=None if s_in is None else dev(s_in, "f32"),
                               q_norm_w=None if qw is None else dev(qw, "f32"),
                               k_norm_w=None if kw is None else dev(kw, "f32"))
    assert_rel(host(out), ref, TOL[dtype], "out")
    assert_rel(host(st), S_ref, TOL[dtype], "state")


def test_linear_prefill_empty_passes_state(S):
    import torch

    s_in = dev(host_normal(1, 4, (1, 2, 128, 128), "f32"), "f32")
    z = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    out, st = S.linear_prefill(z, z, z, z, state_in=s_in)
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(st, s_in)
    # no state_in: the state of an empty sequence is zero
    st2 = torch.full((1, 2, 128, 128), 7.0, dtype=torch.float32, device="cuda")
    S.linear_prefill(z, z, z, z, state_out=st2)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(st2)) == 0


def test_linear_state_alias_and_split_prefill(S):
    """state_out aliasing state_in, and a prefill split at a chunk boundary (with pos0 and the
    carried state) equals the one-shot prefill."""
    import torch

    B, N, H, d = 1, 3000, 2, 128
    q, k, v, g = lin_inputs(31, B, N, H, d, "bf16")
    ref, S_ref = O.linear_prefill(q, k, v, g)
    Q, K, V, G = (dev(x, "bf16") for x in (q, k, v, g))
    st = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    cut = 1280
    o1, _ = S.linear_prefill(Q[:, :cut].contiguous(), K[:, :cut].contiguous(), V[:, :cut].contiguous(),
                             G[:, :cut].contiguous(), state_in=st, state_out=st)
    o2, _ = S.linear_prefill(Q[:, cut:].contiguous(), K[:, cut:].contiguous(), V[:, cut:].contiguous(),
                             G[:, cut:].contiguous(), pos0=cut, state_in=st, state_out=st)
    assert_rel(np.concatenate([host(o1), host(o2)], axis=1), ref, 1e-2, "split out")
    assert_rel(host(st), S_ref, 1e-2, "split state")


# ---------------------------------------------------------------- linear layer decode


@pytest.mark.parametrize("B,H,d,dtype,pos", [(3, 4, 128, "bf16", 1_000_003), (2, 3, 64, "f32", 77),
                                             (8, 32, 128, "bf16", 1_048_575), (1, 2, 128, "f32", 0)])
def test_linear_decode(S, B, H, d, dtype, pos):
    print(f"linear_decode B={B} H={H} d={d} {dtype} pos={pos}", flush=True)
    q, k, v, g = (host_normal(40 + pos % 97, t, (B, H, d), dtype) for t in range(4))
    S0 = host_normal(41, 4, (B, H, d, d), "f32", std=32.0)
    ref, S_ref = O.linear_decode(q, k, v, g, S0, pos)
    st = dev(S0, "f32")
    out = S.linear_decode_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g, dtype), st, pos)
    assert_rel(host(out), ref, TOL[dtype], "out")
    assert_rel(host(st), S_ref, 1e-5, "state")


def test_linear_prefill_then_decode(S):
    B, N, H, d = 1, 700, 2, 128
    q, k, v, g = lin_inputs(55, B, N + 1, H, d, "bf16")
    ref, S_ref = O.linear_prefill(q, k, v, g)
    out, st = S.linear_prefill(*(dev(x[:, :N], "bf16") for x in (q, k, v, g)))
    o = S.linear_decode_step(*(dev(x[:, N], "bf16") for x in (q, k, v, g)), st, N)
    assert_rel(host(o), ref[:, N], 1e-2, "decode after prefill")
    assert_rel(host(st), S_ref, 1e-2, "state")


# ---------------------------------------------------------------- sparse layer: cache + selection


def sparse_case(seed, B, N, Hq, Hkv, d, dtype):
    q = host_normal(seed, 0, (B, N, Hq, d), dtype)
    k = host_normal(seed, 1, (B, N, Hkv, d), dtype)
    v = host_normal(seed, 2, (B, N, Hkv, d), dtype)
    g = host_normal(seed, 3, (B, N, Hq, d), dtype)
    return q, k, v, g


def gpu_sparse_prefill(S, q, k, v, g, dtype, topk, n_local, cap=None):
    import torch

    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    cap = cap or ((N + 63) // 64) * 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros((B, Hkv, cap, d), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append(dev(k, dtype), dev(v, dtype), kc, vc, kp, N)
    Q = dev(q, dtype)
    sel = S.block_select(Q, kp, N, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local)
    out = S.sparse_attn(Q, kc, vc, dev(g, dtype), sel, N, n_local=n_local)
    return dict(out=out, sel=sel, kc=kc, vc=vc, kp=kp)


def oracle_scores(ref):
    qt, kb = ref["q_tilde"], ref["k_bar"]

    def fn(b, g, i):
        nb = max(i, 1)
        return {j: float(qt[b, g, i] @ kb[b, g, j]) for j in range(min(nb, kb.shape[2]))}

    return fn


@pytest.mark.parametrize("B,N,Hq,Hkv,dtype", [(2, 300, 4, 2, "bf16"), (1, 130, 2, 1, "f32")])
def test_kv_append_and_pool(S, B, N, Hq, Hkv, dtype):
    d = 128
    k = host_normal(3, 1, (B, N, Hkv, d), dtype)
    v = host_normal(3, 2, (B, N, Hkv, d), dtype)
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cap = 384
    kc = torch.zeros((B, Hkv, cap, d), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    # two appends: a prefill of N-1 tokens, then one decode token
    S.kv_append(dev(k[:, :N - 1], dtype), dev(v[:, :N - 1], dtype), kc, vc, kp, N - 1)
    S.kv_append(dev(k[:, N - 1:], dtype), dev(v[:, N - 1:], dtype), kc, vc, kp, N)
    kh = O.qk_norm(k)
    assert_rel(host(kc)[:, :, :N], kh.transpose(0, 2, 1, 3), 2 ** -8 if dtype == "bf16" else 1e-6, "k cache")
    assert np.array_equal(host(vc)[:, :, :N], v.transpose(0, 2, 1, 3).astype(np.float64))
    nb = N // 64
    assert_rel(host(kp)[:, :, :nb], O.pool_keys(kh, 64), 2 ** -9 if dtype == "bf16" else 1e-6, "pool")
    assert np.all(host(kp)[:, :, nb:] == 0)  # incomplete block not pooled
    # rebuilding the pools from the cache contents
    kp2 = torch.zeros_like(kp)
    S.kv_pool(kc, kp2, N, 0, nb)
    assert_rel(host(kp2)[:, :, :nb], host(kc)[:, :, :nb * 64].reshape(B, Hkv, nb, 64, d).mean(axis=3),
               1e-6, "kv_pool")


@pytest.mark.parametrize("B,N,Hq,Hkv,dtype,topk,n_local", [
    (1, 512, 2, 2, "f32", 4, 1),          # tiny workload shape (d = 64 below)
    (1, 64 * 40 + 17, 8, 2, "bf16", 8, 2),
    (2, 64 * 23, 4, 1, "bf16", 6, 1),
    (1, 64 * 70, 16, 1, "bf16", 64, 2),   # top-k wider than every row: dense causal
    (1, 64 * 20 + 33, 12, 2, "bf16", 8, 2),  # 6 heads per group: a head quad with 2 empty heads
])
def test_sparse_prefill(S, B, N, Hq, Hkv, dtype, topk, n_local):
    d = 64 if dtype == "f32" else 128
    print(f"sparse_prefill B={B} N={N} Hq={Hq} Hkv={Hkv} {dtype} topk={topk}", flush=True)
    q, k, v, g = sparse_case(11 + N, B, N, Hq, Hkv, d, dtype)
    ref = O.sparse_prefill(q, k, v, g, block=64, topk=topk, n_local=n_local)
    r = gpu_sparse_prefill(S, q, k, v, g, dtype, topk, n_local)
    sel = r["sel"].cpu().numpy()
    nm = check_selection(sel, ref["sel"], oracle_scores(ref), topk, n_local)
    print(f"  rows accepted by the margin rule: {nm}")
    # attention compared against the oracle run on the GPU's selection
    o_ref = O.sparse_attention(O.qk_norm(q), ref["k_hat"], v, sel, 64,
                               1.0 / np.sqrt(d)) * O.sigmoid(g)
    assert_rel(host(r["out"]), o_ref, TOL[dtype], "out")
    if nm == 0:
        assert_rel(host(r["out"]), ref["out"], TOL[dtype], "out vs oracle selection")


def test_block_select_planted_needles_and_ties(S):
    """Structured selection: key blocks aligned with the queries must be found; duplicated key
    blocks tie exactly and the lower index must win."""
    import torch

    rng = np.random.default_rng(5)
    B, N, Hq, Hkv, d = 1, 64 * 48, 4, 1, 128
    q = rng.standard_normal((B, N, Hq, d)).astype(np.float32) * 0.2
    k = rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * 0.2
    q[..., 0] += 3.0
    for j in (5, 17, 30):
        k[:, j * 64:(j + 1) * 64, :, 0] += 3.0
    k[:, 40 * 64:41 * 64] = k[:, 20 * 64:21 * 64]  # exact duplicate of block 20
    from hybrid_sparse_linear_causal_amd.inputs import bf16_round

    q, k = bf16_round(q), bf16_round(k)
    v = host_normal(6, 2, (B, N, Hkv, d), "bf16")
    g = host_normal(6, 3, (B, N, Hq, d), "bf16")
    ref = O.sparse_prefill(q, k, v, g, block=64, topk=6, n_local=2)
    r = gpu_sparse_prefill(S, q, k, v, g, "bf16", 6, 2)
    sel = r["sel"].cpu().numpy()
    check_selection(sel, ref["sel"], oracle_scores(ref), 6, 2)
    for i in range(32, 48):
        assert {5, 17, 30} <= set(sel[0, 0, i].tolist())
    torch.cuda.synchronize()


# ---------------------------------------------------------------- sparse layer decode


@pytest.mark.parametrize("B,Hq,Hkv,L,topk", [(2, 32, 2, 64 * 50 + 13, 16), (1, 16, 1, 64 * 50, 64),
                                             (2, 8, 2, 64 * 3 + 1, 8), (1, 4, 1, 40, 4),
                                             # more blocks than the 64 decode waves of a KV group
                                             (1, 16, 2, 64 * 300 + 3, 160),
                                             # 64 and 65 chosen beside the 3 forced blocks, over 4 slices:
                                             # the largest top-k of the lane-network selection, and the
                                             # smallest of the radix one
                                             (1, 8, 1, 64 * 2000 + 7, 67), (1, 8, 1, 64 * 2000 + 7, 68)])
def test_sparse_decode(S, B, Hq, Hkv, L, topk):
    """Decode at p = L - 1 over a synthetic cache of already-normalised keys (the same bits on
    both sides): append the new token, select, attend."""
    import torch

    d, n_local = 128, 2
    print(f"sparse_decode B={B} Hq={Hq} Hkv={Hkv} L={L} topk={topk}", flush=True)
    cap = ((L + 63) // 64) * 64
    kc_h = host_normal(21, 5, (B, Hkv, L - 1, d), "bf16")
    vc_h = host_normal(21, 6, (B, Hkv, L - 1, d), "bf16")
    q = host_normal(21, 0, (B, 1, Hq, d), "bf16")
    kn = host_normal(21, 1, (B, 1, Hkv, d), "bf16")
    vn = host_normal(21, 2, (B, 1, Hkv, d), "bf16")
    g = host_normal(21, 3, (B, 1, Hq, d), "bf16")
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
    ref = O.sparse_decode(q[:, 0], kn[:, 0], vn[:, 0], g[:, 0], kc_h, vc_h, L, block=64, topk=topk,
                          n_local=n_local)
    i = (L - 1) // 64
    qh = O.qk_norm(q[:, 0])
    G = Hq // Hkv

    def scores(b, gg, ii):
        qt = qh[b, gg * G:(gg + 1) * G].sum(axis=0)
        kb = kc_h[b, gg, : max(ii - 1, 1) * 64].astype(np.float64).reshape(-1, 64, d).mean(axis=1)
        return {j: float(kb[j] @ qt) for j in range(kb.shape[0])}

    gsel = sel.cpu().numpy()
    nm = check_selection(gsel, ref["sel"][:, :, None], scores, topk, n_local, first_block=i)
    if nm == 0:
        assert_rel(host(out)[:, 0], ref["out"], 1e-2, "decode out")
    # the oracle's attention on the GPU's selection, always
    o2 = np.empty_like(ref["out"])
    for b in range(B):
        for gg in range(Hkv):
            o2[b, gg * G:(gg + 1) * G] = oracle_decode_on_selection(
                qh[b, gg * G:(gg + 1) * G], kc_h[b, gg], vc_h[b, gg], O.qk_norm(kn[b, 0, gg]), vn[b, 0, gg],
                gsel[b, gg, 0], 1.0 / np.sqrt(d))
    assert_rel(host(out)[:, 0], o2 * O.sigmoid(g[:, 0]), 1e-2, "decode out (gpu selection)")


def test_decode_select_exact_ties_across_slices(S):
    """Decode selection over ~1,200 candidate blocks (several 512-block slices): two needle
    blocks score highest, 1,001 blocks hold identical keys (exactly equal scores in the oracle
    and on the GPU), the rest score clearly lower. The selection must be the needles plus the
    lowest-index tied blocks, exactly as the oracle's ordering (ties to the lower index)."""
    import torch

    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, topk, n_local = 1, 4, 1, 128, 16, 2
    L = 64 * 1200 + 5
    i = (L - 1) // 64
    kc_h = (rng.standard_normal((B, Hkv, L, d)) * 0.05).astype(np.float32)
    q = (rng.standard_normal((B, 1, Hq, d)) * 0.1).astype(np.float32)
    q[..., 0] += 2.0
    tied = (rng.standard_normal((64, d)) * 0.05).astype(np.float32)
    tied[:, 0] += 0.5
    for j in [7] + list(range(100, 1100)):
        kc_h[0, 0, j * 64:(j + 1) * 64] = tied
    for j in (450, 900):
        kc_h[0, 0, j * 64:(j + 1) * 64, 0] += 2.0
    from hybrid_sparse_linear_causal_amd.inputs import bf16_round

    kc_h, q = bf16_round(kc_h), bf16_round(q)
    cap = ((L + 63) // 64) * 64
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    kc[:, :, :L] = dev(kc_h, "bf16")
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_pool(kc, kp, L, 0, i)
    sel = S.block_select(dev(q, "bf16"), kp, L, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local)
    got = sel.cpu().numpy()[0, 0, 0]
    qt = O.qk_norm(q[0, 0]).sum(axis=0)
    kb = kc_h[0, 0, : i * 64].astype(np.float64).reshape(i, 64, d).mean(axis=1)
    sc = np.full(i - n_local + 1, -np.inf)
    sc[1:] = kb[1: i - n_local + 1] @ qt
    ref = O.select_row(sc, i, topk, n_local)
    assert list(got) == list(ref), (got, ref)
    assert {450, 900, 7, 100} <= set(got.tolist())


# ---------------------------------------------------------------- dense mode of the sparse layer


@pytest.mark.parametrize("B,N,Hq,Hkv,dtype", [
    (1, 512, 2, 2, "f32"),
    (1, 64 * 9 + 33, 8, 2, "bf16"),   # ragged last block
    (2, 64 * 20, 16, 1, "bf16"),
])
def test_dense_attn_prefill(S, B, N, Hq, Hkv, dtype):
    import torch

    d = 64 if dtype == "f32" else 128
    print(f"dense prefill B={B} N={N} Hq={Hq} Hkv={Hkv} {dtype}", flush=True)
    q, k, v, g = sparse_case(41 + N, B, N, Hq, Hkv, d, dtype)
    cap = ((N + 63) // 64) * 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros((B, Hkv, cap, d), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append(dev(k, dtype), dev(v, dtype), kc, vc, kp, N)
    out = S.dense_attn(dev(q, dtype), kc, vc, dev(g, dtype), N)
    ref = O.dense_attention(O.qk_norm(q), O.qk_norm(k), v, 1.0 / np.sqrt(d)) * O.sigmoid(g)
    assert_rel(host(out), ref, TOL[dtype], "dense out")


@pytest.mark.parametrize("L", [64 * 30 + 7, 64 * 150 + 7])
def test_dense_attn_decode(S, L):
    """One decode token over a cache of already-normalised keys, every block attended (151
    blocks: some decode waves take three blocks in turn, reusing their LDS tile)."""
    import torch

    B, Hq, Hkv, d = 2, 32, 2, 128
    print(f"dense_attn_decode L={L}", flush=True)
    cap = ((L + 63) // 64) * 64
    kc_h = host_normal(51, 5, (B, Hkv, L - 1, d), "bf16")
    vc_h = host_normal(51, 6, (B, Hkv, L - 1, d), "bf16")
    q = host_normal(51, 0, (B, 1, Hq, d), "bf16")
    kn = host_normal(51, 1, (B, 1, Hkv, d), "bf16")
    vn = host_normal(51, 2, (B, 1, Hkv, d), "bf16")
    g = host_normal(51, 3, (B, 1, Hq, d), "bf16")
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :, :L - 1] = dev(kc_h, "bf16")
    vc[:, :, :L - 1] = dev(vc_h, "bf16")
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append(dev(kn, "bf16"), dev(vn, "bf16"), kc, vc, kp, L, n_heads=Hq)
    out = S.dense_attn(dev(q, "bf16"), kc, vc, dev(g, "bf16"), L)
    K = np.concatenate([kc_h, O.qk_norm(kn).transpose(0, 2, 1, 3)], axis=2).transpose(0, 2, 1, 3)
    V = np.concatenate([vc_h, vn.transpose(0, 2, 1, 3)], axis=2).transpose(0, 2, 1, 3)
    ref = O.dense_attention(O.qk_norm(q), K, V, 1.0 / np.sqrt(d), q_positions=[L - 1]) * O.sigmoid(g)
    assert_rel(host(out), ref, 1e-2, "dense decode out")


@pytest.mark.parametrize("N,topk", [(64 * 8, 8), (64 * 7 + 5, 8)])
def test_dense_equals_sparse_when_selection_covers_all(S, N, topk):
    """Where the library's switch picks dense mode (kv_len <= topk * 64), block selection keeps
    every causal block and the two modes give bit-identical outputs."""
    import torch

    B, Hq, Hkv, d = 1, 8, 2, 128
    assert S.sparse_layer_uses_dense(batch=B, n_q=N, n_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                                     dtype=torch.bfloat16, kv_len=N, kv_capacity=((N + 63) // 64) * 64,
                                     topk=topk)
    q, k, v, g = sparse_case(61, B, N, Hq, Hkv, d, "bf16")
    r = gpu_sparse_prefill(S, q, k, v, g, "bf16", topk, 2)
    dense = S.dense_attn(dev(q, "bf16"), r["kc"], r["vc"], dev(g, "bf16"), N)
    torch.cuda.synchronize()
    assert torch.equal(dense, r["out"])


# ---------------------------------------------------------------- determinism


def test_deterministic_reruns(S):
    import torch

    q, k, v, g = lin_inputs(77, 1, 2000, 4, 128, "bf16")
    args = [dev(x, "bf16") for x in (q, k, v, g)]
    o1, s1 = S.linear_prefill(*args)
    o2, s2 = S.linear_prefill(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    q, k, v, g = sparse_case(78, 1, 64 * 30, 8, 2, 128, "bf16")
    r1 = gpu_sparse_prefill(S, q, k, v, g, "bf16", 8, 2)
    r2 = gpu_sparse_prefill(S, q, k, v, g, "bf16", 8, 2)
    torch.cuda.synchronize()
    assert torch.equal(r1["sel"], r2["sel"]) and torch.equal(r1["out"], r2["out"])


# ---------------------------------------------------------------- graph capture


def test_decode_step_graph_replay_matches_eager(S):
    """A decode step (3 linear layers + sparse layer: append, select, attention) captured once
    as a HIP graph and replayed three times, with eager work and synchronisation between the
    replays; every replay must reproduce the eager step exactly (same inputs, reset state)."""
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    B, H, Hkv, d, L, topk, n_local = 2, 32, 2, 128, 64 * 300 + 9, 32, 2
    bf = torch.bfloat16
    lin = []
    for li in range(3):
        t = [device_normal(200 + li, tid, (B, H, d)) for tid in range(4)]
        s0 = device_normal(200 + li, 4, (B, H, d, d), dtype="f32")
        lin.append(dict(qkvg=t, s0=s0, state=s0.clone(), out=torch.empty_like(t[0])))
    q, g = device_normal(210, 0, (B, 1, H, d)), device_normal(210, 3, (B, 1, H, d))
    kn, vn = device_normal(210, 1, (B, 1, Hkv, d)), device_normal(210, 2, (B, 1, Hkv, d))
    cap = ((L + 63) // 64) * 64
    kc = torch.zeros((B, Hkv, cap, d), dtype=bf, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :, :L - 1] = device_normal(211, 5, (B, Hkv, L - 1, d))
    vc[:, :, :L - 1] = device_normal(211, 6, (B, Hkv, L - 1, d))
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_pool(kc, kp, L - 1, 0, (L - 1) // 64)
    desc = S.sparse_desc(batch=B, n_q=1, n_heads=H, n_kv_heads=Hkv, head_dim=d, dtype=bf, kv_len=L,
                         kv_capacity=cap, topk=topk, n_local=n_local)
    sel = torch.empty((B, Hkv, 1, topk), dtype=torch.int32, device="cuda")
    ws_sel = torch.empty(S.workspace_bytes(S.OP_BLOCK_SELECT, desc), dtype=torch.uint8, device="cuda")
    ws_att = torch.empty(S.workspace_bytes(S.OP_SPARSE_ATTN, desc), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step():
        for Lr in lin:
            S.linear_decode_step(*Lr["qkvg"], Lr["state"], L - 1, out=Lr["out"])
        S.kv_append(kn, vn, kc, vc, kp, L, n_heads=H)
        S.block_select(q, kp, L, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local, sel=sel, workspace=ws_sel)
        S.sparse_attn(q, kc, vc, g, sel, L, n_local=n_local, out=out, workspace=ws_att)

    def reset():
        for Lr in lin:
            Lr["state"].copy_(Lr["s0"])

    def snapshot():
        return [x.clone() for x in [out, sel] + [Lr["out"] for Lr in lin] + [Lr["state"] for Lr in lin]]

    reset()
    step()
    torch.cuda.synchronize()
    ref = snapshot()
    graph = torch.cuda.CUDAGraph()
    reset()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        reset()
        out.zero_()
        sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep}"
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work between replays
