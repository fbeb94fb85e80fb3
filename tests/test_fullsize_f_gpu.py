"""GPU parity of the backward kernels and the packed-batch prefill at the sizes bench.py times
them, on sampled outputs the oracles compute one by one (inputs: the bench's seeded device
draws, slices copied to the host):

* linear backward, 32,768 and 262,144 tokens x 32 heads, a sampled head. The gradients of a
  window of tokens are those of the layer restricted to the window, given the state entering it
  (numpy oracle forward over the tokens before it) and the state gradient leaving it: the last
  256 tokens (every gradient; nothing follows them) and the first 256 tokens (dq and dg, which
  depend on the tokens up to their own) against the gradient oracle on the window;
* sparse backward, 131,072 tokens: dq and dg of sampled query blocks (their own attention), and
  dk, dv of sampled key blocks (summed over every query block that selected them, 16 heads);
* packed batch of 16 prompts (262,144 tokens): a sampled head of the linear layer for three
  sequences, and sampled query blocks of the sparse layer for two sequences.
"""

import math

import numpy as np
import pytest

import oracle as O
from oracle import sala_oracle_grad as OG
from sala_testutil import assert_rel, check_selection, host

pytestmark = pytest.mark.gpu

TOL = 1e-2  # the bf16 bar, for the forward and the backward alike


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("key,h", [("linear_32k", 7), ("stack_256k", 19)])
def test_linear_backward_full_size_windows(S, key, h):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal

    W = WORKLOADS[key]
    N, H, d, w = W.seq_len, 32, 128, 256
    print(f"linear backward full size N={N} head {h}", flush=True)
    t = [device_normal(W.seed, tid, (1, N, H, d)) for tid in (0, 1, 2, 3, 10)]
    gr = S.linear_backward(*t)
    torch.cuda.synchronize()
    q, k, v, g, dout = (_np(x[:, :, h:h + 1]) for x in t)
    # last window: state entering it from the oracle's forward over the tokens before it
    _, s_in = O.linear_prefill(q[:, :N - w], k[:, :N - w], v[:, :N - w], g[:, :N - w])
    ref = OG.linear_layer_grads(q[:, N - w:], k[:, N - w:], v[:, N - w:], g[:, N - w:], dout[:, N - w:],
                                pos0=N - w, state_in=s_in)
    for n in ("dq", "dk", "dv", "dg"):
        e = assert_rel(_np(gr[n][:, N - w:, h:h + 1]), ref[n], TOL, f"last window {n}")
        print(f"  last {w} tokens {n}: {e:.2e}", flush=True)
    # first window: dq and dg depend only on the tokens up to their own
    ref0 = OG.linear_layer_grads(q[:, :w], k[:, :w], v[:, :w], g[:, :w], dout[:, :w])
    for n in ("dq", "dg"):
        e = assert_rel(_np(gr[n][:, :w, h:h + 1]), ref0[n], TOL, f"first window {n}")
        print(f"  first {w} tokens {n}: {e:.2e}", flush=True)


def test_sparse_backward_full_size_sampled_blocks(S):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal

    W = WORKLOADS["sparse_128k"]
    N, Hq, Hkv, d, topk = W.seq_len, 32, 2, 128, W.topk
    G = Hq // Hkv
    print(f"sparse backward full size N={N}", flush=True)
    q, g = device_normal(W.seed, 0, (1, N, Hq, d)), device_normal(W.seed, 3, (1, N, Hq, d))
    k, v = device_normal(W.seed, 1, (1, N, Hkv, d)), device_normal(W.seed, 2, (1, N, Hkv, d))
    dout = device_normal(W.seed, 10, (1, N, Hq, d))
    kc = torch.zeros((1, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((1, Hkv, N // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append(k, v, kc, vc, kp, N, n_heads=Hq)
    sel = S.block_select(q, kp, N, N, n_kv_heads=Hkv, topk=topk, n_local=W.n_local)
    gr = S.sparse_attn_backward(q, kc, vc, g, sel, N, dout, topk=topk, n_local=W.n_local)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy().astype(np.int64)  # [1, Hkv, nqb, topk]
    gk = 1
    heads = slice(gk * G, (gk + 1) * G)
    k_hat = _np(kc[:, gk:gk + 1]).transpose(0, 2, 1, 3)  # [1, N, 1, d]: the cache contents
    v_h = _np(vc[:, gk:gk + 1]).transpose(0, 2, 1, 3)
    sel_g = gsel[:, gk:gk + 1]

    def rows(blocks):
        return np.concatenate([np.arange(i * 64, (i + 1) * 64) for i in blocks])

    # dq, dg of sampled query blocks
    for i in (0, 1, 65, 1000, N // 64 - 1):
        r = rows([i])
        ref = OG.sparse_attention_grads(_np(q[:, r, heads]), k_hat[:, :(i + 1) * 64], v_h[:, :(i + 1) * 64],
                                        _np(g[:, r, heads]), sel_g, _np(dout[:, r, heads]), q_positions=r)
        e1 = assert_rel(_np(gr["dq"][:, r, heads]), ref["dq"], TOL, f"dq block {i}")
        e2 = assert_rel(_np(gr["dg"][:, r, heads]), ref["dg"], TOL, f"dg block {i}")
        print(f"  query block {i}: dq {e1:.2e} dg {e2:.2e}", flush=True)
    # dk, dv of sampled key blocks: every query block that chose them
    for j in (1200, 1900, N // 64 - 2):  # blocks chosen by up to a few tens of query blocks
        qbs = [i for i in range(N // 64) if j in set(gsel[0, gk, i].tolist())]
        r = rows(qbs)
        L = (max(qbs) + 1) * 64
        ref = OG.sparse_attention_grads(_np(q[:, r, heads]), k_hat[:, :L], v_h[:, :L], _np(g[:, r, heads]), sel_g,
                                        _np(dout[:, r, heads]), q_positions=r)
        kr = slice(j * 64, (j + 1) * 64)
        e1 = assert_rel(_np(gr["dk_cache"][0, gk, kr]), ref["dk_hat"][0, kr, 0], TOL, f"dk block {j}")
        e2 = assert_rel(_np(gr["dv_cache"][0, gk, kr]), ref["dv"][0, kr, 0], TOL, f"dv block {j}")
        print(f"  key block {j} ({len(qbs)} query blocks): dk {e1:.2e} dv {e2:.2e}", flush=True)


def test_varlen_full_size_sampled(S):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal, varlen_lengths

    W = WORKLOADS["varlen_256k"]
    lens = varlen_lengths(W.seed, W.batch, W.seq_len)
    T, H, Hkv, d = sum(lens), 32, 2, 128
    G = H // Hkv
    vl = S.Varlen(lens)
    cu = vl.cu
    print(f"varlen full size T={T} lengths {lens}", flush=True)
    q, k, v, g = (device_normal(W.seed, t, (T, H, d)) for t in range(4))
    out, st = S.linear_prefill_varlen(q, k, v, g, vl)
    torch.cuda.synchronize()
    for s, h in ((5, 3), (7, 30), (2, 11)):  # the shortest prompts, sampled heads
        a, b = cu[s], cu[s + 1]
        ref, S_ref = O.linear_prefill(*(_np(x[None, a:b, h:h + 1]) for x in (q, k, v, g)))
        assert_rel(host(out[None, a:b, h:h + 1]), ref, 1e-2, f"linear seq {s} head {h}")
        assert_rel(host(st[s:s + 1, h:h + 1]), S_ref, 1e-2, f"linear state seq {s} head {h}")
    sk, sv = device_normal(W.seed, 11, (T, Hkv, d)), device_normal(W.seed, 12, (T, Hkv, d))
    cap = ((max(lens) + 63) // 64) * 64
    kc = torch.zeros((len(lens), Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((len(lens), Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append_varlen(sk, sv, kc, vc, kp, vl, n_heads=H)
    sel = S.block_select_varlen(q, kp, vl, cap, n_kv_heads=Hkv, topk=W.topk, n_local=W.n_local)
    o = S.sparse_attn_varlen(q, kc, vc, g, sel, vl, n_local=W.n_local)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy()
    row0 = np.concatenate([[0], np.cumsum([(n + 63) // 64 for n in lens])])
    for s in (5, 10):  # the shortest and the longest prompt
        a, n = cu[s], lens[s]
        nqb = (n + 63) // 64
        sel_s = gsel[row0[s] * Hkv:(row0[s] + nqb) * Hkv].reshape(1, Hkv, nqb, W.topk)
        for gk in range(Hkv):
            kh = O.qk_norm(_np(sk[None, a:a + n, gk:gk + 1]))
            kb = O.pool_keys(kh, 64)
            for i in sorted({0, 1, 2, 40, nqb - 1}):
                if i >= nqb:
                    continue
                r = np.arange(i * 64, min(n, (i + 1) * 64))
                qh = O.qk_norm(_np(q[None, a + r, gk * G:(gk + 1) * G]))
                qt = O.query_block_tilde(qh, 64, 1)[0, 0, 0]
                ncand = max(0, i - W.n_local + 1)
                sc = np.full(max(ncand, 1), -np.inf)
                if ncand:
                    sc[:ncand] = O.block_scores(qt, kb[0, 0, :ncand])
                ref_row = O.select_row(sc, i, W.topk, W.n_local)
                check_selection(sel_s[:, gk:gk + 1, i:i + 1], ref_row[None, None, None],
                                lambda b_, gg, ii: {j: float(sc[j]) for j in range(ncand)}, W.topk, W.n_local,
                                first_block=i)
                sel_arr = np.full((1, 1, i + 1, W.topk), -1, dtype=np.int64)
                sel_arr[0, 0, i] = sel_s[0, gk, i]
                vv = _np(sv[None, a:a + (i + 1) * 64, gk:gk + 1])[:, : min(n, (i + 1) * 64)]
                ref = O.sparse_attention(qh, kh[:, : min(n, (i + 1) * 64)], vv, sel_arr, 64, 1.0 / math.sqrt(d),
                                         q_positions=r) * O.sigmoid(_np(g[None, a + r, gk * G:(gk + 1) * G]))
                assert_rel(host(o[None, a + r, gk * G:(gk + 1) * G]), ref, 1e-2, f"sparse seq {s} group {gk} "
                                                                                  f"block {i}")
        print(f"  sparse seq {s} (n={n}) sampled blocks ok", flush=True)
