"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times, on
sampled outputs the oracle computes one by one:

* linear prefill, 32,768 and 262,144 tokens x 32 heads: whole sampled heads (every token)
  against the oracle's token recurrence on that head;
* sparse prefill, 131,072 and 262,144 tokens (32 query heads over 2 KV heads, top-64 with
  block 0 and 2 local blocks forced): sampled query blocks of both KV groups — selection
  (bit-exact up to the margin rule) and every query row of the block's 16 heads;
* decode at a 1,048,576-token context, batch 8: sampled sequences and KV groups for the
  sparse layer, sampled (sequence, head) states for the linear layer.

Inputs are the seeded device draws the bench uses; slices are copied to the host so the
oracle sees the same bits."""

import math

import numpy as np
import pytest

import oracle as O
from sala_testutil import assert_rel, check_selection, host, oracle_decode_on_selection

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


def _np(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("N,heads", [(32768, (0, 31)), (262144, (17,))])
def test_linear_prefill_full_size(S, N, heads):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal

    W = WORKLOADS["stack_256k"]
    H, d = 32, 128
    seed = 102 if N == 32768 else W.seed
    print(f"linear full size N={N} heads={heads}", flush=True)
    q, k, v, g = (device_normal(seed, t, (1, N, H, d)) for t in range(4))
    out, st = S.linear_prefill(q, k, v, g)
    torch.cuda.synchronize()
    for h in heads:
        sl = [_np(x[:, :, h:h + 1]) for x in (q, k, v, g)]
        ref, S_ref = O.linear_prefill(*sl)
        assert_rel(host(out[:, :, h:h + 1]), ref, 1e-2, f"out head {h}")
        assert_rel(host(st[:, h:h + 1]), S_ref, 1e-2, f"state head {h}")


@pytest.mark.parametrize("N", [131072, 262144])
def test_sparse_prefill_full_size(S, N):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    Hq, Hkv, d, topk, n_local = 32, 2, 128, 64, 2
    G = Hq // Hkv
    seed = 103 if N == 131072 else 104 + 3
    print(f"sparse full size N={N}", flush=True)
    q, g = device_normal(seed, 0, (1, N, Hq, d)), device_normal(seed, 3, (1, N, Hq, d))
    k, v = device_normal(seed, 1, (1, N, Hkv, d)), device_normal(seed, 2, (1, N, Hkv, d))
    kc = torch.zeros((1, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((1, Hkv, N // 64, d), dtype=torch.float32, device="cuda")
    S.kv_append(k, v, kc, vc, kp, N, n_heads=Hq)
    sel = S.block_select(q, kp, N, N, n_kv_heads=Hkv, topk=topk, n_local=n_local)
    out = S.sparse_attn(q, kc, vc, g, sel, N, n_local=n_local)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy()
    nqb = N // 64
    for gk in range(Hkv):
        imax = max(i for i in (0, 1, 2, 63, 64, 65, 1000, nqb - 1) if i < nqb)
        kh = O.qk_norm(_np(k[:, : (imax + 1) * 64, gk:gk + 1]))
        vg = _np(v[:, : (imax + 1) * 64, gk:gk + 1])
        kb = O.pool_keys(kh, 64)
        for i in (0, 1, 2, 63, 64, 65, 1000, nqb - 1):
            qh = O.qk_norm(_np(q[:, i * 64:(i + 1) * 64, gk * G:(gk + 1) * G]))
            qt = O.query_block_tilde(qh, 64, 1)[0, 0, 0]
            ncand = max(0, i - n_local + 1)
            sc = np.full(max(ncand, 1), -np.inf)
            if ncand:
                sc[:ncand] = O.block_scores(qt, kb[0, 0, :ncand])
            ref_row = O.select_row(sc, i, topk, n_local)
            check_selection(gsel[:, gk:gk + 1, i:i + 1], ref_row[None, None, None],
                            lambda b, gg, ii: {j: float(sc[j]) for j in range(ncand)}, topk, n_local,
                            first_block=i)
            sel_arr = np.full((1, 1, i + 1, topk), -1, dtype=np.int64)
            sel_arr[0, 0, i] = gsel[0, gk, i]
            o = O.sparse_attention(qh, kh[:, : (i + 1) * 64], vg[:, : (i + 1) * 64], sel_arr, 64,
                                   1.0 / math.sqrt(d), q_positions=np.arange(i * 64, (i + 1) * 64))
            o = o * O.sigmoid(_np(g[:, i * 64:(i + 1) * 64, gk * G:(gk + 1) * G]))
            assert_rel(host(out[:, i * 64:(i + 1) * 64, gk * G:(gk + 1) * G]), o, 1e-2,
                       f"group {gk} block {i}")


def test_decode_full_size(S):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal

    Dw = WORKLOADS["decode_1m"]
    B, L, H, Hkv, d = Dw.batch, Dw.seq_len, 32, 2, 128
    G = H // Hkv
    print("decode full size", flush=True)
    # linear layer: one step on the std-1024 synthetic state
    sd = Dw.seed
    lq, lk, lv, lg = (device_normal(sd, t, (B, H, d)) for t in range(4))
    state = device_normal(sd, 4, (B, H, d, d), dtype="f32", std=1024.0)
    s0 = {(b, h): _np(state[b:b + 1, h:h + 1]) for b, h in ((0, 0), (7, 31), (3, 12))}
    lo = S.linear_decode_step(lq, lk, lv, lg, state, L - 1)
    torch.cuda.synchronize()
    for (b, h), s_bh in s0.items():
        sl = [_np(x[b:b + 1, h:h + 1]) for x in (lq, lk, lv, lg)]
        ref, S_ref = O.linear_decode(*sl, s_bh, L - 1)
        assert_rel(host(lo[b:b + 1, h:h + 1]), ref, 1e-2, f"linear decode {(b, h)}")
        assert_rel(host(state[b:b + 1, h:h + 1]), S_ref, 1e-5, f"linear state {(b, h)}")
    # sparse layer over a 1M-token cache of N(0,1) keys taken as already normalised
    sd = Dw.seed + 3
    q, g = device_normal(sd, 0, (B, 1, H, d)), device_normal(sd, 3, (B, 1, H, d))
    kn, vn = device_normal(sd, 1, (B, 1, Hkv, d)), device_normal(sd, 2, (B, 1, Hkv, d))
    kc = torch.empty((B, Hkv, L, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    for b in range(B):
        kc[b] = device_normal(sd * 100 + b, 5, (Hkv, L, d))
        vc[b] = device_normal(sd * 100 + b, 6, (Hkv, L, d))
    kp = torch.zeros((B, Hkv, L // 64, d), dtype=torch.float32, device="cuda")
    S.kv_pool(kc, kp, L - 1, 0, (L - 1) // 64)
    samples = {(b, gk): (_np(kc[b:b + 1, gk:gk + 1, :L - 1]), _np(vc[b:b + 1, gk:gk + 1, :L - 1]))
               for b, gk in ((0, 0), (5, 1))}
    S.kv_append(kn, vn, kc, vc, kp, L, n_heads=H)
    sel = S.block_select(q, kp, L, L, n_kv_heads=Hkv, topk=Dw.topk, n_local=Dw.n_local)
    out = S.sparse_attn(q, kc, vc, g, sel, L, n_local=Dw.n_local)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy()
    i = (L - 1) // 64
    for (b, gk), (kch, vch) in samples.items():
        qs = _np(q[b:b + 1, 0, gk * G:(gk + 1) * G])
        gs = _np(g[b:b + 1, 0, gk * G:(gk + 1) * G])
        kns, vns = _np(kn[b:b + 1, 0, gk:gk + 1]), _np(vn[b:b + 1, 0, gk:gk + 1])
        ref = O.sparse_decode(qs, kns, vns, gs, kch, vch, L, block=64, topk=Dw.topk, n_local=Dw.n_local)
        qt = O.qk_norm(qs)[0].sum(axis=0)
        kb = kch[0, 0, : (i - 1) * 64].astype(np.float64).reshape(i - 1, 64, d).mean(axis=1)
        sc = kb @ qt
        nm = check_selection(gsel[b:b + 1, gk:gk + 1], ref["sel"][:, :, None],
                             lambda bb, gg, ii: {j: float(sc[j]) for j in range(len(sc))}, Dw.topk,
                             Dw.n_local, first_block=i)
        if nm == 0:
            assert_rel(host(out[b:b + 1, 0, gk * G:(gk + 1) * G]), ref["out"], 1e-2, f"decode {(b, gk)}")
        # rows accepted by the margin rule included: the oracle's attention on the GPU's selection
        o2 = oracle_decode_on_selection(O.qk_norm(qs)[0], kch[0, 0], vch[0, 0], O.qk_norm(kns[0, 0]),
                                        vns[0, 0], gsel[b, gk, 0], 1.0 / math.sqrt(d))
        assert_rel(host(out[b:b + 1, 0, gk * G:(gk + 1) * G]), (o2 * O.sigmoid(gs[0]))[None], 1e-2,
                   f"decode {(b, gk)} on the gpu selection")
    # the decode step's single call (append in the selection's first kernel, selection levels,
    # attention, combine) over the same cache: appending the same token at the same position
    # again leaves the cache and pooled keys as they are, so the row and output must be the
    # three calls' bit for bit
    kvl = torch.full((B,), L, dtype=torch.int64, device="cuda")
    out_s, sel_s = S.sparse_decode_step(q[:, 0], kn[:, 0], vn[:, 0], g[:, 0], kc, vc, kp, kvl, L, topk=Dw.topk,
                                        n_local=Dw.n_local)
    torch.cuda.synchronize()
    assert torch.equal(sel_s, sel[:, :, 0]), "decode step selection"
    assert torch.equal(out_s, out[:, 0]), "decode step output"
