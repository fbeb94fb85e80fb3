"""Segmented long prefill (a prompt processed in consecutive calls, carrying the linear state
through state_in / pos0 and growing the KV and pooled caches through kv_len), against the
one-shot prefill and, at a 1,048,576-token context, against the oracle on sampled query
blocks; then a decode step on the prefilled caches."""

import math

import numpy as np
import pytest

import oracle as O
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


def _sparse_segmented(S, q, k, v, g, cap, bounds, topk, n_local):
    """Run the sparse layer over the segments [bounds[s], bounds[s+1]) of one prompt."""
    import torch

    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    kc = torch.zeros((B, Hkv, cap, d), dtype=q.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    outs, sels = [], []
    for s0, s1 in zip(bounds[:-1], bounds[1:]):
        S.kv_append(k[:, s0:s1].contiguous(), v[:, s0:s1].contiguous(), kc, vc, kp, s1, n_heads=Hq)
        qs = q[:, s0:s1].contiguous()
        sel = S.block_select(qs, kp, s1, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local)
        outs.append(S.sparse_attn(qs, kc, vc, g[:, s0:s1].contiguous(), sel, s1, n_local=n_local))
        sels.append(sel)
    return torch.cat(outs, 1), torch.cat(sels, 2), kc, vc, kp


def test_sparse_segmented_equals_one_shot(S):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    B, N, Hq, Hkv, d, topk, n_local = 1, 64 * 150, 8, 2, 128, 16, 2
    q, g = device_normal(71, 0, (B, N, Hq, d)), device_normal(71, 3, (B, N, Hq, d))
    k, v = device_normal(71, 1, (B, N, Hkv, d)), device_normal(71, 2, (B, N, Hkv, d))
    one, sel1, *_ = _sparse_segmented(S, q, k, v, g, N, [0, N], topk, n_local)
    seg, sel2, *_ = _sparse_segmented(S, q, k, v, g, N, [0, 64 * 40, 64 * 90, N], topk, n_local)
    torch.cuda.synchronize()
    assert torch.equal(sel1, sel2)
    assert torch.equal(one, seg)


def test_linear_segmented_equals_one_shot_and_oracle(S):
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    B, N, H, d = 1, 5000, 4, 128
    q, k, v, g = (device_normal(72, t, (B, N, H, d)) for t in range(4))
    out1, st1 = S.linear_prefill(q, k, v, g)
    st = None
    outs = []
    for s0, s1 in ((0, 1024), (1024, 3072), (3072, N)):
        o, st = S.linear_prefill(*(x[:, s0:s1].contiguous() for x in (q, k, v, g)), pos0=s0, state_in=st)
        outs.append(o)
    torch.cuda.synchronize()
    seg = torch.cat(outs, 1)
    ref, S_ref = O.linear_prefill(*(x.float().cpu().numpy() for x in (q, k, v, g)))
    assert_rel(host(seg), ref, 1e-2, "segmented out")
    assert_rel(host(out1), ref, 1e-2, "one-shot out")
    assert_rel(host(st), S_ref, 1e-2, "segmented state")
    assert_rel(host(seg), host(out1), 1e-2, "segmented vs one-shot")


def test_sparse_segmented_1m_context_sampled(S):
    """One sparse layer prefilled over 1,048,576 tokens in 8 segments of 131,072 (rows of up
    to 16,381 candidate blocks), sampled query blocks against the oracle, then one decode step
    at position 1,048,576 on the prefilled caches."""
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    B, Hq, Hkv, d, topk, n_local = 1, 32, 2, 128, 64, 2
    G = Hq // Hkv
    N, SEG = 1 << 20, 1 << 17
    cap = N + 64
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    k_all = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v_all = torch.empty_like(k_all)
    last = {}
    for s in range(N // SEG):
        s0, s1 = s * SEG, (s + 1) * SEG
        print(f"segment {s}: tokens {s0}..{s1}", flush=True)
        q, g = device_normal(80 + s, 0, (B, SEG, Hq, d)), device_normal(80 + s, 3, (B, SEG, Hq, d))
        k, v = device_normal(80 + s, 1, (B, SEG, Hkv, d)), device_normal(80 + s, 2, (B, SEG, Hkv, d))
        k_all[:, s0:s1], v_all[:, s0:s1] = k, v
        S.kv_append(k, v, kc, vc, kp, s1, n_heads=Hq)
        sel = S.block_select(q, kp, s1, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local)
        out = S.sparse_attn(q, kc, vc, g, sel, s1, n_local=n_local)
        if s == N // SEG - 1:
            last = dict(q=q, g=g, sel=sel, out=out, s0=s0)
    torch.cuda.synchronize()
    gsel = last["sel"].cpu().numpy()
    nqb_seg = SEG // 64
    qb0 = last["s0"] // 64
    for gk in range(Hkv):
        kh = O.qk_norm(k_all[:, :, gk:gk + 1].float().cpu().numpy())
        vg = v_all[:, :, gk:gk + 1].float().cpu().numpy()
        kb = O.pool_keys(kh, 64)
        for r in (0, 1, 777, nqb_seg - 1):
            i = qb0 + r
            qh = O.qk_norm(last["q"][:, r * 64:(r + 1) * 64, gk * G:(gk + 1) * G].float().cpu().numpy())
            qt = O.query_block_tilde(qh, 64, 1)[0, 0, 0]
            ncand = i - n_local + 1
            sc = np.full(ncand, -np.inf)
            sc[1:] = O.block_scores(qt, kb[0, 0, 1:ncand])
            ref_row = O.select_row(sc, i, topk, n_local)
            check_selection(gsel[:, gk:gk + 1, r:r + 1], ref_row[None, None, None],
                            lambda b, gg, ii: {j: float(sc[j]) for j in range(1, ncand)}, topk, n_local,
                            first_block=i)
            sel_arr = np.full((1, 1, i + 1, topk), -1, dtype=np.int64)
            sel_arr[0, 0, i] = gsel[0, gk, r]
            o = O.sparse_attention(qh, kh[:, :(i + 1) * 64], vg[:, :(i + 1) * 64], sel_arr, 64,
                                   1.0 / math.sqrt(d), q_positions=np.arange(i * 64, (i + 1) * 64))
            o = o * O.sigmoid(last["g"][:, r * 64:(r + 1) * 64, gk * G:(gk + 1) * G].float().cpu().numpy())
            assert_rel(host(last["out"][:, r * 64:(r + 1) * 64, gk * G:(gk + 1) * G]), o, 1e-2,
                       f"group {gk} block {i}")
    # decode one token at position N on the prefilled caches
    qd, gd = device_normal(99, 0, (B, 1, Hq, d)), device_normal(99, 3, (B, 1, Hq, d))
    kd, vd = device_normal(99, 1, (B, 1, Hkv, d)), device_normal(99, 2, (B, 1, Hkv, d))
    S.kv_append(kd, vd, kc, vc, kp, N + 1, n_heads=Hq)
    sel = S.block_select(qd, kp, N + 1, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local)
    out = S.sparse_attn(qd, kc, vc, gd, sel, N + 1, n_local=n_local)
    torch.cuda.synchronize()
    gk = 1
    k_h = k_all[:, :, gk:gk + 1].float().cpu().numpy()
    kch = O.qk_norm(k_h).transpose(0, 2, 1, 3)
    vch = v_all[:, :, gk:gk + 1].float().cpu().numpy().transpose(0, 2, 1, 3)
    ref = O.sparse_decode(qd[:, 0, gk * G:(gk + 1) * G].float().cpu().numpy(),
                          kd[:, 0, gk:gk + 1].float().cpu().numpy(), vd[:, 0, gk:gk + 1].float().cpu().numpy(),
                          gd[:, 0, gk * G:(gk + 1) * G].float().cpu().numpy(), kch, vch, N + 1, block=64,
                          topk=topk, n_local=n_local, k_bar=O.pool_keys(O.qk_norm(k_h), 64)[:, :, : N // 64 - 1])
    i = N // 64
    qt = O.qk_norm(qd[:, 0, gk * G:(gk + 1) * G].float().cpu().numpy())[0].sum(axis=0)
    kbd = O.pool_keys(O.qk_norm(k_h), 64)[0, 0, : i - 1]
    scd = kbd @ qt
    nm = check_selection(sel.cpu().numpy()[:, gk:gk + 1], ref["sel"][:, :, None],
                         lambda bb, gg, ii: {j: float(scd[j]) for j in range(len(scd))}, topk, n_local,
                         first_block=i)
    if nm == 0:
        assert_rel(host(out[:, 0, gk * G:(gk + 1) * G]), ref["out"], 1e-2, "decode at 1M")
    # rows accepted by the margin rule included: the oracle's attention on the GPU's selection
    o2 = oracle_decode_on_selection(O.qk_norm(qd[:, 0, gk * G:(gk + 1) * G].float().cpu().numpy())[0], kch[0, 0],
                                    vch[0, 0], O.qk_norm(kd[0, 0, gk].float().cpu().numpy()),
                                    vd[0, 0, gk].float().cpu().numpy(), sel.cpu().numpy()[0, gk, 0], 1.0 / math.sqrt(d))
    assert_rel(host(out[:, 0, gk * G:(gk + 1) * G]),
               (o2 * O.sigmoid(gd[0, 0, gk * G:(gk + 1) * G].float().cpu().numpy()))[None], 1e-2,
               "decode at 1M on the gpu selection")
