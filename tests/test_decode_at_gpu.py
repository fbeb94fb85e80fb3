"""GPU parity of the decode entry points that take each sequence's own position
(sala_linear_decode_step_at, sala_sparse_decode_step) against the oracle's single-sequence
decode run per sequence, on seeded bf16-representable inputs; and bit-equality with the
one-position decode calls when every sequence sits at the same position."""

import numpy as np
import pytest

import oracle as O
from hybrid_sparse_linear_causal_amd.inputs import host_normal
from sala_testutil import assert_rel, check_selection, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


def test_linear_decode_step_at(S):
    import torch

    B, H, d = 4, 2, 128
    pos = [0, 5, 1000, 70000]
    print(f"linear_decode_step_at B={B} pos={pos}", flush=True)
    q, k, v, g = (host_normal(31, t, (B, H, d), "bf16") for t in range(4))
    s0 = host_normal(31, 4, (B, H, d, d), "f32", std=4.0)
    st = dev(s0, "f32")
    out = S.linear_decode_step_at(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "bf16"), st,
                                  torch.tensor(pos, dtype=torch.int64, device="cuda"))
    for b in range(B):
        ref, S_ref = O.linear_decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], s0[b:b + 1], pos[b])
        assert_rel(host(out)[b:b + 1], ref, 1e-2, f"out {b}")
        assert_rel(host(st)[b:b + 1], S_ref, 1e-5, f"state {b}")
    # all at one position: bit-identical to the one-position call
    st2, st3 = dev(s0, "f32"), dev(s0, "f32")
    a = S.linear_decode_step_at(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "bf16"), st2,
                                torch.full((B,), 777, dtype=torch.int64, device="cuda"))
    b_ = S.linear_decode_step(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "bf16"), st3, 777)
    torch.cuda.synchronize()
    assert torch.equal(a, b_) and torch.equal(st2, st3)


@pytest.mark.parametrize("lens,Hq,Hkv,topk", [
    ([130, 1000, 3000, 64], 4, 2, 8),          # contexts within one slice and across slices, a block edge
    ([40, 64 * 40 + 1], 16, 1, 16),            # a context too short for candidates beside a long one
])
def test_sparse_decode_step_per_sequence(S, lens, Hq, Hkv, topk):
    """Sequence b decodes its token at position lens[b] - 1 over a synthetic cache of normalised
    keys: append, select and attend in one call; each against the oracle's decode."""
    import torch

    d, n_local, B = 128, 2, len(lens)
    L = max(lens)
    cap = ((L + 63) // 64) * 64
    print(f"sparse_decode_step lens={lens} Hq={Hq} Hkv={Hkv} topk={topk}", flush=True)
    kc_h = host_normal(41, 5, (B, Hkv, L, d), "bf16")
    vc_h = host_normal(41, 6, (B, Hkv, L, d), "bf16")
    q = host_normal(41, 0, (B, Hq, d), "bf16")
    kn = host_normal(41, 1, (B, Hkv, d), "bf16")
    vn = host_normal(41, 2, (B, Hkv, d), "bf16")
    g = host_normal(41, 3, (B, Hq, d), "bf16")
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    for b, n in enumerate(lens):  # each cache holds its first n - 1 tokens, pooled
        kc[b, :, :n - 1] = dev(kc_h[b, :, :n - 1], "bf16")
        vc[b, :, :n - 1] = dev(vc_h[b, :, :n - 1], "bf16")
        if (n - 1) // 64:
            S.kv_pool(kc[b:b + 1], kp[b:b + 1], n - 1, 0, (n - 1) // 64)
    kvl = torch.tensor(lens, dtype=torch.int64, device="cuda")
    out, sel = S.sparse_decode_step(dev(q, "bf16"), dev(kn, "bf16"), dev(vn, "bf16"), dev(g, "bf16"), kc, vc, kp,
                                    kvl, L, topk=topk, n_local=n_local)
    gsel, go = sel.cpu().numpy(), host(out)
    qh = O.qk_norm(q)
    G = Hq // Hkv
    for b, n in enumerate(lens):
        ref = O.sparse_decode(q[b:b + 1], kn[b:b + 1], vn[b:b + 1], g[b:b + 1], kc_h[b:b + 1, :, :n - 1],
                              vc_h[b:b + 1, :, :n - 1], n, block=64, topk=topk, n_local=n_local)
        i = (n - 1) // 64

        def scores(_, gg, ii, b=b):
            qt = qh[b, gg * G:(gg + 1) * G].sum(axis=0)
            kb = kc_h[b, gg, : max(ii - 1, 1) * 64].astype(np.float64).reshape(-1, 64, d).mean(axis=1)
            return {j: float(kb[j] @ qt) for j in range(kb.shape[0])}

        nm = check_selection(gsel[b:b + 1, :, None], ref["sel"][:, :, None], scores, topk, n_local, first_block=i)
        assert nm == 0, "margin rows: rerun with other seeds"
        e = assert_rel(go[b:b + 1], ref["out"], 1e-2, f"out {b}")
        # the appended token's normalised key is in the cache at position n - 1
        assert_rel(host(kc)[b, :, n - 1], O.qk_norm(kn[b]), 2 ** -8, f"appended key {b}")
        print(f"  seq {b}: L={n} rel err {e:.2e}", flush=True)


def test_sparse_decode_step_equals_one_position_path(S):
    """Every sequence at the same length: bit-identical to kv_append + block_select + sparse_attn."""
    import torch

    B, Hq, Hkv, d, L, topk = 2, 8, 2, 128, 64 * 37 + 5, 16
    cap = ((L + 63) // 64) * 64
    kc_h = host_normal(51, 5, (B, Hkv, L - 1, d), "bf16")
    vc_h = host_normal(51, 6, (B, Hkv, L - 1, d), "bf16")
    q, g = (dev(host_normal(51, t, (B, Hq, d), "bf16"), "bf16") for t in (0, 3))
    kn, vn = (dev(host_normal(51, t, (B, Hkv, d), "bf16"), "bf16") for t in (1, 2))
    caches = []
    for _ in range(2):
        kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        kc[:, :, :L - 1] = dev(kc_h, "bf16")
        vc[:, :, :L - 1] = dev(vc_h, "bf16")
        kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
        S.kv_pool(kc, kp, L - 1, 0, (L - 1) // 64)
        caches.append((kc, vc, kp))
    kc, vc, kp = caches[0]
    out_a, sel_a = S.sparse_decode_step(q, kn, vn, g, kc, vc, kp, torch.full((B,), L, dtype=torch.int64,
                                                                              device="cuda"), L, topk=topk)
    kc2, vc2, kp2 = caches[1]
    S.kv_append(kn.unsqueeze(1), vn.unsqueeze(1), kc2, vc2, kp2, L, n_heads=Hq)
    sel_b = S.block_select(q.unsqueeze(1), kp2, L, cap, n_kv_heads=Hkv, topk=topk)
    out_b = S.sparse_attn(q.unsqueeze(1), kc2, vc2, g.unsqueeze(1), sel_b, L)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b[:, :, 0]) and torch.equal(out_a, out_b[:, 0])
    assert torch.equal(kc, kc2) and torch.equal(kp, kp2)


def test_decode_at_graph_replays_with_advancing_positions(S):
    """One decode step (a linear layer at per-sequence positions, then the sparse layer at
    per-sequence cache lengths) captured once as a HIP graph. The positions live in device
    tensors, so the same graph serves later steps: each replay, after the positions and the new
    tokens are updated in place, must equal the eager step on a copy of the caches and states."""
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    B, H, Hkv, d, topk = 2, 8, 2, 128, 8
    lens = [500, 1300]
    cap = 1408
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    for b, n in enumerate(lens):
        kc[b, :, :n - 1] = device_normal(61, 5 + b, (Hkv, n - 1, d))
        vc[b, :, :n - 1] = device_normal(61, 7 + b, (Hkv, n - 1, d))
        S.kv_pool(kc[b:b + 1], kp[b:b + 1], n - 1, 0, (n - 1) // 64)
    state = device_normal(62, 4, (B, H, d, d), dtype="f32")
    lin_in = [torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    q, g = (torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    kn, vn = (torch.empty((B, Hkv, d), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    kvl = torch.tensor(lens, dtype=torch.int64, device="cuda")
    pos = kvl - 1
    lout, sout = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda"), torch.empty_like(q)
    sel = torch.empty((B, Hkv, topk), dtype=torch.int32, device="cuda")
    desc = S.sparse_desc(batch=B, n_q=1, n_heads=H, n_kv_heads=Hkv, head_dim=d, dtype=torch.bfloat16,
                         kv_len=cap, kv_capacity=cap, topk=topk, n_local=2)
    ws = torch.empty(S.workspace_bytes(S.OP_SPARSE_DECODE_STEP, desc), dtype=torch.uint8, device="cuda")

    def step(st, k_c, v_c, k_p):
        S.linear_decode_step_at(*lin_in, st, pos, out=lout)
        S.sparse_decode_step(q, kn, vn, g, k_c, v_c, k_p, kvl, cap, topk=topk, sel=sel, out=sout, workspace=ws)

    def new_tokens(t):
        for i, x in enumerate(lin_in):
            x.copy_(device_normal(70 + t, i, (B, H, d)))
        q.copy_(device_normal(80 + t, 0, (B, H, d)))
        g.copy_(device_normal(80 + t, 3, (B, H, d)))
        kn.copy_(device_normal(80 + t, 1, (B, Hkv, d)))
        vn.copy_(device_normal(80 + t, 2, (B, Hkv, d)))

    new_tokens(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    scratch = [state.clone(), kc.clone(), vc.clone(), kp.clone()]
    with torch.cuda.stream(s):
        step(*scratch)  # warm-up on copies, before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(state, kc, vc, kp)
    ref_state, ref_kc, ref_vc, ref_kp = state.clone(), kc.clone(), vc.clone(), kp.clone()
    for t in range(3):
        new_tokens(t)
        # eager reference on copies
        step(ref_state, ref_kc, ref_vc, ref_kp)
        torch.cuda.synchronize()
        ref = [lout.clone(), sout.clone(), sel.clone()]
        lout.zero_(); sout.zero_(); sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b_, n in zip([lout, sout, sel], ref, ("linear out", "sparse out", "sel")):
            assert torch.equal(a, b_), f"step {t}: {n}"
        assert torch.equal(state, ref_state) and torch.equal(kc, ref_kc) and torch.equal(kp, ref_kp)
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work between replays
        kvl += 1  # the next token of every sequence
        pos += 1
