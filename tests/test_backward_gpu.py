"""GPU parity of the backward entry points against the gradient oracle (float64 autograd of the
forward definitions, oracle/sala_oracle_grad.py) on the same bf16-representable seeded inputs.

Tolerance: max|gpu - ref| <= 1e-2 * max|ref| per gradient, the bf16 bar of the forward. The
kernels feed MFMA with bf16 operands (the normalised, rotated q and k, dO = dout * sigmoid(g),
the intra-chunk score tile and the chunk-entry state), each a relative rounding of at most 2^-9,
and every gradient passes through two such products plus the fp32 norm / RoPE / gate transposes
(measured errors are listed in the test output)."""

import numpy as np
import pytest

from hybrid_sparse_linear_causal_amd.inputs import host_normal
from oracle import sala_oracle_grad as G
from sala_testutil import assert_rel, dev, host

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


@pytest.mark.parametrize("B,N,H,pos0,with_state,with_w", [
    (1, 333, 2, 17, True, True),     # 6 segments of 64 tokens, ragged last chunk
    (2, 200, 3, 0, False, False),
    (1, 1500, 2, 5, True, False),    # 24 segments
    (1, 64, 1, 3, False, True),      # exactly one chunk
    (1, 1, 2, 9, True, True),        # a single token
])
def test_linear_backward(S, B, N, H, pos0, with_state, with_w):
    print(f"linear_backward B={B} N={N} H={H} pos0={pos0} state={with_state} w={with_w}", flush=True)
    d = 128
    q, k, v, g, dout = (host_normal(300 + N, t, (B, N, H, d), "bf16") for t in range(5))
    s_in = host_normal(301, 5, (B, H, d, d), "f32", std=4.0) if with_state else None
    ds_out = host_normal(301, 6, (B, H, d, d), "f32", std=0.05) if with_state else None
    qw = (1.0 + 0.25 * host_normal(302, 7, (d,), "f32")) if with_w else np.ones(d)
    kw = (1.0 + 0.25 * host_normal(302, 8, (d,), "f32")) if with_w else np.ones(d)
    ref = G.linear_layer_grads(q, k, v, g, dout, dstate_out=ds_out, pos0=pos0, state_in=s_in,
                               q_norm_w=qw, k_norm_w=kw)
    got = S.linear_backward(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "bf16"), dev(dout, "bf16"),
                            pos0=pos0, state_in=None if s_in is None else dev(s_in, "f32"),
                            dstate_out=None if ds_out is None else dev(ds_out, "f32"),
                            q_norm_w=dev(qw, "f32") if with_w else None, k_norm_w=dev(kw, "f32") if with_w else None,
                            need_norm_w_grads=True)
    errs = {}
    for name in ("dq", "dk", "dv", "dg", "dq_norm_w", "dk_norm_w"):
        errs[name] = assert_rel(host(got[name]), ref[name], TOL, name)
    ds_ref = ref["dstate_in"] if with_state else G.linear_layer_grads(
        q, k, v, g, dout, pos0=pos0, state_in=np.zeros((B, H, d, d)), q_norm_w=qw, k_norm_w=kw)["dstate_in"]
    errs["dstate_in"] = assert_rel(host(got["dstate_in"]), ds_ref, TOL, "dstate_in")
    print("  relative errors:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)


def test_linear_backward_empty_sequence(S):
    """N = 0: the state passes through, so dstate_in = dstate_out; the weight gradients are 0."""
    import torch

    ds_out = dev(host_normal(7, 1, (1, 2, 128, 128), "f32"), "f32")
    z = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    got = S.linear_backward(z, z, z, z, z, dstate_out=ds_out, need_norm_w_grads=True)
    torch.cuda.synchronize()
    assert torch.equal(got["dstate_in"], ds_out)
    assert int(torch.count_nonzero(got["dq_norm_w"])) == 0 and got["dq"].numel() == 0


# ---------------------------------------------------------------- sparse layer


def _sparse_setup(S, seed, B, kv_len, n_q, Hq, Hkv, topk, with_w):
    """Caches filled by kv_append (the prefix, then the n_q queried tokens), the selection of the
    queried tokens by block_select; returns host copies for the oracle."""
    import torch

    d, cap = 128, ((kv_len + 63) // 64) * 64
    q, g, dout = (host_normal(seed, t, (B, n_q, Hq, d), "bf16") for t in range(3))
    k, v = (host_normal(seed, t, (B, kv_len, Hkv, d), "bf16") for t in (3, 4))
    qw = (1.0 + 0.25 * host_normal(seed, 5, (d,), "f32")) if with_w else None
    kw = (1.0 + 0.25 * host_normal(seed, 6, (d,), "f32")) if with_w else None
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    p0 = kv_len - n_q
    wk = None if kw is None else dev(kw, "f32")
    if p0 > 0:
        S.kv_append(dev(k[:, :p0], "bf16"), dev(v[:, :p0], "bf16"), kc, vc, kp, p0, n_heads=Hq, k_norm_w=wk)
    S.kv_append(dev(k[:, p0:], "bf16"), dev(v[:, p0:], "bf16"), kc, vc, kp, kv_len, n_heads=Hq, k_norm_w=wk)
    qd = dev(q, "bf16")
    wq = None if qw is None else dev(qw, "f32")
    sel = S.block_select(qd, kp, kv_len, cap, n_kv_heads=Hkv, topk=topk, n_local=2, q_norm_w=wq)
    # oracle inputs: the cache contents token-major, the selection indexed by absolute query block
    k_hat = host(kc)[:, :, :kv_len].transpose(0, 2, 1, 3)
    v_h = host(vc)[:, :, :kv_len].transpose(0, 2, 1, 3)
    sel_h = sel.cpu().numpy()
    nqb_all = (kv_len + 63) // 64
    sel_full = np.full((B, Hkv, nqb_all, topk), -1, dtype=np.int64)
    sel_full[:, :, p0 // 64:] = sel_h
    return dict(q=q, g=g, dout=dout, k=k, qw=qw, kw=kw, kc=kc, vc=vc, sel=sel, qd=qd, wq=wq, wk=wk,
                k_hat=k_hat, v=v_h, sel_full=sel_full, p0=p0, cap=cap)


@pytest.mark.parametrize("B,kv_len,n_q,Hq,Hkv,topk,with_w", [
    (1, 640, 640, 4, 2, 4, True),       # 10 query blocks
    (1, 2150, 2150, 2, 1, 6, False),    # 34 query blocks: block 0 chosen by 34 > one slice; ragged tail; 2 heads
    (1, 640, 256, 4, 2, 4, True),       # queries continue a cached prefix of 384 tokens
    (2, 384, 384, 32, 2, 3, False),     # a 16-head GQA group (4 head quads), batch 2
    (1, 17000, 17000, 2, 1, 4, True),   # 266 query blocks: two ranges of the dK/dV slices (256 query blocks each)
])
def test_sparse_attn_backward(S, B, kv_len, n_q, Hq, Hkv, topk, with_w):
    print(f"sparse_attn_backward B={B} kv_len={kv_len} n_q={n_q} Hq={Hq} Hkv={Hkv} topk={topk} w={with_w}",
          flush=True)
    c = _sparse_setup(S, 500 + kv_len + n_q, B, kv_len, n_q, Hq, Hkv, topk, with_w)
    got = S.sparse_attn_backward(c["qd"], c["kc"], c["vc"], dev(c["g"], "bf16"), c["sel"], kv_len,
                                 dev(c["dout"], "bf16"), topk=topk, q_norm_w=c["wq"], need_norm_w_grad=True)
    qw = c["qw"] if with_w else np.ones(128)
    ref = G.sparse_attention_grads(c["q"], c["k_hat"], c["v"], c["g"], c["sel_full"], c["dout"], q_norm_w=qw,
                                   q_positions=np.arange(c["p0"], kv_len))
    errs = {}
    errs["dq"] = assert_rel(host(got["dq"]), ref["dq"], TOL, "dq")
    errs["dg"] = assert_rel(host(got["dg"]), ref["dg"], TOL, "dg")
    errs["dq_norm_w"] = assert_rel(host(got["dq_norm_w"]), ref["dq_norm_w"], TOL, "dq_norm_w")
    dk = host(got["dk_cache"])
    dv = host(got["dv_cache"])
    errs["dk_cache"] = assert_rel(dk[:, :, :kv_len].transpose(0, 2, 1, 3), ref["dk_hat"], TOL, "dk_cache")
    errs["dv_cache"] = assert_rel(dv[:, :, :kv_len].transpose(0, 2, 1, 3), ref["dv"], TOL, "dv_cache")
    assert np.all(dk[:, :, kv_len:] == 0) and np.all(dv[:, :, kv_len:] == 0)  # capacity past kv_len
    print("  relative errors:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)

    # the key normalisation of the appended tokens, given this cache gradient
    dk_new, dkw = S.kv_norm_backward(dev(c["k"][:, c["p0"]:], "bf16"), got["dk_cache"], kv_len, n_heads=Hq,
                                     k_norm_w=c["wk"], need_norm_w_grad=True)
    kref = G.key_norm_grads(c["k"][:, c["p0"]:], dk[:, :, c["p0"]:kv_len].transpose(0, 2, 1, 3),
                            c["kw"] if with_w else np.ones(128))
    assert_rel(host(dk_new), kref["dk"], 1e-4, "dk_new")
    assert_rel(host(dkw), kref["dk_norm_w"], 1e-4, "dk_norm_w")


def test_sparse_attn_backward_repeatable(S):
    """The key/value gradients are summed in a fixed order: two calls give identical bits."""
    import torch

    c = _sparse_setup(S, 77, 1, 2150, 2150, 2, 1, 6, False)
    a = S.sparse_attn_backward(c["qd"], c["kc"], c["vc"], dev(c["g"], "bf16"), c["sel"], 2150, dev(c["dout"], "bf16"))
    b = S.sparse_attn_backward(c["qd"], c["kc"], c["vc"], dev(c["g"], "bf16"), c["sel"], 2150, dev(c["dout"], "bf16"))
    torch.cuda.synchronize()
    for n in ("dq", "dg", "dk_cache", "dv_cache"):
        assert torch.equal(a[n], b[n]), n


def test_sparse_attn_backward_from_saved_forward(S):
    """The backward given the forward's out and lse (no forward rerun) against the oracle and the
    recomputing backward; the forward's lse against the log2-sum-exp2 of the oracle's scaled
    scores over the selected keys (scipy)."""
    import torch
    from scipy.special import logsumexp

    B, kv_len, n_q, Hq, Hkv, topk = 1, 2150, 2150, 4, 2, 6
    c = _sparse_setup(S, 91, B, kv_len, n_q, Hq, Hkv, topk, True)
    g = dev(c["g"], "bf16")
    lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device="cuda")
    out = S.sparse_attn(c["qd"], c["kc"], c["vc"], g, c["sel"], kv_len, q_norm_w=c["wq"], lse=lse)
    saved = S.sparse_attn_backward(c["qd"], c["kc"], c["vc"], g, c["sel"], kv_len, dev(c["dout"], "bf16"),
                                   topk=topk, q_norm_w=c["wq"], need_norm_w_grad=True, out=out, lse=lse)
    rerun = S.sparse_attn_backward(c["qd"], c["kc"], c["vc"], g, c["sel"], kv_len, dev(c["dout"], "bf16"),
                                   topk=topk, q_norm_w=c["wq"], need_norm_w_grad=True)
    ref = G.sparse_attention_grads(c["q"], c["k_hat"], c["v"], c["g"], c["sel_full"], c["dout"], q_norm_w=c["qw"],
                                   q_positions=np.arange(c["p0"], kv_len))
    errs = {}
    for n, rn in (("dq", "dq"), ("dg", "dg"), ("dq_norm_w", "dq_norm_w")):
        errs[n] = assert_rel(host(saved[n]), ref[rn], TOL, n)
        assert_rel(host(saved[n]), host(rerun[n]), TOL, n + " vs rerun")
    dk, dv = host(saved["dk_cache"]), host(saved["dv_cache"])
    errs["dk_cache"] = assert_rel(dk[:, :, :kv_len].transpose(0, 2, 1, 3), ref["dk_hat"], TOL, "dk_cache")
    errs["dv_cache"] = assert_rel(dv[:, :, :kv_len].transpose(0, 2, 1, 3), ref["dv"], TOL, "dv_cache")
    print("  relative errors:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    # lse of a sample of rows: log2 sum over the selected causal keys of exp(scale * q^ . k^)
    import oracle as O
    qh = O.qk_norm(c["q"], c["qw"])
    got = host(lse)
    for t in (0, 63, 64, 1000, 2149):
        i = t // 64
        for h in range(Hq):
            gk = h // (Hq // Hkv)
            keys = np.concatenate([np.arange(j * 64, min(kv_len, (j + 1) * 64)) for j in c["sel_full"][0, gk, i]
                                   if j >= 0])
            keys = keys[keys <= t]
            s = (c["k_hat"][0, keys, gk] @ qh[0, t, h]) / np.sqrt(128)
            want = logsumexp(s) / np.log(2)
            assert abs(got[0, t, h] - want) <= 1e-2 * max(1.0, abs(want)), (t, h, got[0, t, h], want)
