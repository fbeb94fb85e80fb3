"""GPU parity of grouped (GQA) linear heads against the oracle: query head h reads the state of
KV head h // (H / Hkv), and the state is per KV head ("MiniCPM-SALA：融合稀疏与线性注意力实现高效
长上下文建模" §1 names grouped key/value heads as the KV-saving technique; the linear layers here
take it as an option, the state shared by each KV head's query group). Prefill (bf16 over several
segments and one segment, f32), decode at one and at per-sequence positions, packed batches, and
the 32-query / 2-KV-head shape at 32,768 tokens on sampled heads.
Tolerance max|gpu - ref| <= 1e-2 * max|ref| (bf16), 1e-4 * max|ref| (f32)."""

import numpy as np
import pytest

import oracle as O
from hybrid_sparse_linear_causal_amd.inputs import host_normal
from sala_testutil import assert_rel, dev, host

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


def _inputs(seed, B, N, H, Hkv, d, dtype):
    return (host_normal(seed, 0, (B, N, H, d), dtype), host_normal(seed, 1, (B, N, Hkv, d), dtype),
            host_normal(seed, 2, (B, N, Hkv, d), dtype), host_normal(seed, 3, (B, N, H, d), dtype))


@pytest.mark.parametrize("B,N,H,Hkv,d,dtype,pos0,with_state,with_w,alias", [
    (1, 3000, 8, 2, 128, "bf16", 17, True, True, False),    # many segments
    (2, 777, 4, 1, 128, "bf16", 5, True, False, True),      # one segment, state_out aliasing state_in
    (1, 64, 6, 3, 128, "bf16", 0, False, False, False),
    (1, 300, 6, 2, 64, "f32", 9, True, True, False),
    (2, 129, 4, 2, 128, "f32", 0, True, False, True),
])
def test_linear_prefill_grouped(S, B, N, H, Hkv, d, dtype, pos0, with_state, with_w, alias):
    import torch

    print(f"grouped linear prefill B={B} N={N} H={H} Hkv={Hkv} d={d} {dtype}", flush=True)
    q, k, v, g = _inputs(400 + N, B, N, H, Hkv, d, dtype)
    s_in = host_normal(401, 4, (B, Hkv, d, d), "f32", std=8.0) if with_state else None
    qw = (1.0 + 0.25 * host_normal(402, 5, (d,), "f32")) if with_w else None
    kw = (1.0 + 0.25 * host_normal(402, 6, (d,), "f32")) if with_w else None
    ref, S_ref = O.linear_prefill(q, k, v, g, pos0=pos0, state_in=s_in, q_norm_w=qw, k_norm_w=kw)
    st_in = None if s_in is None else dev(s_in, "f32")
    out, st = S.linear_prefill(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g, dtype), pos0=pos0, state_in=st_in,
                               state_out=st_in if alias else None, q_norm_w=None if qw is None else dev(qw, "f32"),
                               k_norm_w=None if kw is None else dev(kw, "f32"))
    torch.cuda.synchronize()
    e1 = assert_rel(host(out), ref, TOL[dtype], "out")
    e2 = assert_rel(host(st), S_ref, TOL[dtype], "state")
    print(f"  relative errors: out {e1:.2e}, state {e2:.2e}", flush=True)


def test_linear_prefill_grouped_32k_sampled(S):
    """32,768 tokens, 32 query heads over 2 KV heads: whole sampled query heads and both states."""
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    B, N, H, Hkv, d = 1, 32768, 32, 2, 128
    q, g = device_normal(403, 0, (B, N, H, d)), device_normal(403, 3, (B, N, H, d))
    k, v = device_normal(403, 1, (B, N, Hkv, d)), device_normal(403, 2, (B, N, Hkv, d))
    out, st = S.linear_prefill(q, k, v, g)
    torch.cuda.synchronize()
    for h in (0, 17, 31):
        kvh = h // (H // Hkv)
        sl = [x[:, :, i:i + 1].float().cpu().numpy() for x, i in ((q, h), (k, kvh), (v, kvh), (g, h))]
        ref, S_ref = O.linear_prefill(*sl)
        assert_rel(host(out[:, :, h:h + 1]), ref, 1e-2, f"out head {h}")
        assert_rel(host(st[:, kvh:kvh + 1]), S_ref, 1e-2, f"state kv head {kvh}")


@pytest.mark.parametrize("B,H,Hkv,d,dtype,pos", [(3, 8, 2, 128, "bf16", 1_000_003), (2, 6, 3, 64, "f32", 77),
                                                 (8, 32, 2, 128, "bf16", 1_048_575)])
def test_linear_decode_grouped(S, B, H, Hkv, d, dtype, pos):
    q, g = (host_normal(404, t, (B, H, d), dtype) for t in (0, 3))
    k, v = (host_normal(404, t, (B, Hkv, d), dtype) for t in (1, 2))
    S0 = host_normal(404, 4, (B, Hkv, d, d), "f32", std=32.0)
    ref, S_ref = O.linear_decode(q, k, v, g, S0, pos)
    st = dev(S0, "f32")
    out = S.linear_decode_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g, dtype), st, pos)
    assert_rel(host(out), ref, TOL[dtype], "out")
    assert_rel(host(st), S_ref, 1e-5, "state")


def test_linear_decode_step_at_grouped(S):
    import torch

    B, H, Hkv, d = 3, 8, 2, 128
    pos = [0, 4097, 70000]
    q, g = (host_normal(405, t, (B, H, d), "bf16") for t in (0, 3))
    k, v = (host_normal(405, t, (B, Hkv, d), "bf16") for t in (1, 2))
    S0 = host_normal(405, 4, (B, Hkv, d, d), "f32", std=4.0)
    st = dev(S0, "f32")
    out = S.linear_decode_step_at(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "bf16"), st,
                                  torch.tensor(pos, dtype=torch.int64, device="cuda"))
    for b in range(B):
        ref, S_ref = O.linear_decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], S0[b:b + 1], pos[b])
        assert_rel(host(out)[b:b + 1], ref, 1e-2, f"out {b}")
        assert_rel(host(st)[b:b + 1], S_ref, 1e-5, f"state {b}")


def test_linear_prefill_varlen_grouped(S):
    seqlens, pos0, H, Hkv, d = [333, 0, 1500, 64], [17, 3, 0, 4096], 4, 2, 128
    ns, T = len(seqlens), sum(seqlens)
    q, g = (host_normal(406, t, (T, H, d), "bf16") for t in (0, 3))
    k, v = (host_normal(406, t, (T, Hkv, d), "bf16") for t in (1, 2))
    s_in = host_normal(406, 4, (ns, Hkv, d, d), "f32", std=4.0)
    ref, S_ref = O.linear_prefill_varlen(q, k, v, g, seqlens, pos0, state_in=s_in)
    vl = S.Varlen(seqlens, pos0)
    out, st = S.linear_prefill_varlen(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "bf16"), vl,
                                      state_in=dev(s_in, "f32"))
    assert_rel(host(out), ref, 1e-2, "out")
    assert_rel(host(st), S_ref, 1e-2, "state")
