"""GPU parity of the backward entry points against the gradient oracle (float64 autograd of the
forward definitions, oracle/sala_oracle_grad.py) on the same bf16-representable seeded inputs.

Tolerance: max|gpu - ref| <= 2e-2 * max|ref| per gradient. The kernels feed MFMA with bf16
operands (the normalised, rotated q and k, dO = dout * sigmoid(g), the intra-chunk score tile
and the chunk-entry state), each a relative rounding of at most 2^-9, and every gradient passes
through two such products, plus the fp32 norm / RoPE / gate transposes; 2e-2 bounds that
(measured errors are listed in the test output)."""

import numpy as np
import pytest

from hybrid_sparse_linear_causal_amd.inputs import host_normal
from oracle import sala_oracle_grad as G
from sala_testutil import assert_rel, dev, host

pytestmark = pytest.mark.gpu

TOL = 2e-2


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
