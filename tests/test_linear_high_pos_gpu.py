"""GPU parity of the linear layer's prefill at positions near 1M, where RoPE angles are large
(p * theta_0 ~ 1e6 rad): the kernels reduce each segment's starting angle in fp64 and advance it
by a fixed 64-position rotation per chunk in fp32, so accuracy over a whole call at such
positions is what is checked here, against the oracle's float64 angles. Tolerance
max|gpu - ref| <= 1e-2 * max|ref| (bf16)."""

import numpy as np
import pytest

import oracle as O
from hybrid_sparse_linear_causal_amd.inputs import host_normal
from sala_testutil import assert_rel, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


def test_linear_prefill_last_4096_of_1m(S):
    """The last 4,096 tokens of a 1,048,576-token prompt (pos0 = 1,044,480), entering with a
    state of the size 1M tokens leave (std 1024 per entry)."""
    B, N, H, d, pos0 = 1, 4096, 4, 128, 1_044_480
    q, k, v, g = (host_normal(960, t, (B, N, H, d)) for t in range(4))
    s_in = host_normal(960, 4, (B, H, d, d), "f32", std=1024.0)
    ref, S_ref = O.linear_prefill(q, k, v, g, pos0=pos0, state_in=s_in)
    out, st = S.linear_prefill(*(dev(x, "bf16") for x in (q, k, v, g)), pos0=pos0, state_in=dev(s_in, "f32"))
    e1 = assert_rel(host(out), ref, 1e-2, "out")
    e2 = assert_rel(host(st), S_ref, 1e-2, "state")
    print(f"  relative errors: out {e1:.2e}, state {e2:.2e}", flush=True)


@pytest.mark.parametrize("heads", [(0, 29)])
def test_linear_prefill_segment_at_917504(S, heads):
    """The seventh 131,072-token segment of a 1M prompt processed in eight calls (pos0 = 917,504,
    32 heads, the segmented 1M workload's call shape), with a small entering state so that the
    segment's own rotated keys dominate the readout: sampled whole heads against the oracle."""
    import torch

    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    B, N, H, d, pos0 = 1, 131072, 32, 128, 917_504
    q, k, v, g = (device_normal(961, t, (B, N, H, d)) for t in range(4))
    s_in = device_normal(961, 4, (B, H, d, d), dtype="f32", std=32.0)
    out, st = S.linear_prefill(q, k, v, g, pos0=pos0, state_in=s_in)
    torch.cuda.synchronize()
    for h in heads:
        sl = [x[:, :, h:h + 1].float().cpu().numpy() for x in (q, k, v, g)]
        ref, S_ref = O.linear_prefill(*sl, pos0=pos0, state_in=s_in[:, h:h + 1].cpu().numpy())
        e1 = assert_rel(host(out[:, :, h:h + 1]), ref, 1e-2, f"out head {h}")
        e2 = assert_rel(host(st[:, h:h + 1]), S_ref, 1e-2, f"state head {h}")
        print(f"  head {h}: relative errors out {e1:.2e}, state {e2:.2e}", flush=True)
