"""sala_sparse_decode_step_noalloc (scratch memory from the library's static device array, no
allocation during the call) against sala_sparse_decode_step with a caller workspace, through the
C ABI: identical selections, outputs and cache contents on two calls in a row, the second with
a smaller input (fewer sequences, shorter contexts), so the second call runs on scratch memory
that still holds the first call's partial results. (Argument errors, including calls needing
more scratch than the array holds, are checked on the CPU in test_abi.py.)"""

import pytest

from hybrid_sparse_linear_causal_amd.inputs import host_normal
from sala_testutil import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_sparse_linear_causal_amd import sala

    sala.lib()
    return sala


def _case(S, seed, lens, Hq, Hkv, topk):
    """Two identical sets of caches (one per entry point) holding each sequence's first
    lens[b] - 1 tokens, pooled, and the step's new tokens."""
    import torch

    B, d = len(lens), 128
    L = max(lens)
    cap = ((L + 63) // 64) * 64
    kc_h = host_normal(seed, 5, (B, Hkv, L, d), "bf16")
    vc_h = host_normal(seed, 6, (B, Hkv, L, d), "bf16")
    sets = []
    for _ in range(2):
        kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        kp = torch.zeros((B, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
        for b, n in enumerate(lens):
            kc[b, :, :n - 1] = dev(kc_h[b, :, :n - 1], "bf16")
            vc[b, :, :n - 1] = dev(vc_h[b, :, :n - 1], "bf16")
            if (n - 1) // 64:
                S.kv_pool(kc[b:b + 1], kp[b:b + 1], n - 1, 0, (n - 1) // 64)
        sets.append((kc, vc, kp))
    tok = dict(q=dev(host_normal(seed, 0, (B, Hq, d), "bf16"), "bf16"),
               k_new=dev(host_normal(seed, 1, (B, Hkv, d), "bf16"), "bf16"),
               v_new=dev(host_normal(seed, 2, (B, Hkv, d), "bf16"), "bf16"),
               g=dev(host_normal(seed, 3, (B, Hq, d), "bf16"), "bf16"))
    kvl = torch.tensor(lens, dtype=torch.int64, device="cuda")
    return sets, tok, kvl, L


def test_noalloc_decode_step_matches_workspace_call(S):
    import torch

    cases = [(61, [64 * 700 + 3, 64 * 300, 129, 64 * 520 + 40], 32, 2, 32),   # 4 sequences, up to 44.8K
             (62, [64 * 90 + 1, 70], 16, 1, 16)]                              # then a smaller call
    for seed, lens, Hq, Hkv, topk in cases:
        print(f"noalloc decode step lens={lens} Hq={Hq} Hkv={Hkv} topk={topk}", flush=True)
        (a, b), tok, kvl, L = _case(S, seed, lens, Hq, Hkv, topk)
        args = (tok["q"], tok["k_new"], tok["v_new"], tok["g"])
        out_w, sel_w = S.sparse_decode_step(*args, *a, kvl, L, topk=topk)
        out_n, sel_n = S.sparse_decode_step_noalloc(*args, *b, kvl, L, topk=topk)
        torch.cuda.synchronize()
        assert torch.equal(sel_w, sel_n), "selection"
        assert torch.equal(out_w, out_n), "output"
        for x, y in zip(a, b):
            assert torch.equal(x, y), "caches after the append"

