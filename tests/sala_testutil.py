"""Helpers shared by the GPU parity tests: device transfer, the tolerance rule and the
selection margin rule. Holds no arithmetic of the method."""

import numpy as np

import oracle as O

MARGIN = 1e-3


def dev(x, dtype):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_rel(gpu, ref, tol, what=""):
    """max |gpu - ref| <= tol * max |ref| (the acceptance rule for floating point)."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    err = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    assert err <= tol * scale, f"{what}: max err {err:.3e} > {tol} * {scale:.3e}"
    return err / max(scale, 1e-300)


def check_selection(gpu_sel, ref_sel, scores_fn, topk, n_local, first_block=0):
    """Bit-exact selection, except rows whose r-th / (r+1)-th candidate scores are closer than
    MARGIN: there every GPU-chosen candidate must score >= s_r - MARGIN and the forced blocks,
    ordering and padding must still be exact. scores_fn(b, g, i) -> oracle candidate scores
    (index j -> score) for query block i. Returns the number of rows accepted by the margin rule.
    """
    gpu_sel = np.asarray(gpu_sel)
    ref_sel = np.asarray(ref_sel)
    assert gpu_sel.shape == ref_sel.shape
    B, G, R, K = gpu_sel.shape
    by_margin = 0
    for b in range(B):
        for g in range(G):
            for r in range(R):
                a, e = gpu_sel[b, g, r].tolist(), ref_sel[b, g, r].tolist()
                if a == e:
                    continue
                i = first_block + r
                # structure: ascending, forced present, same count, -1 padded
                va = [x for x in a if x >= 0]
                assert va == sorted(set(va)) and a[len(va):] == [-1] * (K - len(va)), (b, g, i, a)
                assert len(va) == len([x for x in e if x >= 0]), (b, g, i, a, e)
                forced = {0} | set(range(max(0, i - n_local + 1), i + 1))
                assert forced <= set(va), (b, g, i, a)
                sc = scores_fn(b, g, i)
                cands = list(range(1, i - n_local + 1))
                ranked = sorted(cands, key=lambda j: (-sc[j], j))
                rr = topk - len(forced)
                s_r, s_r1 = sc[ranked[rr - 1]], sc[ranked[rr]]
                assert s_r - s_r1 < MARGIN, f"row {(b, g, i)}: selections differ with margin {s_r - s_r1}"
                for j in set(va) - forced:
                    assert sc[j] >= s_r - MARGIN, (b, g, i, j, sc[j], s_r)
                by_margin += 1
    return by_margin


def oracle_decode_on_selection(q_hat, k_cache_hat, v_cache, k_hat_new, v_new, sel_row, scale):
    """The oracle's sparse attention (O.sparse_attention) for one decode query over the blocks
    of a given selection row (the GPU's), for the query heads of one KV group.

    q_hat [G, d] (normalised queries); k_cache_hat, v_cache [p, d]: the normalised keys and the
    values of positions 0 .. p-1; k_hat_new, v_new [d]: the token at position p (the query's own).
    The selected blocks are gathered in ascending order and renumbered 0 .. m-1; the query's
    own block is the last of them, so the oracle's token-level causal mask applies unchanged at
    the query's renumbered position. Returns o [G, d] (before the gate)."""
    p = k_cache_hat.shape[0]
    blks = [int(j) for j in sel_row if j >= 0]
    assert blks == sorted(set(blks)) and blks[-1] == p // 64, (blks, p)
    old = np.concatenate([np.arange(j * 64, min(p, j * 64 + 64)) for j in blks])
    K = np.concatenate([np.asarray(k_cache_hat)[old].astype(np.float64), np.asarray(k_hat_new, np.float64)[None]])
    V = np.concatenate([np.asarray(v_cache)[old].astype(np.float64), np.asarray(v_new, np.float64)[None]])
    m = len(blks)
    sel_c = np.full((1, 1, m, len(sel_row)), -1, dtype=np.int64)
    sel_c[0, 0, m - 1, :m] = np.arange(m)
    q_pos = (m - 1) * 64 + (p - blks[-1] * 64)
    assert q_pos == K.shape[0] - 1
    return O.sparse_attention(np.asarray(q_hat, np.float64)[None, None], K[None, :, None], V[None, :, None],
                              sel_c, 64, scale, q_positions=[q_pos])[0, 0]
