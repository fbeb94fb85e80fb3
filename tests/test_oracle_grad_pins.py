"""Pins of the gradient oracle (oracle/sala_oracle_grad.py) to things other than itself. CPU only.

1. Its torch forward equals the numpy oracle's forward (which test_oracle_pins.py pins to the
   pages), for both layers.
2. Every gradient equals central finite differences of the numpy oracle's forward, along
   random directions and at single coordinates: this check never runs the torch code, so a
   slip in the re-expression, or in autograd's use, fails it.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import sala_oracle_grad as G

RNG = np.random.default_rng(2024)


def rnd(*shape):
    return RNG.standard_normal(shape)


def fd(f, x, u, h=1e-5):
    """Central difference of the scalar function f at x along direction u."""
    return (f(x + h * u) - f(x - h * u)) / (2 * h)


# ------------------------------------------------------------------ linear layer


def _linear_case(with_w=True, with_state=True, Hkv=2):
    B, N, H, d = 1, 6, 2, 8
    return dict(q=rnd(B, N, H, d), k=rnd(B, N, Hkv, d), v=rnd(B, N, Hkv, d), g=rnd(B, N, H, d),
                state_in=rnd(B, Hkv, d, d) if with_state else None,
                q_norm_w=rnd(d) if with_w else None, k_norm_w=rnd(d) if with_w else None,
                dout=rnd(B, N, H, d), dstate_out=rnd(B, Hkv, d, d) if with_state else None)


def _linear_loss(case, pos0):
    def loss(**over):
        a = {k: over.get(k, case[k]) for k in ("q", "k", "v", "g", "state_in", "q_norm_w", "k_norm_w")}
        out, S = O.linear_prefill(a["q"], a["k"], a["v"], a["g"], pos0=pos0, state_in=a["state_in"],
                                  q_norm_w=a["q_norm_w"], k_norm_w=a["k_norm_w"])
        val = float(np.sum(out * case["dout"]))
        if case["dstate_out"] is not None:
            val += float(np.sum(S * case["dstate_out"]))
        return val
    return loss


def test_linear_torch_forward_equals_numpy_oracle():
    c = _linear_case()
    out, S = O.linear_prefill(c["q"], c["k"], c["v"], c["g"], pos0=11, state_in=c["state_in"],
                              q_norm_w=c["q_norm_w"], k_norm_w=c["k_norm_w"])
    t = {k: (None if c[k] is None else torch.tensor(c[k])) for k in c}
    out_t, S_t = G.linear_layer(t["q"], t["k"], t["v"], t["g"], pos0=11, state_in=t["state_in"],
                                q_norm_w=t["q_norm_w"], k_norm_w=t["k_norm_w"])
    np.testing.assert_allclose(out_t.numpy(), out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S_t.numpy(), S, rtol=0, atol=1e-12)


@pytest.mark.parametrize("with_w,with_state", [(True, True), (False, False)])
def test_linear_grads_match_finite_differences(with_w, with_state):
    c = _linear_case(with_w, with_state)
    pos0 = 5
    gr = G.linear_layer_grads(c["q"], c["k"], c["v"], c["g"], c["dout"], dstate_out=c["dstate_out"], pos0=pos0,
                              state_in=c["state_in"], q_norm_w=c["q_norm_w"], k_norm_w=c["k_norm_w"])
    loss = _linear_loss(c, pos0)
    pairs = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg")]
    if with_state:
        pairs.append(("state_in", "dstate_in"))
    if with_w:
        pairs += [("q_norm_w", "dq_norm_w"), ("k_norm_w", "dk_norm_w")]
    for name, gname in pairs:
        x = c[name]
        for _ in range(2):  # random directions
            u = rnd(*x.shape)
            num = fd(lambda xx: loss(**{name: xx}), x, u)
            ana = float(np.sum(gr[gname] * u))
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(num)), (name, num, ana)
        # two single coordinates
        for flat in (0, x.size - 1):
            u = np.zeros(x.size)
            u[flat] = 1.0
            u = u.reshape(x.shape)
            num = fd(lambda xx: loss(**{name: xx}), x, u)
            assert abs(num - gr[gname].reshape(-1)[flat]) <= 1e-6 * max(1.0, abs(num)), (name, flat)
    if not with_state:
        assert gr["dstate_in"] is None and gr["dq_norm_w"] is None


def test_linear_grads_gqa_heads_share_state():
    """With 2 query heads per KV head the k, v gradients sum both heads' contributions: checked
    by finite differences (the numpy oracle maps query head h to KV head h // 2)."""
    B, N, H, Hkv, d = 1, 4, 4, 2, 8
    c = dict(q=rnd(B, N, H, d), k=rnd(B, N, Hkv, d), v=rnd(B, N, Hkv, d), g=rnd(B, N, H, d), state_in=None,
             q_norm_w=None, k_norm_w=None, dout=rnd(B, N, H, d), dstate_out=None)
    gr = G.linear_layer_grads(c["q"], c["k"], c["v"], c["g"], c["dout"])
    loss = _linear_loss(c, 0)
    for name, gname in (("k", "dk"), ("v", "dv")):
        u = rnd(*c[name].shape)
        num = fd(lambda xx: loss(**{name: xx}), c[name], u)
        assert abs(num - float(np.sum(gr[gname] * u))) <= 1e-6 * max(1.0, abs(num))


# ------------------------------------------------------------------ sparse layer


def _sparse_case():
    B, N, H, Hkv, d, blk = 1, 20, 4, 2, 8, 4
    q, g, dout = rnd(B, N, H, d), rnd(B, N, H, d), rnd(B, N, H, d)
    k_hat, v = O.qk_norm(rnd(B, N, Hkv, d)), rnd(B, N, Hkv, d)
    nqb = (N + blk - 1) // blk
    sel = np.full((B, Hkv, nqb, 3), -1, dtype=np.int64)
    for gh in range(Hkv):
        for i in range(nqb):
            picks = sorted({0, i} | ({i - 1} if i >= 1 else set()) | ({(i * 3 + gh) % (i + 1)}))
            sel[0, gh, i, :len(picks[:3])] = picks[:3]
    return dict(q=q, k_hat=k_hat, v=v, g=g, dout=dout, sel=sel, block=blk, q_norm_w=rnd(d))


def _sparse_loss(c):
    scale = 1.0 / np.sqrt(c["q"].shape[-1])

    def loss(**over):
        a = {k: over.get(k, c[k]) for k in ("q", "k_hat", "v", "g", "q_norm_w")}
        o = O.sparse_attention(O.qk_norm(a["q"], a["q_norm_w"]), a["k_hat"], a["v"], c["sel"], c["block"], scale)
        return float(np.sum(o * O.sigmoid(a["g"]) * c["dout"]))
    return loss


def test_sparse_torch_forward_equals_numpy_oracle():
    c = _sparse_case()
    scale = 1.0 / np.sqrt(c["q"].shape[-1])
    ref = O.sparse_attention(O.qk_norm(c["q"], c["q_norm_w"]), c["k_hat"], c["v"], c["sel"], c["block"], scale)
    ref = ref * O.sigmoid(c["g"])
    got = G.sparse_attention_layer(*(torch.tensor(c[k]) for k in ("q", "k_hat", "v", "g")), c["sel"],
                                   block=c["block"], q_norm_w=torch.tensor(c["q_norm_w"]))
    np.testing.assert_allclose(got.detach().numpy(), ref, rtol=0, atol=1e-12)


def test_sparse_grads_match_finite_differences():
    c = _sparse_case()
    gr = G.sparse_attention_grads(c["q"], c["k_hat"], c["v"], c["g"], c["sel"], c["dout"], block=c["block"],
                                  q_norm_w=c["q_norm_w"])
    loss = _sparse_loss(c)
    for name, gname in (("q", "dq"), ("k_hat", "dk_hat"), ("v", "dv"), ("g", "dg"), ("q_norm_w", "dq_norm_w")):
        x = c[name]
        for _ in range(2):
            u = rnd(*x.shape)
            num = fd(lambda xx: loss(**{name: xx}), x, u)
            ana = float(np.sum(gr[gname] * u))
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(num)), (name, num, ana)


def test_sparse_grads_vanish_outside_the_selection():
    """Keys of blocks no query selects, and key positions after every query that selects them,
    get zero gradient (the selection and the causal mask cut them off)."""
    c = _sparse_case()
    gr = G.sparse_attention_grads(c["q"], c["k_hat"], c["v"], c["g"], c["sel"], c["dout"], block=c["block"])
    used = np.zeros((c["k_hat"].shape[1], c["k_hat"].shape[2]), dtype=bool)
    for gh in range(c["sel"].shape[1]):
        for i in range(c["sel"].shape[2]):
            for j in c["sel"][0, gh, i]:
                if j >= 0:
                    used[j * c["block"]:(j + 1) * c["block"], gh] = True
    assert np.all(gr["dk_hat"][0][~used] == 0) and np.all(gr["dv"][0][~used] == 0)


def test_key_norm_grads_match_finite_differences():
    k, w, dk_hat = rnd(1, 5, 2, 8), rnd(8), rnd(1, 5, 2, 8)
    gr = G.key_norm_grads(k, dk_hat, w)

    def loss(kk=k, ww=w):
        return float(np.sum(O.qk_norm(kk, ww) * dk_hat))

    for x, gname, f in ((k, "dk", lambda xx: loss(kk=xx)), (w, "dk_norm_w", lambda xx: loss(ww=xx))):
        u = rnd(*x.shape)
        num = fd(f, x, u)
        assert abs(num - float(np.sum(gr[gname] * u))) <= 1e-6 * max(1.0, abs(num))


def test_sparse_grads_with_query_positions_match_finite_differences():
    """Queries at later positions (a prompt continued after earlier tokens are cached): the
    q_positions path of the torch re-expression against the numpy oracle by finite differences."""
    c = _sparse_case()
    qpos = np.arange(8, 20)  # the last 12 tokens (blocks 2..4 of 4 tokens) query the cache
    q, g, dout = c["q"][:, 8:], c["g"][:, 8:], c["dout"][:, 8:]
    sel = c["sel"]
    scale = 1.0 / np.sqrt(q.shape[-1])
    gr = G.sparse_attention_grads(q, c["k_hat"], c["v"], g, sel, dout, block=c["block"], q_positions=qpos)

    def loss(qq=q, kk=c["k_hat"], vv=c["v"]):
        o = O.sparse_attention(O.qk_norm(qq), kk, vv, sel, c["block"], scale, q_positions=qpos)
        return float(np.sum(o * O.sigmoid(g) * dout))

    for x, gname, f in ((q, "dq", lambda xx: loss(qq=xx)), (c["k_hat"], "dk_hat", lambda xx: loss(kk=xx)),
                        (c["v"], "dv", lambda xx: loss(vv=xx))):
        u = rnd(*x.shape)
        num = fd(f, x, u)
        assert abs(num - float(np.sum(gr[gname] * u))) <= 1e-6 * max(1.0, abs(num))
