"""Pins for the oracle's mixture-of-experts MLP with router replay (CPU only).

Checked against things other than the oracle itself: the dense SwiGLU block composed from
the separately pinned linear / norm / SwiGLU primitives (an MoE whose experts are all equal
is that block), torch's topk and softmax for the routing, and the invariances the pages fix
(the auxiliary flow reuses the primary's choice; the primary path never sees the auxiliary)."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
from oracle.linear import grouped_linear, rmsnorm, swiglu_couple
from oracle.moe import moe_mlp, ranking, route
from oracle.numerics import widen


def dense_block(x, gain, eps, w_gate_up, w_down, b=None, c=None):
    """The dense MLP sublayer: norm, shared gate/up, SwiGLU with b, down, c, residual."""
    h = rmsnorm(x, gain, eps)
    inter = swiglu_couple(grouped_linear(h, w_gate_up), b)
    m = grouped_linear(inter, w_down)
    if c is not None:
        m[1] = m[1] + widen(c) * m[0]
    return np.asarray(x, np.float64) + m


def same_experts(c, E):
    """The case with every expert equal to expert 0."""
    c.w_gate_up = np.repeat(c.w_gate_up[:1], E, axis=0)
    c.w_down = np.repeat(c.w_down[:1], E, axis=0)
    return c


@pytest.mark.parametrize("k1,k2", [(2, 2), (3, 1), (1, 1), (4, 4)])
def test_equal_experts_reduce_to_the_dense_block(k1, k2):
    c = same_experts(gen.moe_case(1, 3, 64, 4, 32, router_std=0.3), 4)
    got, _ = moe_mlp(c.x, c.gain, c.eps, c.w_router, c.w_gate_up, c.w_down, k1, k2, c.b, c.c)
    want = dense_block(c.x, c.gain, c.eps, c.w_gate_up[0], c.w_down[0], c.b, c.c)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_aux_fanout_past_the_primary_gets_no_b_coupling():
    """k2 > k1 with equal experts: the auxiliary output mixes the coupled dense block (weight:
    its mass on the primary's experts) and the uncoupled one (the rest)."""
    c = same_experts(gen.moe_case(2, 3, 64, 4, 32, router_std=0.3), 4)
    k1, k2 = 1, 3
    got, mid = moe_mlp(c.x, c.gain, c.eps, c.w_router, c.w_gate_up, c.w_down, k1, k2, c.b, None)
    coupled = dense_block(c.x, c.gain, c.eps, c.w_gate_up[0], c.w_down[0], c.b)
    plain = dense_block(c.x, c.gain, c.eps, c.w_gate_up[0], c.w_down[0], None)
    share = mid["weights"][1][:, :k1].sum(-1)[:, None]
    x = c.x[1].astype(np.float64)
    want = x + share * (coupled[1] - x) + (1 - share) * (plain[1] - x)
    assert np.allclose(got[1], want, rtol=0, atol=1e-12)
    assert np.allclose(got[0], plain[0], rtol=0, atol=1e-12)


def test_routing_matches_torch_topk_and_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((2, 6, 16))
    for k1, k2 in ((2, 2), (4, 2), (2, 5)):
        ids, w = route(logits, k1, k2)
        lp = torch.from_numpy(logits[0])
        for f, k in ((0, k1), (1, k2)):
            top = torch.topk(lp, k, dim=-1).indices.numpy()        # distinct logits: unique order
            assert np.array_equal(ids[f], top)
            zf = torch.gather(torch.from_numpy(logits[f]), -1, torch.from_numpy(top))
            assert np.allclose(w[f], torch.softmax(zf, dim=-1).numpy(), rtol=0, atol=1e-15)
    # equal logits rank the lower expert id first
    tie = np.zeros((1, 8))
    tie[0, [5, 2, 7]] = 1.0
    assert list(ranking(tie)[0][:4]) == [2, 5, 7, 0]


def test_router_replay_aux_reuses_primary_choice_and_primary_is_blind_to_aux():
    c = gen.moe_case(4, 4, 64, 8, 32, router_std=0.5)
    k1, k2 = 2, 3
    base, mid = moe_mlp(c.x, c.gain, c.eps, c.w_router, c.w_gate_up, c.w_down, k1, k2, c.b, c.c)
    x2 = c.x.copy()
    x2[1] = np.random.default_rng(9).standard_normal(x2[1].shape).astype(np.float32) * 3
    other, mid2 = moe_mlp(x2, c.gain, c.eps, c.w_router, c.w_gate_up, c.w_down, k1, k2, c.b, c.c)
    assert np.array_equal(mid2["ids"][1], mid["ids"][1])           # the choice is the primary's
    assert np.array_equal(mid["ids"][1][:, :k1], mid["ids"][0])     # same ranking, k2 > k1 extends it
    assert not np.allclose(mid2["weights"][1], mid["weights"][1])   # ... weighted by its own logits
    assert np.array_equal(other[0], base[0])                        # primary blind to the aux row
    # the aux's own choice (its logits' top-k2) would in general differ: the replay is a real constraint
    own = np.argsort(-mid2["logits"][1], axis=-1, kind="stable")[:, :k2]
    assert not np.array_equal(np.sort(own, -1), np.sort(mid2["ids"][1], -1))


def test_uncoupled_equal_rows_give_equal_flows():
    c = gen.moe_case(5, 3, 64, 4, 32, couple=False, router_std=0.3)
    x = np.stack([c.x[0], c.x[0]])
    got, _ = moe_mlp(x, c.gain, c.eps, c.w_router, c.w_gate_up, c.w_down, 2, 2)
    assert np.array_equal(got[0], got[1])


def test_selection_override_is_used():
    c = gen.moe_case(6, 2, 64, 4, 32)
    ids = [np.array([[3], [1]]), np.array([[3], [1]])]
    wts = [np.ones((2, 1)), np.ones((2, 1))]
    got, _ = moe_mlp(c.x, c.gain, c.eps, c.w_router, c.w_gate_up, c.w_down, 1, 1, None, None, selection=(ids, wts))
    for bb, e in ((0, 3), (1, 1)):
        want = dense_block(c.x[:, bb:bb + 1], c.gain, c.eps, c.w_gate_up[e], c.w_down[e])
        assert np.allclose(got[:, bb:bb + 1], want, rtol=0, atol=1e-12)
