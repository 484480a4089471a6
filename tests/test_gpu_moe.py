"""GPU parity of the mixture-of-experts block with router replay (dfx_dual_flow_moe_mlp).

Checked as a chain on the GPU's own intermediates (dfx_dual_flow_moe_mlp_taps): the normed
rows' bf16 decisions; router logits within their accumulation bound; the ranking a valid
descending order of the exact logits up to those bounds, and the auxiliary's experts exactly
the head of the primary's ranking (router replay); the weights as the softmax of the GPU's
logits; the expert lists bit-exact from the selections; each expert's bf16 intermediate (with
the b coupling) and the zero rows of flows that did not pick the expert; the output rows from
the GPU's intermediates and weights within the accumulation bound."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import bf16_decisions_agree, dev, unpack_rows
from oracle.linear import rmsnorm
from oracle.moe import moe_mlp
from oracle.numerics import widen

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
KMAX = 16


def gamma(k):
    """fp32 accumulation bound of a k-term dot product on the matrix cores (32-term blocks
    added in sequence, split-K partials)."""
    return (k / 32 + 64) * U


def run(c, F, k1, k2, couple=True):
    B, H = c.x.shape[1], c.x.shape[2]
    E, I = c.w_down.shape[0], c.w_down.shape[2]
    w = dfx.MoeWeights.from_row_major(dev(c.gain), dev(c.w_router), dev(c.w_gate_up), dev(c.w_down), k1, k2, c.eps,
                                      dev(c.b) if couple else None, dev(c.c) if couple else None)
    x = dev(c.x[:F].copy())
    ws = dfx.Workspace()
    dfx.moe_mlp(x, w, workspace=ws)
    torch.cuda.synchronize()
    t = dfx.moe_taps(w, B, F)
    buf = ws.buf.cpu().numpy()

    def region(name, dtype, shape):
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return buf[t[name]: t[name] + n].view(dtype).reshape(shape)

    out = dict(x=x.cpu().numpy().astype(np.float64), h=region("h", np.uint16, (F, B, H)),
               logits=region("logits", np.float32, (F, B, E)).astype(np.float64),
               ids=region("ids", np.int32, (F, B, KMAX)), wts=region("weights", np.float32, (F, B, KMAX)),
               counts=region("counts", np.int32, (E,)), seqs=region("seqs", np.int32, (E, B)))
    stride = t["inter_stride"]
    inter = buf[t["inter"]: t["inter"] + E * stride * 2].view(np.uint16).reshape(E, stride)
    out["inter"] = [unpack_rows(inter[e], F, int(out["counts"][e]), I) for e in range(E)]
    return out


def check_chain(c, F, k1, k2, couple=True, rows=None, cols=None):
    """Every stage from the GPU's previous one. rows: sequences checked past the routing;
    cols: intermediate / output columns checked (None: all)."""
    g = run(c, F, k1, k2, couple)
    B, H = c.x.shape[1], c.x.shape[2]
    E, I = c.w_down.shape[0], c.w_down.shape[2]
    b_vec = c.b if (couple and F == 2) else None
    c_vec = c.c if (couple and F == 2) else None
    rows = np.arange(B) if rows is None else np.asarray(rows)
    x0 = c.x[:F].astype(np.float64)
    # normed rows
    exact = rmsnorm(x0, c.gain, c.eps, rounded=False)
    r = 1.0 / np.sqrt(np.mean(x0 * x0, axis=-1, keepdims=True) + c.eps)
    bf16_decisions_agree(g["h"], exact, rel=1.0,
                         scale=np.abs(widen(c.gain)) * r * np.abs(x0) * (H / 2 + 8) * U + 4 * U * np.abs(exact))
    h = widen(g["h"])
    # router logits
    wr = widen(c.w_router)
    L = h @ wr.T
    ltol = (H / 64 + 8) * U * (np.abs(h) @ np.abs(wr).T) + 1e-30
    assert np.all(np.abs(g["logits"] - L) <= ltol)
    # ranking: each pick a maximum of the rest up to the bounds; the aux takes the same head
    ids = g["ids"]
    kmax = max(k1, k2) if F == 2 else k1
    head = ids[1, :, :k2] if (F == 2 and k2 >= k1) else ids[0, :, :k1]
    assert np.all(ids[0, :, k1:] == -1) and (F == 1 or np.all(ids[1, :, k2:] == -1))
    if F == 2:
        m = min(k1, k2)
        assert np.array_equal(ids[0, :, :m], ids[1, :, :m])        # router replay, bit-exact
    for b in range(B):
        sel = list(head[b])
        assert len(set(sel)) == kmax and all(0 <= e < E for e in sel)
        for rank, e in enumerate(sel):
            rest = [o for o in range(E) if o not in sel[:rank]]
            assert L[0, b, e] + ltol[0, b, e] >= max(L[0, b, o] - ltol[0, b, o] for o in rest)
    # weights: softmax of the GPU's own logits over each flow's experts
    for f, k in ((0, k1), (1, k2))[:F]:
        z = np.take_along_axis(g["logits"][f], ids[f, :, :k].astype(np.int64), axis=-1)
        e_ = np.exp(z - z.max(-1, keepdims=True))
        want = e_ / e_.sum(-1, keepdims=True)
        tol = want * (np.abs(z - z.max(-1, keepdims=True)) + 16) * 2 * U + 1e-30
        assert np.all(np.abs(g["wts"][f, :, :k] - want) <= tol)
        assert np.all(g["wts"][f, :, k:] == 0)
    # expert lists, bit-exact from the selections
    used = np.zeros((E, B), bool)
    for f, k in ((0, k1), (1, k2))[:F]:
        for b in range(B):
            used[ids[f, b, :k], b] = True
    assert np.array_equal(g["counts"], used.sum(1))
    for e in range(E):
        assert np.array_equal(g["seqs"][e, : g["counts"][e]], np.nonzero(used[e])[0])
    # intermediates of the checked rows, with b where the primary also ran the expert
    cI = np.arange(I) if cols is None else np.asarray(cols)
    picks = lambda f, b: set(ids[f, b, : (k1 if f == 0 else k2)].tolist())
    n_same = n_all = 0
    for e in range(E):
        if g["counts"][e] == 0:
            continue
        seq = list(g["seqs"][e, : g["counts"][e]])
        wg, wu = widen(c.w_gate_up[e][cI]), widen(c.w_gate_up[e][I + cI])
        for b in rows:
            if b not in seq:
                continue
            r = seq.index(b)
            hb = h[:, b]
            gate, up = hb @ wg.T, hb @ wu.T
            eg = gamma(H) * (np.abs(hb) @ np.abs(wg).T)
            eu = gamma(H) * (np.abs(hb) @ np.abs(wu).T)
            sig = 1.0 / (1.0 + np.exp(-gate))
            val = gate * sig * up
            err = 1.1 * eg * np.abs(up) + np.abs(gate * sig) * eu + 6 * U * np.abs(val)
            got = g["inter"][e][:, r][:, cI]
            if e not in picks(0, b):
                assert np.all(got[0] == 0)                  # a zero row: the primary did not pick e
                val[0], err[0] = 0.0, 0.0
            if F == 2 and e in picks(1, b):
                if b_vec is not None:
                    val[1] = val[1] + widen(b_vec)[cI] * val[0]
                    err[1] = err[1] + np.abs(widen(b_vec)[cI]) * err[0]
                n_same += bf16_decisions_agree(got[1], val[1], rel=1.0, scale=err[1] + U * np.abs(val[1]))
                n_all += 1
            if e in picks(0, b):
                n_same += bf16_decisions_agree(got[0], val[0], rel=1.0, scale=err[0] + U * np.abs(val[0]))
                n_all += 1
    # output rows from the GPU's intermediates and weights
    cH = np.arange(H) if cols is None else np.asarray(cols) % H
    for b in rows:
        m = np.zeros((F, len(cH)))
        mabs = np.zeros((F, len(cH)))
        for f, k in ((0, k1), (1, k2))[:F]:
            for j in range(k):
                e = int(ids[f, b, j])
                r = list(g["seqs"][e, : g["counts"][e]]).index(b)
                it = widen(g["inter"][e][f, r])
                wd = widen(c.w_down[e][cH])
                w = float(g["wts"][f, b, j])
                m[f] += w * (it @ wd.T)
                mabs[f] += abs(w) * (np.abs(it) @ np.abs(wd).T)
        if c_vec is not None:
            m[1] = m[1] + widen(c_vec)[cH] * m[0]
            mabs[1] = mabs[1] + np.abs(widen(c_vec)[cH]) * mabs[0]
        want = x0[:, b][:, cH] + m
        bound = (gamma(I) + (KMAX + 2) * U) * mabs + 2 * U * np.abs(want) + 1e-30
        assert np.all(np.abs(g["x"][:, b][:, cH] - want) <= bound)
    return g


SMALL = dict(hidden=256, num_experts=8, intermediate=128, router_std=0.3, w_std=0.05)


@pytest.mark.parametrize("F", [2, 1])
@pytest.mark.parametrize("k1,k2", [(2, 2), (1, 3), (4, 1)])
def test_moe_chain_small(F, k1, k2):
    c = gen.moe_case(960 + 10 * k1 + k2, 5, **SMALL)
    g = check_chain(c, F, k1, k2)
    # end to end against the oracle from x (its own routing; the small rows make ties unlikely)
    want, mid = moe_mlp(c.x[:F], c.gain, c.eps, c.w_router, c.w_gate_up, c.w_down, k1, k2,
                        c.b if F == 2 else None, c.c if F == 2 else None)
    assert np.array_equal(mid["ids"][0], g["ids"][0, :, :k1])
    err = np.abs(g["x"] - want)
    assert np.median(err) < 1e-3 and err.max() < 5e-2


def test_moe_two_row_groups_and_uncoupled():
    # 40 sequences over 2 experts, the auxiliary on both: every expert serves all 40 sequences,
    # two 32-row groups, the second partly filled
    c = gen.moe_case(971, 40, hidden=256, num_experts=2, intermediate=128, router_std=0.3, w_std=0.05)
    g = check_chain(c, 2, 1, 2)
    assert np.array_equal(g["counts"], [40, 40])
    check_chain(c, 2, 2, 1, couple=False)


def test_moe_split_k_down_projection_and_unused_experts():
    # intermediate 2048 over 8 experts: the down projection runs in K splits; 3 sequences with
    # fan-out 1 leave most of 16 experts unused (never read)
    c = gen.moe_case(972, 3, hidden=256, num_experts=16, intermediate=2048, router_std=0.3, w_std=0.03)
    g = check_chain(c, 2, 1, 1)
    assert (g["counts"] == 0).sum() >= 13


def test_moe_single_expert_equals_dense_block_on_gpu():
    c = gen.moe_case(973, 4, hidden=256, num_experts=1, intermediate=256, w_std=0.05)
    g = check_chain(c, 2, 1, 1)
    assert np.all(g["wts"][:, :, 0] == 1.0) and np.all(g["ids"][:, :, 0] == 0)


def test_moe_aux_rows_do_not_change_primary_or_choice():
    c = gen.moe_case(974, 6, **SMALL)
    a = run(c, 2, 2, 2)
    c2 = gen.moe_case(974, 6, **SMALL)
    c2.x[1] = np.random.default_rng(1).standard_normal(c2.x[1].shape).astype(np.float32) * 3
    b = run(c2, 2, 2, 2)
    assert np.array_equal(a["x"][0], b["x"][0]) and np.array_equal(a["ids"], b["ids"])


def test_moe_full_size_sampled():
    """hidden 4096, 8 experts of intermediate 14336, fan-outs 2 / 2 at batch 32: routing and lists
    whole, intermediates and outputs on sampled rows and columns."""
    c = gen.moe_case(975, 32, hidden=4096, num_experts=8, intermediate=14336, router_std=0.02)
    cols = np.random.default_rng(2).choice(4096, 96, replace=False)
    check_chain(c, 2, 2, 2, rows=[0, 13, 31], cols=cols)


def test_moe_largest_fanouts():
    """64 experts, the primary on 8 and the auxiliary on 16 (the largest fan-out), 6 sequences."""
    c = gen.moe_case(976, 6, hidden=128, num_experts=64, intermediate=64, router_std=0.3, w_std=0.05)
    g = check_chain(c, 2, 8, 16)
    assert np.all(g["ids"][1, :, :16] >= 0) and np.all(g["ids"][0, :, 8:] == -1)
