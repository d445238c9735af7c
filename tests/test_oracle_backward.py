"""Pins for the backward oracle (oracle/backward.py) against facts that do not
come from its gradient formulas: central finite differences of the forward,
the forward against the C oracle, exact invariants of softmax attention, and
the special cases where one branch is plain (causal, banded or block-mean)
attention, differentiated by torch autograd in float64.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as BW
from tests import helpers as H


def _tiny(**kw):
    p = H.problem(q_len=40, kv_len=40, n_groups=2, heads_per_group=2, d_qk=8, d_v=6,
                  block=8, top_k=3, window=12)
    p.update(kw)
    return p


def _inputs64(prob, seed=0):
    """float64 inputs (held in 'f32' problems: no storage rounding anywhere)."""
    rng = np.random.default_rng(seed)
    B, T, L = prob["batch"], prob["q_len"], prob["kv_len"]
    G, hpg = prob["n_groups"], prob["heads_per_group"]
    Hh = G * hpg
    q = rng.standard_normal((B, T, Hh, prob["d_qk"]))
    k = rng.standard_normal((B, L, G, prob["d_qk"]))
    k += 0.7 * rng.standard_normal((B, L // prob["block"] + 1, 1, prob["d_qk"])).repeat(prob["block"], axis=1)[:, :L]
    v = rng.standard_normal((B, L, G, prob["d_v"]))
    gates = rng.uniform(-1.5, 1.5, (B, T, Hh, 3)) if prob["gate_logits"] else rng.uniform(0.1, 1.0, (B, T, Hh, 3))
    dout = rng.standard_normal((B, T, Hh, prob["d_v"]))
    return q, k, v, gates, dout


def _selection(prob, q, k, v):
    """A valid selection from the C oracle on float32 copies."""
    q32, k32, v32 = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v))
    kc, vc = oracle.pool(prob, k32, v32)
    idx, _, _ = oracle.select(prob, q32, kc, vc, want_imp=False, want_cmp=False)
    return idx.reshape(prob["batch"], prob["q_len"], prob["n_groups"], prob["top_k"])


def _loss(prob, q, k, v, gates, idx, dout):
    out, _ = BW.forward(prob, q, k, v, gates, idx, rounded=False)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("gate_logits", [0, 1])
@pytest.mark.parametrize("branches", [(1, 1, 1), (1, 0, 0), (0, 1, 0), (0, 0, 1)])
def test_backward_matches_finite_differences(gate_logits, branches):
    prob = _tiny(gate_logits=gate_logits, use_cmp=branches[0], use_slc=branches[1], use_win=branches[2])
    q, k, v, gates, dout = _inputs64(prob, seed=3 + gate_logits)
    idx = _selection(prob, q, k, v)
    dq, dk, dv, dg = BW.backward(prob, q, k, v, gates, idx, dout, rounded=False)
    rng = np.random.default_rng(11)
    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("gates", gates, dg)):
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, 12, replace=False):
            keep = flat[i]
            flat[i] = keep + eps
            lp = _loss(prob, q, k, v, gates, idx, dout)
            flat[i] = keep - eps
            lm = _loss(prob, q, k, v, gates, idx, dout)
            flat[i] = keep
            fd = (lp - lm) / (2 * eps)
            an = grad.reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, an)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_matches_c_oracle(dtype):
    prob = H.problem(q_len=96, kv_len=160, n_groups=2, heads_per_group=3, d_qk=16, d_v=8,
                     block=16, top_k=3, window=24, dtype=dtype, gate_logits=1)
    x = H.make(prob)
    ref = oracle.forward(prob, x["q"], x["k"], x["v"], x["gates"])
    idx = ref["idx"].reshape(prob["batch"], prob["q_len"], prob["n_groups"], prob["top_k"])
    out, O = BW.forward(prob, x["q"], x["k"], x["v"], x["gates"], idx, rounded=True)
    R = prob["batch"] * prob["q_len"]
    np.testing.assert_allclose(out.reshape(R, -1, prob["d_v"]), ref["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(O[1].reshape(R, -1, prob["d_v"]), ref["o_slc"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(O[2].reshape(R, -1, prob["d_v"]), ref["o_win"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(O[0].reshape(R, -1, prob["d_v"]), ref["o_cmp"], rtol=0, atol=1e-12)


def test_invariants_key_gradients_sum_to_zero_and_value_gradients_to_weighted_dout():
    # sum_s dS[s] = 0 for every row and branch, so dk summed over all keys
    # (the pooled part included) vanishes; probabilities sum to one, so dv
    # summed over all keys is the sum of gamma_b * dout over rows whose key
    # set is not empty.
    prob = H.problem(q_len=80, kv_len=120, n_groups=2, heads_per_group=2, d_qk=16, d_v=8,
                     block=8, top_k=4, window=20)
    q, k, v, gates, dout = _inputs64(prob, seed=5)
    idx = _selection(prob, q, k, v)
    dq, dk, dv, dg = BW.backward(prob, q, k, v, gates, idx, dout)
    hpg = prob["heads_per_group"]
    for g in range(prob["n_groups"]):
        np.testing.assert_allclose(dk[0, :, g].sum(axis=0), 0.0, atol=1e-10)
        want = np.zeros(prob["d_v"])
        for t in range(prob["q_len"]):
            sets = BW.key_sets(prob, idx, 0, t, g)
            for br in range(3):
                if len(sets[br]):
                    want += (gates[0, t, g * hpg:(g + 1) * hpg, br][:, None] * dout[0, t, g * hpg:(g + 1) * hpg]).sum(0)
        np.testing.assert_allclose(dv[0, :, g].sum(axis=0), want, rtol=0, atol=1e-10)


def _autograd_attention(q, k, v, mask, scale, dout):
    """dq, dk, dv of softmax attention with a boolean mask [T, N] by torch
    autograd in float64 (GQA: q [T, hpg, d], k, v [N, d] shared)."""
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    logits = torch.einsum("thd,nd->thn", qt, kt) * scale
    logits = logits.masked_fill(~torch.from_numpy(mask)[:, None, :], float("-inf"))
    o = torch.einsum("thn,nd->thd", torch.softmax(logits, dim=-1), vt)
    (o * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_selected_branch_with_every_block_is_causal_attention():
    prob = H.problem(q_len=64, kv_len=64, n_groups=1, heads_per_group=3, d_qk=8, d_v=8, block=8,
                     top_k=8, window=0, use_cmp=0, use_slc=1, use_win=0)
    q, k, v, _, dout = _inputs64(prob, seed=7)
    idx = _selection(prob, q, k, v)
    dq, dk, dv, _ = BW.backward(prob, q, k, v, None, idx, dout)
    mask = np.tril(np.ones((64, 64), dtype=bool))
    rq, rk, rv = _autograd_attention(q[0], k[0, :, 0], v[0, :, 0], mask, H.default_scale(prob), dout[0])
    np.testing.assert_allclose(dq[0], rq, atol=1e-12)
    np.testing.assert_allclose(dk[0, :, 0], rk, atol=1e-12)
    np.testing.assert_allclose(dv[0, :, 0], rv, atol=1e-12)


def test_window_branch_is_banded_attention():
    prob = H.problem(q_len=50, kv_len=70, n_groups=1, heads_per_group=2, d_qk=8, d_v=4, block=8,
                     top_k=2, window=9, use_cmp=0, use_slc=0, use_win=1)
    q, k, v, _, dout = _inputs64(prob, seed=8)
    idx = _selection(prob, q, k, v)
    dq, dk, dv, _ = BW.backward(prob, q, k, v, None, idx, dout)
    pos = H.positions(prob)
    s = np.arange(70)
    mask = (s[None, :] <= pos[:, None]) & (s[None, :] > pos[:, None] - 9)
    rq, rk, rv = _autograd_attention(q[0], k[0, :, 0], v[0, :, 0], mask, H.default_scale(prob), dout[0])
    np.testing.assert_allclose(dq[0], rq, atol=1e-12)
    np.testing.assert_allclose(dk[0, :, 0], rk, atol=1e-12)
    np.testing.assert_allclose(dv[0, :, 0], rv, atol=1e-12)


def test_compressed_branch_is_attention_over_block_means():
    # torch differentiates through its own mean of each block (the pooling's
    # 1 / block spreading), then attention over the means under the
    # block-causal mask
    prob = H.problem(q_len=48, kv_len=76, n_groups=1, heads_per_group=2, d_qk=8, d_v=4, block=8,
                     top_k=2, window=0, use_cmp=1, use_slc=0, use_win=0)
    q, k, v, _, dout = _inputs64(prob, seed=9)
    idx = _selection(prob, q, k, v)
    dq, dk, dv, _ = BW.backward(prob, q, k, v, None, idx, dout, rounded=False)
    nb = 76 // 8
    qt = torch.tensor(q[0], requires_grad=True)
    kt = torch.tensor(k[0, :, 0], requires_grad=True)
    vt = torch.tensor(v[0, :, 0], requires_grad=True)
    kc = kt[:nb * 8].reshape(nb, 8, -1).mean(1)
    vc = vt[:nb * 8].reshape(nb, 8, -1).mean(1)
    pos = torch.from_numpy(H.positions(prob))
    vis = (torch.arange(nb)[None, :] + 1) * 8 <= pos[:, None] + 1
    logits = torch.einsum("thd,nd->thn", qt, kc) * H.default_scale(prob)
    logits = logits.masked_fill(~vis[:, None, :], float("-inf"))
    pr = torch.nan_to_num(torch.softmax(logits, dim=-1), nan=0.0)
    o = torch.einsum("thn,nd->thd", pr, vc)
    (o * torch.from_numpy(dout[0])).sum().backward()
    np.testing.assert_allclose(dq[0], qt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk[0, :, 0], kt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv[0, :, 0], vt.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("gate_logits", [0, 1])
def test_query_grads_of_chosen_rows_equal_the_full_backward(gate_logits):
    prob = _tiny(gate_logits=gate_logits, q_len=30, kv_len=52)
    q, k, v, gates, dout = _inputs64(prob, seed=12)
    idx = _selection(prob, q, k, v)
    dq, _, _, dg = BW.backward(prob, q, k, v, gates, idx, dout)
    rows = np.array([0, 7, 29])
    dq_r, dg_r = BW.query_grads(prob, q, k, v, gates, idx, dout, rows)
    np.testing.assert_allclose(dq_r, dq.reshape(-1, *dq.shape[2:])[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dg_r, dg.reshape(-1, *dg.shape[2:])[rows], rtol=0, atol=1e-12)


def test_branch_lse_is_torch_logsumexp_on_the_plain_cases():
    # selected branch with every block chosen = causal, window = banded,
    # compressed = block-causal over torch's own block means
    prob = H.problem(q_len=40, kv_len=64, n_groups=1, heads_per_group=3, d_qk=8, d_v=4, block=8,
                     top_k=8, window=11, use_cmp=1, use_slc=1, use_win=1)
    q, k, v, _, _ = _inputs64(prob, seed=21)
    idx = _selection(prob, q, k, v)
    lse = BW.branch_lse(prob, q, k, v, idx, rounded=False)
    sc = H.default_scale(prob)
    pos = torch.from_numpy(H.positions(prob))
    s = torch.arange(64)
    qt, kt = torch.from_numpy(q[0]), torch.from_numpy(k[0, :, 0])
    z = torch.einsum("thd,sd->ths", qt, kt) * sc
    causal = s[None, :] <= pos[:, None]
    band = causal & (s[None, :] > pos[:, None] - 11)
    for br, mask in ((1, causal), (2, band)):
        want = torch.logsumexp(z.masked_fill(~mask[:, None, :], float("-inf")), dim=-1).numpy()
        np.testing.assert_allclose(lse[br, 0], want, rtol=0, atol=1e-12)
    kc = kt.reshape(8, 8, -1).mean(1)
    zc = torch.einsum("thd,nd->thn", qt, kc) * sc
    vis = (torch.arange(8)[None, :] + 1) * 8 <= pos[:, None] + 1
    want = torch.logsumexp(zc.masked_fill(~vis[:, None, :], float("-inf")), dim=-1).numpy()
    np.testing.assert_allclose(lse[0, 0], want, rtol=0, atol=1e-12)   # -inf where no block is complete
    assert np.all(np.isneginf(lse[0, 0][H.positions(prob) < 7]))


def test_branch_lse_single_key_and_disabled_branches():
    # a one-token window holds the query's own key: lse is that one logit
    prob = _tiny(window=1, use_cmp=0, use_slc=1, use_win=1)
    q, k, v, _, _ = _inputs64(prob, seed=22)
    idx = _selection(prob, q, k, v)
    lse = BW.branch_lse(prob, q, k, v, idx, rounded=False)
    sc = H.default_scale(prob)
    pos = H.positions(prob)
    for t in range(prob["q_len"]):
        for h in range(4):
            want = sc * float(q[0, t, h] @ k[0, pos[t], h // 2])
            assert abs(lse[2, 0, t, h] - want) <= 1e-12 * max(1.0, abs(want))
    assert np.all(np.isneginf(lse[0]))            # compressed branch off
    assert np.all(np.isfinite(lse[1]))            # the forced current block is never empty


@pytest.mark.parametrize("gate_logits", [0, 1])
def test_gradient_magnitudes_bound_the_gradients(gate_logits):
    """|sum of terms| <= sum of |terms|: every gradient entry lies within its
    magnitude (the basis of the element-wise GPU tolerance)."""
    prob = _tiny(gate_logits=gate_logits)
    q, k, v, gates, dout = _inputs64(prob, seed=7)
    idx = _selection(prob, q, k, v)
    grads = BW.backward(prob, q, k, v, gates, idx, dout, rounded=False)
    mags = BW.backward_magnitudes(prob, q, k, v, gates, idx, dout, rounded=False)
    for name, g, a in zip(("dq", "dk", "dv", "dgates"), grads, mags):
        assert g.shape == a.shape, name
        assert np.all(a >= 0), name
        assert np.all(np.abs(g) <= a * (1 + 1e-12) + 1e-300), name


def test_gradient_magnitudes_equal_the_gradients_when_no_term_cancels():
    """With v, dout and the gates non-negative, every term of dv and of
    dgates (softmax weights times non-negative values) is non-negative, so
    their magnitudes are the gradients themselves; a dropped term or a wrong
    weight in the magnitudes would show here."""
    prob = _tiny()
    q, k, v, gates, dout = _inputs64(prob, seed=9)
    v, dout = np.abs(v), np.abs(dout)
    idx = _selection(prob, q, k, v)
    _, _, dv, dg = BW.backward(prob, q, k, v, gates, idx, dout, rounded=False)
    _, _, av, ag = BW.backward_magnitudes(prob, q, k, v, gates, idx, dout, rounded=False)
    np.testing.assert_allclose(av, dv, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(ag, dg, rtol=1e-12, atol=1e-300)
