"""TEST INFRASTRUCTURE ONLY -- fp64 numpy statement of the NSA backward pass.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares nothing with the GPU library.

What is differentiated ([P1] "Zhang Xiaojun Business Interviews #94"
transcript, s4 "Inside Native Sparse Attention": the gated sum of the
compressed, selected and window branches; s6 "Why Sparse Attention Wins":
NSA trains end to end, the top-k choice itself passes no gradient, and the
compressed branch's output is what carries a training signal to every
block).  For query row t (position p = L - T + t), head h of group g and
branch b with key set S_b(t) and values V:

    P_b[s]  = softmax_s( scale * q_h . k_s )          s in S_b(t)
    O_b     = sum_s P_b[s] v_s                         (0 for an empty set)
    out     = sum_b gamma_b O_b                        gamma_b = gate (or its sigmoid)

Given dout = dL/dout, with the selection idx held fixed (it is an argument,
not a function of the inputs):

    dgamma_b = <dout, O_b>
    dP_b[s]  = gamma_b <dout, v_s>
    dS_b[s]  = P_b[s] (dP_b[s] - gamma_b dgamma_b)    (softmax derivative)
    dq_h    += scale * sum_s dS_b[s] k_s
    dk_s    += scale * dS_b[s] q_h                     (summed over the group's heads)
    dv_s    += P_b[s] gamma_b dout

The compressed branch's keys and values are the block means, so its dk_j
and dv_j reach every token of block j divided by the block size.  The
summaries are rounded to the storage type in the forward exactly as the
forward oracle rounds them; that rounding is passed through unchanged here
(its derivative is taken as 1), the reading that makes the pooling's
gradient the mean's.  Gate logits (gate_logits = 1) add the sigmoid's
derivative: dlogit = dgamma * s (1 - s).

Everything is computed in float64 from the stored inputs (bf16 bit
patterns or float32).  Pins (tests/test_oracle_backward.py): central finite
differences of this module's forward for every input and gate mode, this
forward against the C oracle, exact invariants (key gradients sum to zero,
value gradients sum to the gated upstream gradient), and torch autograd on
the branches that are plain attention (causal, banded, over block means).
"""
from __future__ import annotations

import numpy as np


def _widen(a, prob):
    """Stored tensor -> float64 (bf16 patterns are widened exactly)."""
    a = np.asarray(a)
    if prob["dtype"] == "bf16" and a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _round_store(x, prob):
    """Round float64 values to the storage type and back (nearest, ties to even)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if prob["dtype"] != "bf16":
        return f.astype(np.float64)
    u = f.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint32)
    return (r << np.uint32(16)).view(np.float32).astype(np.float64)


def _shapes(prob):
    B, T, L = prob["batch"], prob["q_len"], prob["kv_len"]
    G, hpg = prob["n_groups"], prob["heads_per_group"]
    bs = prob["block"]
    sb = prob.get("sel_block", 0) or bs
    return B, T, L, G, hpg, bs, sb


def _scale(prob):
    s = float(prob.get("scale", 0.0) or 0.0)
    return s if s > 0 else 1.0 / np.sqrt(prob["d_qk"])


def _branches(prob):
    return [b for b, key in enumerate(("use_cmp", "use_slc", "use_win")) if prob[key]]


def _gamma(prob, gates):
    """Branch weights [B, T, H, 3] as float64, and the sigmoid's derivative factor."""
    B, T, L, G, hpg, _, _ = _shapes(prob)
    H = G * hpg
    on = _branches(prob)
    if gates is None:
        if len(on) != 1:
            raise ValueError("gates may be omitted only when exactly one branch is on")
        gm = np.zeros((B, T, H, 3))
        gm[..., on[0]] = 1.0
        return gm, np.zeros((B, T, H, 3))
    x = _widen(gates, prob).reshape(B, T, H, 3)
    if prob["gate_logits"]:
        s = 1.0 / (1.0 + np.exp(-x))
        return s, s * (1.0 - s)
    return x, np.ones_like(x)


def pooled(prob, k, v, rounded=True):
    """Block means [B, nb, G, d] in float64 (rounded to storage when asked)."""
    B, T, L, G, hpg, bs, _ = _shapes(prob)
    nb = L // bs
    kk, vv = _widen(k, prob), _widen(v, prob)
    # explicit last dimensions: with no complete block the arrays are empty
    kc = kk[:, :nb * bs].reshape(B, nb, bs, G, kk.shape[-1]).mean(axis=2)
    vc = vv[:, :nb * bs].reshape(B, nb, bs, G, vv.shape[-1]).mean(axis=2)
    if rounded:
        kc, vc = _round_store(kc, prob), _round_store(vc, prob)
    return kc, vc


def key_sets(prob, idx, b, t, g):
    """Key sets of row (b, t) and group g: (summary ids, selected positions, window positions)."""
    B, T, L, G, hpg, bs, sb = _shapes(prob)
    p = L - T + t
    nb = L // bs
    ncmp = min((p + 1) // bs, nb)
    sel = []
    for j in np.asarray(idx)[b, t, g]:
        j = int(j)
        if j >= 0 and j * sb <= p:
            sel.extend(range(j * sb, min(j * sb + sb, p + 1)))
    sel = np.array(sorted(sel), dtype=np.int64)
    w = prob["window"]
    win = np.arange(max(0, p - w + 1), p + 1, dtype=np.int64) if w > 0 else np.zeros(0, np.int64)
    return np.arange(ncmp, dtype=np.int64), sel, win


def _softmax_rows(s):
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def forward(prob, q, k, v, gates, idx, rounded=True):
    """out [B, T, H, d_v] and the branch outputs O [3, B, T, H, d_v] (float64)
    on the GIVEN selection idx [B, T, G, top_k]."""
    B, T, L, G, hpg, bs, sb = _shapes(prob)
    H, dv = G * hpg, prob["d_v"]
    c = _scale(prob)
    qq, kk, vv = _widen(q, prob), _widen(k, prob), _widen(v, prob)
    kc, vc = pooled(prob, k, v, rounded)
    gam, _ = _gamma(prob, gates)
    O = np.zeros((3, B, T, H, dv))
    on = _branches(prob)
    for b in range(B):
        for t in range(T):
            for g in range(G):
                hs = slice(g * hpg, (g + 1) * hpg)
                qh = qq[b, t, hs]
                sets = key_sets(prob, idx, b, t, g)
                for br in on:
                    s_ids = sets[br]
                    if len(s_ids) == 0:
                        continue
                    K = kc[b, s_ids, g] if br == 0 else kk[b, s_ids, g]
                    V = vc[b, s_ids, g] if br == 0 else vv[b, s_ids, g]
                    P = _softmax_rows(c * qh @ K.T)
                    O[br, b, t, hs] = P @ V
    out = np.einsum("kbthd,bthk->bthd", O, gam)
    return out, O


def branch_lse(prob, q, k, v, idx, rounded=True, rows=None):
    """Per branch the natural log-sum-exp of the scaled logits over the row's
    key set, lse_b = log sum_s exp(scale * q_h . k_s) (the softmax's
    normaliser, so that P_b[s] = exp(scale * q_h . k_s - lse_b)): float64
    [3, B, T, H] (or [3, R, H] for the flat rows b * T + t listed in rows),
    -inf for an empty key set or a branch that is off.  With forward()'s O
    this is what a training forward keeps for the backward."""
    B, T, L, G, hpg, bs, sb = _shapes(prob)
    H = G * hpg
    c = _scale(prob)
    kc, _ = pooled(prob, k, v, rounded)
    flat = np.arange(B * T) if rows is None else np.asarray(rows, dtype=np.int64)
    lse = np.full((3, len(flat), H), -np.inf)
    for ri, r in enumerate(flat):
        b, t = int(r) // T, int(r) % T
        qr = _widen(q[b, t], prob)
        for g in range(G):
            hs = slice(g * hpg, (g + 1) * hpg)
            sets = key_sets(prob, idx, b, t, g)
            for br in _branches(prob):
                s_ids = sets[br]
                if len(s_ids) == 0:
                    continue
                K = kc[b, s_ids, g] if br == 0 else _widen(k[b, s_ids, g], prob)
                z = c * qr[hs] @ K.T                           # [hpg, n]
                m = z.max(axis=1)
                lse[br, ri, hs] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return lse if rows is not None else lse.reshape(3, B, T, H)


def _branch_grads(qh, doh, K, V, gb, c):
    """One (row, group, branch): the softmax over the key set and the
    gradient terms.  Returns (dq part [hpg, dqk], dK [n, dqk], dV [n, dv],
    dgamma [hpg])."""
    P = _softmax_rows(c * qh @ K.T)                # [hpg, n]
    O = P @ V                                      # [hpg, dv]
    dgb = np.sum(doh * O, axis=1)                  # [hpg]
    dP = gb * (doh @ V.T)                          # [hpg, n]
    dS = P * (dP - gb * dgb[:, None])
    return c * dS @ K, c * dS.T @ qh, P.T @ (gb * doh), dgb


def backward(prob, q, k, v, gates, idx, dout, rounded=True):
    """Gradients (dq [B,T,H,d_qk], dk [B,L,G,d_qk], dv [B,L,G,d_v],
    dgates [B,T,H,3] or None), float64, on the GIVEN selection idx."""
    B, T, L, G, hpg, bs, sb = _shapes(prob)
    H, dqk, dv = G * hpg, prob["d_qk"], prob["d_v"]
    nb = L // bs
    c = _scale(prob)
    qq, kk, vv = _widen(q, prob), _widen(k, prob), _widen(v, prob)
    do = _widen(dout, prob).reshape(B, T, H, dv)
    kc, vc = pooled(prob, k, v, rounded)
    gam, dsig = _gamma(prob, gates)
    on = _branches(prob)

    dq = np.zeros((B, T, H, dqk))
    dk = np.zeros((B, L, G, dqk))
    dvv = np.zeros((B, L, G, dv))
    dkc = np.zeros((B, nb, G, dqk))
    dvc = np.zeros((B, nb, G, dv))
    dgam = np.zeros((B, T, H, 3))
    for b in range(B):
        for t in range(T):
            for g in range(G):
                hs = slice(g * hpg, (g + 1) * hpg)
                sets = key_sets(prob, idx, b, t, g)
                for br in on:
                    s_ids = sets[br]
                    if len(s_ids) == 0:
                        continue
                    K = kc[b, s_ids, g] if br == 0 else kk[b, s_ids, g]
                    V = vc[b, s_ids, g] if br == 0 else vv[b, s_ids, g]
                    dqp, dK, dV, dgb = _branch_grads(qq[b, t, hs], do[b, t, hs], K, V,
                                                     gam[b, t, hs, br][:, None], c)
                    dgam[b, t, hs, br] = dgb
                    dq[b, t, hs] += dqp
                    if br == 0:
                        dkc[b, s_ids, g] += dK
                        dvc[b, s_ids, g] += dV
                    else:
                        np.add.at(dk, (b, s_ids, g), dK)
                        np.add.at(dvv, (b, s_ids, g), dV)
    # the mean's gradient: every token of block j gets dkc_j / bs
    dk[:, :nb * bs] += np.repeat(dkc, bs, axis=1) / bs
    dvv[:, :nb * bs] += np.repeat(dvc, bs, axis=1) / bs
    dgates = None
    if gates is not None:
        dgates = dgam * dsig
        for br in range(3):
            if br not in on:
                dgates[..., br] = 0.0
    return dq, dk, dvv, dgates


def _branch_magnitudes(qh, doh, K, V, gb, c):
    """The terms of _branch_grads taken in absolute value: for every entry of
    a gradient, the sum of |term| over the products that form it, with the
    softmax gradient dS bounded by P (|dP| + |gamma D|).  A rounding of
    relative size u in any factor of a term moves the entry by at most u
    times this magnitude."""
    P = _softmax_rows(c * qh @ K.T)
    O = P @ V
    D = np.sum(doh * O, axis=1)
    dP = gb * (doh @ V.T)
    AS = P * (np.abs(dP) + np.abs(gb * D[:, None]))
    return (c * AS @ np.abs(K), c * AS.T @ np.abs(qh), P.T @ np.abs(gb * doh),
            np.sum(np.abs(doh) * (P @ np.abs(V)), axis=1))


def backward_magnitudes(prob, q, k, v, gates, idx, dout, rounded=True):
    """Per-entry magnitudes of the gradients (the shapes of backward's):
    each entry's sum of absolute values of the terms that backward adds up,
    accumulated over the branches and key sets exactly as backward does.
    Tests bound the error of a bf16-operand, fp32-accumulated gradient
    entry by a small multiple of 2^-9 times its magnitude."""
    B, T, L, G, hpg, bs, sb = _shapes(prob)
    H, dqk, dv = G * hpg, prob["d_qk"], prob["d_v"]
    nb = L // bs
    c = _scale(prob)
    qq, kk, vv = _widen(q, prob), _widen(k, prob), _widen(v, prob)
    do = _widen(dout, prob).reshape(B, T, H, dv)
    kc, vc = pooled(prob, k, v, rounded)
    gam, dsig = _gamma(prob, gates)
    on = _branches(prob)
    aq = np.zeros((B, T, H, dqk))
    ak = np.zeros((B, L, G, dqk))
    av = np.zeros((B, L, G, dv))
    akc = np.zeros((B, nb, G, dqk))
    avc = np.zeros((B, nb, G, dv))
    ag = np.zeros((B, T, H, 3))
    for b in range(B):
        for t in range(T):
            for g in range(G):
                hs = slice(g * hpg, (g + 1) * hpg)
                sets = key_sets(prob, idx, b, t, g)
                for br in on:
                    s_ids = sets[br]
                    if len(s_ids) == 0:
                        continue
                    K = kc[b, s_ids, g] if br == 0 else kk[b, s_ids, g]
                    V = vc[b, s_ids, g] if br == 0 else vv[b, s_ids, g]
                    mq, mK, mV, mg = _branch_magnitudes(qq[b, t, hs], do[b, t, hs], K, V,
                                                        gam[b, t, hs, br][:, None], c)
                    ag[b, t, hs, br] = mg
                    aq[b, t, hs] += mq
                    if br == 0:
                        akc[b, s_ids, g] += mK
                        avc[b, s_ids, g] += mV
                    else:
                        np.add.at(ak, (b, s_ids, g), mK)
                        np.add.at(av, (b, s_ids, g), mV)
    ak[:, :nb * bs] += np.repeat(akc, bs, axis=1) / bs
    av[:, :nb * bs] += np.repeat(avc, bs, axis=1) / bs
    agates = None
    if gates is not None:
        agates = ag * np.abs(dsig)
        for br in range(3):
            if br not in on:
                agates[..., br] = 0.0
    return aq, ak, av, agates


def query_grads(prob, q, k, v, gates, idx, dout, rows, kc=None, vc=None):
    """dq [R, H, d_qk] and dgates [R, H, 3] (or None) of the listed flat rows
    b * T + t alone -- the query-side terms of backward(), which depend on
    nothing but the row's own key sets.  kc, vc: float64 summaries as pooled()
    returns them (computed when omitted)."""
    B, T, L, G, hpg, bs, sb = _shapes(prob)
    H, dqk, dv = G * hpg, prob["d_qk"], prob["d_v"]
    c = _scale(prob)
    if kc is None or vc is None:
        kc, vc = pooled(prob, k, v, True)
    on = _branches(prob)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((len(rows), H, dqk))
    dgam = np.zeros((len(rows), H, 3))
    dsig_rows = np.zeros((len(rows), H, 3))
    for ri, r in enumerate(rows):
        b, t = int(r) // T, int(r) % T
        qr = _widen(q[b, t], prob)
        dor = _widen(dout[b, t], prob).reshape(H, dv)
        if gates is None:
            gam = np.zeros((H, 3))
            gam[:, on[0]] = 1.0
        else:
            x = _widen(gates[b, t], prob).reshape(H, 3)
            if prob["gate_logits"]:
                gam = 1.0 / (1.0 + np.exp(-x))
                dsig_rows[ri] = gam * (1.0 - gam)
            else:
                gam = x
                dsig_rows[ri] = 1.0
        for g in range(G):
            hs = slice(g * hpg, (g + 1) * hpg)
            sets = key_sets(prob, idx, b, t, g)
            for br in on:
                s_ids = sets[br]
                if len(s_ids) == 0:
                    continue
                K = kc[b, s_ids, g] if br == 0 else _widen(k[b, s_ids, g], prob)
                V = vc[b, s_ids, g] if br == 0 else _widen(v[b, s_ids, g], prob)
                dqp, _, _, dgb = _branch_grads(qr[hs], dor[hs], K, V, gam[hs, br][:, None], c)
                dq[ri, hs] += dqp
                dgam[ri, hs, br] = dgb
    dgates = None
    if gates is not None:
        dgates = dgam * dsig_rows
        for br in range(3):
            if br not in on:
                dgates[..., br] = 0.0
    return dq, dgates
