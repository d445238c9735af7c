"""Helpers of the GPU parity tests: upload, run through the C ABI, compare
with the oracle under the selection tie-band rule."""
from __future__ import annotations

import numpy as np

from long_context_dynamic_amd import inputs, nsa

TIE_REL = 1e-4          # near-tie band: |I_j - s_r| <= 1e-4 * s_r
TOL = {"f32": 1e-4, "bf16": 2e-2}
# a branch's log-sum-exp: fp32 logits of exact bf16 products, fp32 sums
LSE_ATOL, LSE_RTOL = 1e-4, 1e-4


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 step at |x|: the most the final rounding to bf16 can move x."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def out_tolerance(prob: dict, ref: np.ndarray, out_f32: bool) -> np.ndarray:
    """The parity bound on the accumulated result, plus the final rounding
    when the output is stored as bf16."""
    tol = TOL[prob["dtype"]]
    if prob["dtype"] == "bf16" and not out_f32:
        return tol + half_ulp_bf16(ref)
    return np.full(ref.shape, tol)


def upload(x: dict, prob: dict) -> dict:
    return {k: nsa.to_device(a, prob) for k, a in x.items()}


def widen_out(t, prob) -> np.ndarray:
    a = nsa.to_host_bits(t)
    if a.dtype == np.uint16:
        return inputs.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def sample_rows(prob: dict, count: int, seed: int = 0) -> np.ndarray:
    """Flat rows b*T + t: the first and last token, tokens around block
    boundaries, and random ones."""
    T, B, bs = prob["q_len"], prob["batch"], prob["block"]
    rng = np.random.default_rng(seed)
    picks = {0, T - 1, min(bs - 1, T - 1), min(bs, T - 1), T // 2}
    while len(picks) < min(count, T):
        picks.add(int(rng.integers(0, T)))
    ts = np.array(sorted(picks), dtype=np.int64)
    bs_ = rng.integers(0, B, size=len(ts)) if B > 1 else np.zeros(len(ts), np.int64)
    return np.sort(bs_ * T + ts)


def sel_block(prob) -> int:
    """Tokens per selection block (the compression block unless decoupled)."""
    return prob.get("sel_block", 0) or prob["block"]


def forced_set(prob, p):
    F = set()
    if prob["force_first"]:
        F.add(0)
    if prob["force_current"]:
        F.add(p // sel_block(prob))
    return F


def check_selection(prob: dict, rows, got_idx: np.ndarray, ora_idx: np.ndarray, ora_imp: np.ndarray) -> int:
    """Compare a GPU selection [R,G,n] with the oracle's.  Outside the near-tie
    band the choice must be identical; inside it any choice with the right
    count passes.  Returns how many (row, group) pairs needed the band."""
    T, L, bs, n = prob["q_len"], prob["kv_len"], sel_block(prob), prob["top_k"]
    nb = L // bs
    band = 0
    for ri, r in enumerate(rows):
        t = int(r) % T
        p = L - T + t
        nvis = min((p + 1) // bs, nb)
        F = forced_set(prob, p)
        for g in range(got_idx.shape[1]):
            got, want = got_idx[ri, g], ora_idx[ri, g]
            if np.array_equal(got, want):
                continue
            chosen = [int(j) for j in got if j >= 0]
            k = len(chosen)
            assert chosen == sorted(set(chosen)), (r, g, got)
            assert np.all(got[k:] == -1), (r, g, got)
            C = [j for j in range(nvis) if j not in F]
            rr = min(n - len(F), len(C))
            assert F <= set(chosen) and len(chosen) == len(F) + rr, (r, g, got, want)
            assert set(chosen) <= (F | set(C)), (r, g, got)
            imp = ora_imp[ri, g]
            s_r = sorted((imp[j] for j in C), reverse=True)[rr - 1]
            lo, hi = s_r * (1 - TIE_REL), s_r * (1 + TIE_REL)
            for j in C:
                if imp[j] > hi:
                    assert j in chosen, (r, g, j, imp[j], s_r, got, want)
                if imp[j] < lo:
                    assert j not in chosen, (r, g, j, imp[j], s_r, got, want)
            band += 1
    return band


def gather_rows(t_out: np.ndarray, prob: dict, rows) -> np.ndarray:
    """[B, T, ...] -> [R, ...] for flat rows."""
    T = prob["q_len"]
    flat = t_out.reshape((prob["batch"] * T,) + t_out.shape[2:])
    return flat[np.asarray(rows)]
