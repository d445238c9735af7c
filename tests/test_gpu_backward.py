"""GPU parity of nsa_backward against the fp64 backward oracle
(oracle/backward.py), on the oracle's own selection.

Tolerance (bf16 operands, fp32 accumulation): every operand of the matrix
products is rounded to bf16 once (q, k, v, dout as stored; P, gamma*P and
dS rounded when packed), a relative error of at most 2^-9 per factor, and
the sums run in fp32.  The error of a gradient entry is then a sum of
independently rounded terms, so it is bounded entry by entry by a small
multiple of 2^-9 times the entry's magnitude -- the sum of the absolute
values of its terms, which the oracle computes alongside the gradients
(ELEM_K).  Per tensor, the error also stays below 1% of the tensor's largest
entry (GRAD_REL), and an RMS bound (GRAD_RMS) catches a systematic error of
any one term.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as BW
from long_context_dynamic_amd import inputs, nsa, workloads
from tests import gpu_util as U

GRAD_REL = 1e-2   # max |gpu - ref| <= GRAD_REL * max |ref|  (per tensor)
GRAD_RMS = 4e-3   # rms(gpu - ref) <= GRAD_RMS * rms(ref)
# element-wise: |gpu - ref| <= ELEM_K * 2^-9 * magnitude + ELEM_FLOOR * max |ref|,
# the magnitude being the entry's sum of |terms| (oracle backward_magnitudes).
# Each term carries at most a few bf16 roundings of relative 2^-9 (P or dS
# packed for a product, the dS factor's own inputs), fp32 sums add far less;
# ELEM_K = 8 covers them with room.  The floor only admits fp32 noise on
# entries whose terms cancel exactly.
ELEM_K = 8.0
ELEM_FLOOR = 1e-6

BASE = dict(workloads.get("nsa_prefill_8k"), q_len=700, kv_len=700, n_groups=2, top_k=8, window=100)

CASES = [
    ("ragged T=L=700 G2 top8 w100", dict(BASE)),
    ("logits, queries at the end T=300 L=1000", dict(BASE, q_len=300, kv_len=1000, top_k=6, window=200,
                                                      gate_logits=1)),
    ("d64 slc only T=L=520", dict(BASE, q_len=520, kv_len=520, n_groups=1, d_qk=64, d_v=64, use_cmp=0,
                                   use_win=0, top_k=4)),
    ("cmp only T=L=600", dict(BASE, q_len=600, kv_len=600, n_groups=1, use_slc=0, use_win=0)),
    ("win only T=L=333 w64", dict(BASE, q_len=333, kv_len=333, n_groups=1, use_cmp=0, use_slc=0, window=64)),
    ("dq128 dv64 no forced blocks", dict(BASE, q_len=640, kv_len=640, d_qk=128, d_v=64, force_first=0,
                                          force_current=0, top_k=5)),
    ("long T=L=4200 G1 top16 w512", dict(BASE, q_len=4200, kv_len=4200, n_groups=1, top_k=16, window=512)),
    ("two sequences T=300 L=450 G2 logits", dict(BASE, batch=2, q_len=300, kv_len=450, top_k=6, gate_logits=1)),
    ("no complete block T=L=40", dict(BASE, q_len=40, kv_len=40)),
]


def _ids():
    return [c[0] for c in CASES]


def _inputs(prob):
    x = inputs.generate(prob, want=("q", "k", "v", "gates", "dout"))
    if not (prob["use_cmp"] + prob["use_slc"] + prob["use_win"] > 1):
        x["gates"] = None
    return x


def _oracle_idx(prob, x):
    kc, vc = oracle.pool(prob, x["k"], x["v"])
    idx, _, _ = oracle.select(prob, x["q"], kc, vc, want_imp=False, want_cmp=False)
    return idx.reshape(prob["batch"], prob["q_len"], prob["n_groups"], prob["top_k"])


def _run_gpu(prob, x, idx):
    d = {k: nsa.to_device(a, prob) for k, a in x.items() if a is not None}
    import torch
    idx_t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    dq, dk, dv, dg = nsa.backward(prob, d["q"], d["k"], d["v"], d.get("gates"), idx_t, d["dout"])
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv, dg)]


def _compare(name, got, ref, mag=None):
    err = np.abs(got - ref)
    scale = max(np.abs(ref).max(), 1e-30)
    rms_ref = max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    rel, rms = err.max() / scale, np.sqrt(np.mean(err ** 2)) / rms_ref
    msg = f"[bwd] {name}: max|ref| {scale:.3g} max err {err.max():.3g} (rel {rel:.2e}) rms rel {rms:.2e}"
    if mag is not None:
        bound = ELEM_K * 2.0 ** -9 * mag + ELEM_FLOOR * scale
        worst = float((err / bound).max())
        msg += f" worst err/element bound {worst:.3f}"
    print(msg, flush=True)
    assert rel <= GRAD_REL, (name, rel)
    assert rms <= GRAD_RMS, (name, rms)
    if mag is not None:
        bad = np.argwhere(err > bound)
        assert len(bad) == 0, (name, len(bad), tuple(bad[0]), float(err[tuple(bad[0])]), float(bound[tuple(bad[0])]))


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(CASES)), ids=_ids())
def test_backward_matches_oracle(i):
    name, prob = CASES[i]
    print(f"[case] backward {name}", flush=True)
    x = _inputs(prob)
    idx = _oracle_idx(prob, x)
    got = _run_gpu(prob, x, idx)
    ref = BW.backward(prob, x["q"], x["k"], x["v"], x["gates"], idx, x["dout"])
    mags = BW.backward_magnitudes(prob, x["q"], x["k"], x["v"], x["gates"], idx, x["dout"])
    for nm, g, r, a in zip(("dq", "dk", "dv", "dgates"), got, ref, mags):
        if r is None:
            assert g is None
            continue
        _compare(f"{name} {nm}", g, r, a)


@pytest.mark.gpu
def test_backward_is_deterministic():
    name, prob = CASES[0]
    x = _inputs(prob)
    idx = _oracle_idx(prob, x)
    a = _run_gpu(prob, x, idx)
    b = _run_gpu(prob, x, idx)
    for ga, gb in zip(a, b):
        assert np.array_equal(ga, gb)


def _random_selection(prob, seed=0):
    """A valid selection for every row: the forced blocks, then distinct
    random complete blocks before the query (the structure a top-k choice
    has; the backward takes any such selection)."""
    rng = np.random.default_rng(seed)
    B, T, L, G, n = prob["batch"], prob["q_len"], prob["kv_len"], prob["n_groups"], prob["top_k"]
    idx = np.full((B, T, G, n), -1, dtype=np.int32)
    for t in range(T):
        p = L - T + t
        nvis = min((p + 1) // 64, L // 64)
        forced = sorted({0, p // 64})
        cand = np.setdiff1d(np.arange(nvis), forced)
        for b in range(B):
            for g in range(G):
                pick = rng.choice(cand, size=min(n - len(forced), len(cand)), replace=False) if len(cand) else []
                row = np.sort(np.concatenate([np.array(forced), np.asarray(pick, dtype=np.int64)]))
                idx[b, t, g, :len(row)] = row
    return idx


@pytest.mark.gpu
def test_backward_full_size_64k_sampled_rows_and_sums():
    """The 64k workload as bench.py times it: dq and dgates of sampled rows
    against the oracle's query-side terms, and two sums over every key that
    hold at any size (key gradients sum to zero per group; value gradients
    sum to the gated upstream gradient of all rows)."""
    import torch
    prob = workloads.get("nsa_prefill_64k")
    print("[case] backward full size nsa_prefill_64k", flush=True)
    x = inputs.generate(prob, want=("q", "k", "v", "gates", "dout"))
    idx = _random_selection(prob, seed=1)
    d = {k: nsa.to_device(a, prob) for k, a in x.items()}
    idx_t = torch.from_numpy(idx).cuda()
    dq, dk, dv, dg = nsa.backward(prob, d["q"], d["k"], d["v"], d["gates"], idx_t, d["dout"])
    torch.cuda.synchronize()
    rows = U.sample_rows(prob, 24, seed=3)
    ref_dq, ref_dg = BW.query_grads(prob, x["q"], x["k"], x["v"], x["gates"], idx, x["dout"], rows)
    got_dq = dq.reshape(-1, *dq.shape[2:])[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    got_dg = dg.reshape(-1, *dg.shape[2:])[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    _compare("64k sampled dq", got_dq, ref_dq)
    _compare("64k sampled dgates", got_dg, ref_dg)
    # sums over all keys, per group (fp64 on the device)
    G, hpg, T, L = prob["n_groups"], prob["heads_per_group"], prob["q_len"], prob["kv_len"]
    sk = dk.double().sum(dim=1)[0].cpu().numpy()              # [G, dqk]
    ak = dk.double().abs().sum(dim=1)[0].cpu().numpy()
    sv = dv.double().sum(dim=1)[0].cpu().numpy()              # [G, dv]
    gam = inputs.bf16_bits_to_f32(x["gates"][0]).astype(np.float64)  # [T, H, 3]
    pos = L - T + np.arange(T)
    w = gam[:, :, 1] + gam[:, :, 2] + gam[:, :, 0] * (pos >= 63)[:, None]  # rows whose sets are not empty
    want = np.zeros_like(sv)
    for g in range(G):
        for c0 in range(0, T, 8192):
            dob = inputs.bf16_bits_to_f32(x["dout"][0, c0:c0 + 8192, g * hpg:(g + 1) * hpg]).astype(np.float64)
            want[g] += np.einsum("th,thd->d", w[c0:c0 + 8192, g * hpg:(g + 1) * hpg], dob)
    rel_k = np.abs(sk).max() / ak.max()
    rel_v = np.abs(sv - want).max() / np.abs(want).max()
    print(f"[bwd] 64k sum dk {rel_k:.2e} of sum |dk|; sum dv off by {rel_v:.2e}", flush=True)
    assert rel_k <= 1e-4
    assert rel_v <= 1e-3


@pytest.mark.gpu
def test_backward_without_dgates_output_matches():
    """dgates is optional: leaving it out changes nothing else."""
    name, prob = CASES[1]
    x = _inputs(prob)
    idx = _oracle_idx(prob, x)
    import torch
    d = {k: nsa.to_device(a, prob) for k, a in x.items() if a is not None}
    idx_t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    full = nsa.backward(prob, d["q"], d["k"], d["v"], d["gates"], idx_t, d["dout"])
    part = nsa.backward(prob, d["q"], d["k"], d["v"], d["gates"], idx_t, d["dout"], want_dgates=False)
    torch.cuda.synchronize()
    assert part[3] is None
    for a_, b_ in zip(full[:3], part[:3]):
        assert torch.equal(a_, b_)
