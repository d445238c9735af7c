"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs.  Pooling is bit-exact; selections match outside the near-tie band
(oracle's r-th / (r+1)-th importance gap under 1e-4 relative); outputs are
compared with oracle attention evaluated on the GPU's own selection, to
max |err| <= 2e-2 (bf16) or 1e-4 (fp32).

Cases: each named workload, once at a reduced size the oracle finishes in
seconds (several tiles and a ragged tail) checked on every row, and once at
its full size checked on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from long_context_dynamic_amd import inputs, nsa, workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

# (workload, overrides, rows to check: None = all rows, int = sample size)
CASES = [
    ("nsa_tiny_fp32", {}, None),
    ("nsa_tiny_fp32", dict(q_len=700, kv_len=1000, window=100), None),
    ("nsa_prefill_8k", dict(q_len=1000, kv_len=1000), None),
    ("nsa_prefill_8k", dict(q_len=333, kv_len=1100, gate_logits=1), None),
    ("nsa_prefill_8k", {}, 48),
    ("nsa_prefill_8k", dict(q_len=1000, kv_len=1300, block=32, sel_block=64), None),
    ("nsa_prefill_8k", dict(q_len=600, kv_len=600, block=16, sel_block=64, top_k=8, force_first=0), None),
    ("nsa_tiny_fp32", dict(q_len=500, kv_len=700, block=16, sel_block=48, top_k=5), None),
    ("nsa_prefill_64k", {}, 20),
    # a longer ragged prefill checked on every row, and two sequences of one launch
    ("nsa_prefill_8k", dict(q_len=4500, kv_len=4600), None),
    ("nsa_prefill_8k", dict(batch=2, q_len=2100, kv_len=2100, n_groups=2), None),
    # the largest summary count the matrix-core path takes (2048: the top-k's
    # 32-values-per-lane form), queries at the end of a 128k cache
    ("nsa_prefill_8k", dict(q_len=300, kv_len=131072), None),
    # degenerate shapes: no complete block (empty compressed branch, only the
    # partial current block to select), the shortest prefill above the
    # decoding path, a zero window, a window longer than the sequence
    ("nsa_prefill_8k", dict(q_len=40, kv_len=40), None),
    ("nsa_prefill_8k", dict(q_len=9, kv_len=70), None),
    ("nsa_prefill_8k", dict(q_len=200, kv_len=200, window=0), None),
    ("nsa_prefill_8k", dict(q_len=300, kv_len=300, window=1000), None),
    ("nsa_tiny_fp32", dict(q_len=5, kv_len=5), None),
    ("nsa_decode_64x64k", dict(batch=3, kv_len=40), None),
    ("moba_32k", dict(q_len=300, kv_len=300), None),
    ("moba_32k", dict(q_len=3, kv_len=1000), None),
    ("moba_32k", dict(q_len=2600, kv_len=2600), 160),
    ("moba_32k", dict(q_len=700, kv_len=3000), None),
    ("moba_32k", dict(batch=2, q_len=1000, kv_len=12000, block=64, top_k=8, d_qk=64, d_v=64, force_first=1), None),
    ("moba_32k", dict(q_len=1200, kv_len=40000, block=64, top_k=8, d_qk=64, d_v=64), None),
    ("moba_32k", dict(q_len=900, kv_len=5000, block=128, top_k=2, force_first=1, force_current=0), None),
    ("moba_32k", {}, 24),
    ("moba_128k", {}, 16),
    ("moba_1m", {}, 8),
    ("nsa_decode_64x64k", dict(batch=6, kv_len=4096 + 17), None),
    ("nsa_decode_64x64k", dict(batch=4, kv_len=4096 + 40, block=32, sel_block=64), None),
    # more than 1024 summaries (the step kernel keeps its logits in global memory), other head dims
    ("nsa_decode_64x64k", dict(batch=2, kv_len=40000, block=32, sel_block=64), None),
    ("nsa_decode_64x64k", dict(batch=3, kv_len=9000, d_qk=128, d_v=64, top_k=12, window=256), None),
    # several new tokens per sequence in one decoding launch: every row has
    # its own position, visible summaries, current block and window
    ("nsa_decode_64x64k", dict(batch=2, q_len=5, kv_len=4096 + 17), None),
    ("nsa_decode_64x64k", dict(batch=3, q_len=3, kv_len=40), None),
    ("nsa_decode_64x64k", dict(batch=2, q_len=8, kv_len=3000 + 63, block=32, sel_block=64), None),
]


def _ids():
    return [f"{n}-{'-'.join(f'{k}{v}' for k, v in o.items()) or 'full'}" for n, o, _ in CASES]


_cache = {}


def _case(i):
    """Inputs, device tensors and the oracle's selection for CASES[i] (cached per case)."""
    if i in _cache:
        return _cache[i]
    _cache.clear()
    torch.cuda.empty_cache()
    name, over, nrows = CASES[i]
    prob = workloads.get(name, **over)
    print(f"[case] {name} {over}", flush=True)
    x = inputs.generate(prob)
    t = U.upload(x, prob)
    rows = (np.arange(prob["batch"] * prob["q_len"]) if nrows is None
            else U.sample_rows(prob, nrows, seed=i))
    kc, vc = oracle.pool(prob, x["k"], x["v"])
    idx, imp, ocmp = oracle.select(prob, x["q"], kc, vc, rows=rows, want_cmp=bool(prob["use_cmp"]))
    _cache[i] = (prob, x, t, rows, (kc, vc, idx, imp, ocmp))
    return _cache[i]


@pytest.mark.parametrize("i", range(len(CASES)), ids=_ids())
def test_compress_is_bit_exact(i):
    prob, x, t, rows, (kc, vc, *_) = _case(i)
    gkc, gvc = nsa.compress(prob, t["k"], t["v"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nsa.to_host_bits(gkc), kc)
    np.testing.assert_array_equal(nsa.to_host_bits(gvc), vc)


@pytest.mark.parametrize("i", range(len(CASES)), ids=_ids())
def test_select_topk(i):
    prob, x, t, rows, (kc, vc, idx, imp, _) = _case(i)
    gkc = nsa.to_device(kc, prob)
    gidx, gscore = nsa.select_topk(prob, t["q"], gkc)
    torch.cuda.synchronize()
    got = U.gather_rows(gidx.cpu().numpy(), prob, rows)
    band = U.check_selection(prob, rows, got, idx, imp)
    print(f"rows={len(rows)} groups={prob['n_groups']} tie-band pairs={band}")
    # scores: importance of each chosen block, +inf forced, -inf padding
    sc = U.gather_rows(gscore.cpu().numpy(), prob, rows)
    T, bs = prob["q_len"], prob["block"]
    for ri, r in enumerate(rows):
        p = prob["kv_len"] - T + int(r) % T
        F = U.forced_set(prob, p)
        for g in range(prob["n_groups"]):
            for slot, j in enumerate(got[ri, g]):
                s = sc[ri, g, slot]
                if j < 0:
                    assert s == -np.inf
                elif j in F:
                    assert s == np.inf
                else:
                    assert abs(s - imp[ri, g, j]) <= 1e-5 + 1e-4 * imp[ri, g, j], (r, g, j, s, imp[ri, g, j])


@pytest.mark.parametrize("i", range(len(CASES)), ids=_ids())
def test_sparse_attn_on_given_selection(i):
    prob, x, t, rows, (kc, vc, idx, imp, _) = _case(i)
    # run on the oracle's own selection, every row filled in
    full_idx = np.full((prob["batch"] * prob["q_len"], prob["n_groups"], prob["top_k"]), -1, np.int32)
    full_idx[rows] = idx
    sel_rows = rows
    gidx = torch.from_numpy(full_idx.reshape(prob["batch"], prob["q_len"], prob["n_groups"], -1)).cuda()
    out, lse = nsa.sparse_attn(prob, t["q"], t["k"], t["v"], gidx, out_f32=True)
    torch.cuda.synchronize()
    oprob = dict(prob, use_cmp=0, use_slc=1, use_win=0)
    _, want, _ = oracle.attend(oprob, x["q"], x["k"], x["v"], None, idx, None, rows=sel_rows)
    got = U.gather_rows(out.cpu().numpy().astype(np.float64), prob, sel_rows)
    err = np.abs(got - want).max()
    print(f"max |o_slc - oracle| = {err:.3e}")
    assert err <= U.TOL[prob["dtype"]]
    # the branch's log-sum-exp (natural log, -inf for an empty key set)
    want_lse = oracle.selected_lse(prob, x["q"], x["k"], idx, rows=sel_rows)
    got_lse = U.gather_rows(lse.cpu().numpy().astype(np.float64), prob, sel_rows)
    empty = np.isneginf(want_lse)
    assert np.array_equal(np.isneginf(got_lse), empty)
    lerr = np.abs(got_lse[~empty] - want_lse[~empty])
    print(f"max |lse - oracle| = {lerr.max() if lerr.size else 0.0:.3e}")
    assert np.all(lerr <= U.LSE_ATOL + U.LSE_RTOL * np.abs(want_lse[~empty]))


@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("i", range(len(CASES)), ids=_ids())
def test_forward(i, out_f32):
    prob, x, t, rows, (kc, vc, idx, imp, ocmp) = _case(i)
    gkc = nsa.to_device(kc, prob)
    gidx, _ = nsa.select_topk(prob, t["q"], gkc, want_score=False)
    gates = t["gates"] if (prob["use_cmp"] + prob["use_slc"] + prob["use_win"]) > 1 else None
    out = torch.full((prob["batch"], prob["q_len"], workloads.n_heads(prob), prob["d_v"]), float("nan"),
                     dtype=torch.float32 if out_f32 else nsa.torch_dtype(prob), device="cuda")
    nsa.forward(prob, t["q"], t["k"], t["v"], gates, out=out, out_f32=out_f32)
    torch.cuda.synchronize()
    gsel = U.gather_rows(gidx.cpu().numpy(), prob, rows)
    U.check_selection(prob, rows, gsel, idx, imp)
    want, _, _ = oracle.attend(prob, x["q"], x["k"], x["v"], x["gates"] if gates is not None else None,
                               gsel, ocmp if prob["use_cmp"] else None, rows=rows)
    got = U.gather_rows(U.widen_out(out, prob), prob, rows)
    assert np.all(np.isfinite(got))
    err = np.abs(got - want)
    tol = U.out_tolerance(prob, want, out_f32)
    print(f"max |out - oracle| = {err.max():.3e} (worst err - tol {np.max(err - tol):.3e})")
    assert np.all(err <= tol)
    assert not torch.isnan(out).any().item()  # every element written


def test_forward_is_deterministic():
    prob = workloads.get("nsa_prefill_8k", q_len=4200, kv_len=4200)
    x = inputs.generate(prob)
    t = U.upload(x, prob)
    a = nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"])
    b = nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_with_given_summary_cache_matches_internal():
    prob = workloads.get("nsa_decode_64x64k", batch=3, kv_len=3000)
    x = inputs.generate(prob)
    t = U.upload(x, prob)
    kc, vc = nsa.compress(prob, t["k"], t["v"])
    a = nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"], k_cmp=kc, v_cmp=vc, out_f32=True)
    b = nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"], out_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_all_blocks_selected_equals_dense_causal_attention():
    # top-k covering every block turns the selected branch into full attention
    prob = workloads.get("nsa_prefill_8k", q_len=640, kv_len=640, top_k=16, use_cmp=0, use_win=0)
    x = inputs.generate(prob)
    t = U.upload(x, prob)
    out = nsa.forward(prob, t["q"], t["k"], t["v"], None, out_f32=True)
    torch.cuda.synchronize()
    q = inputs.bf16_bits_to_f32(x["q"][0]).astype(np.float64)
    k = inputs.bf16_bits_to_f32(x["k"][0]).astype(np.float64)
    v = inputs.bf16_bits_to_f32(x["v"][0]).astype(np.float64)
    got = out.cpu().numpy()[0]
    T = 640
    mask = np.tril(np.ones((T, T), bool))
    for h in (0, 17, 63):
        g = h // 16
        s = q[:, h] @ k[:, g].T / np.sqrt(192)
        s[~mask] = -np.inf
        pr = np.exp(s - s.max(1, keepdims=True))
        pr /= pr.sum(1, keepdims=True)
        assert np.abs(got[:, h] - pr @ v[:, g]).max() <= 2e-2


def test_decode_full_size_sampled_sequences():
    """64 sequences x 65536-token caches (the batched-decode workload, same
    launch as the benchmark); 4 sequences checked against the oracle."""
    prob = workloads.get("nsa_decode_64x64k")
    B, L, G, H = prob["batch"], prob["kv_len"], prob["n_groups"], workloads.n_heads(prob)
    dq, dv = prob["d_qk"], prob["d_v"]
    dev = {"q": torch.empty((B, 1, H, dq), dtype=torch.bfloat16, device="cuda"),
           "k": torch.empty((B, L, G, dq), dtype=torch.bfloat16, device="cuda"),
           "v": torch.empty((B, L, G, dv), dtype=torch.bfloat16, device="cuda"),
           "gates": torch.empty((B, 1, H, 3), dtype=torch.bfloat16, device="cuda")}
    check = [0, 21, 42, 63]
    host = {}
    for b in range(B):
        xs = inputs.generate_sequence(prob, b)
        for name, arr in xs.items():
            dev[name][b:b + 1].copy_(nsa.to_device(arr, prob))
        if b in check:
            host[b] = xs
    kc, vc = nsa.compress(prob, dev["k"], dev["v"])
    out = nsa.forward(prob, dev["q"], dev["k"], dev["v"], dev["gates"], k_cmp=kc, v_cmp=vc)
    gidx, _ = nsa.select_topk(prob, dev["q"], kc, want_score=False)
    torch.cuda.synchronize()
    one = dict(prob, batch=1)
    for b in check:
        xs = host[b]
        okc, ovc = oracle.pool(one, xs["k"], xs["v"])
        np.testing.assert_array_equal(nsa.to_host_bits(kc[b:b + 1]), okc)
        idx, imp, ocmp = oracle.select(one, xs["q"], okc, ovc)
        got_idx = gidx[b:b + 1].cpu().numpy().reshape(1, G, -1)
        band = U.check_selection(one, [0], got_idx, idx, imp)
        want, _, _ = oracle.attend(one, xs["q"], xs["k"], xs["v"], xs["gates"], got_idx, ocmp)
        got = U.widen_out(out[b:b + 1], prob).reshape(1, H, dv)
        err = np.abs(got - want)
        print(f"seq {b}: max err {err.max():.3e}, tie-band groups {band}")
        assert np.all(err <= U.out_tolerance(prob, want, False))


def test_moba_forward_applies_the_gate():
    # one branch with gates given: the output is the gate times that branch
    prob = workloads.get("moba_32k", q_len=640, kv_len=1600, gate_logits=1)
    x = inputs.generate(prob)
    t = U.upload(x, prob)
    out = nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"], out_f32=True)
    gidx, _ = nsa.select_topk(prob, t["q"], nsa.compress(prob, t["k"], t["v"])[0], want_score=False)
    torch.cuda.synchronize()
    rows = np.arange(prob["q_len"])
    kc, vc = oracle.pool(prob, x["k"], x["v"])
    idx, imp, _ = oracle.select(prob, x["q"], kc, vc, rows=rows)
    gsel = U.gather_rows(gidx.cpu().numpy(), prob, rows)
    U.check_selection(prob, rows, gsel, idx, imp)
    want, _, _ = oracle.attend(prob, x["q"], x["k"], x["v"], x["gates"], gsel, None, rows=rows)
    got = U.gather_rows(U.widen_out(out, prob), prob, rows)
    assert np.abs(got - want).max() <= U.TOL[prob["dtype"]]


@pytest.mark.parametrize("name,over", [("nsa_decode_64x64k", dict(batch=2, kv_len=5000)),
                                       ("moba_32k", dict(q_len=3000, kv_len=3000))])
def test_compress_of_a_growing_cache_keeps_its_summaries(name, over):
    """A decode cache grows token by token: pooling a prefix of it gives the
    same bits as the first summaries of pooling the whole of it (a summary
    depends only on its own block), so summaries can be made once per
    completed block and kept."""
    prob = workloads.get(name, **over)
    x = inputs.generate(prob)
    t = U.upload(x, prob)
    kc, vc = nsa.compress(prob, t["k"], t["v"])
    bs = prob["block"]
    for L in (bs - 1, bs, 3 * bs + 5, prob["kv_len"] - 1):
        short = dict(prob, kv_len=L, q_len=min(prob["q_len"], L))
        kc2, vc2 = nsa.compress(short, t["k"][:, :L].contiguous(), t["v"][:, :L].contiguous())
        torch.cuda.synchronize()
        nb = L // bs
        assert torch.equal(kc2.view(torch.int16), kc[:, :nb].view(torch.int16)), L
        assert torch.equal(vc2.view(torch.int16), vc[:, :nb].view(torch.int16)), L


@pytest.mark.parametrize("name,over", [("nsa_prefill_8k", dict(q_len=700, kv_len=1100)),
                                       ("nsa_decode_64x64k", dict(batch=3, kv_len=5000))])
def test_exact_ties_pick_the_lower_block_ids(name, over):
    """Every block's keys repeated from one of the first four blocks: blocks
    with the same keys have the same summary, so their importances are
    exactly equal in the oracle and on the GPU, and the selection must take
    the lower block ids among them (reading R6).  The near-tie band would
    accept either order, so each (row, group) whose four distinct
    importances are more than 1e-4 apart is compared with the oracle's
    selection exactly."""
    prob = workloads.get(name, **over)
    x = inputs.generate(prob)
    bs, nb = prob["block"], prob["kv_len"] // prob["block"]
    for j in range(4, nb):
        x["k"][:, j * bs:(j + 1) * bs] = x["k"][:, (j % 4) * bs:(j % 4 + 1) * bs]
    t = U.upload(x, prob)
    rows = np.arange(prob["batch"] * prob["q_len"])
    kc, vc = oracle.pool(prob, x["k"], x["v"])
    idx, imp, _ = oracle.select(prob, x["q"], kc, vc, rows=rows, want_cmp=False)
    gidx, _ = nsa.select_topk(prob, t["q"], nsa.to_device(kc, prob))
    got = U.gather_rows(gidx.cpu().numpy(), prob, rows)
    exact = 0
    for ri in range(len(rows)):
        for g in range(prob["n_groups"]):
            v = np.sort(imp[ri, g][:4][np.isfinite(imp[ri, g][:4])])
            if len(v) > 1 and np.min(np.diff(v) / v[1:]) <= U.TIE_REL:
                continue
            np.testing.assert_array_equal(got[ri, g], idx[ri, g], err_msg=f"row {rows[ri]} group {g}")
            exact += 1
    U.check_selection(prob, rows, got, idx, imp)
    print(f"{exact} of {len(rows) * prob['n_groups']} (row, group) pairs compared exactly")
    assert exact >= 0.9 * len(rows) * prob["n_groups"]
