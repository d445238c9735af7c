"""GPU parity of the learned block compression (nsa_compress_mlp) and the gate
projection (nsa_gate_proj) against the fp64 oracle (oracle/learned.py), with
seeded random-initialised weights.
  Gate projection, entry by entry: the oracle's bound for bf16 operands with
fp32 accumulation (gate_proj_error_bound: n 2^-24 times the sum of the
absolute products, times the sigmoid's slope of at most 1/4), half a bf16
step of the stored result and 1e-6 for the device's exponential -- about
one bf16 step at the gates' scale.
  Compression: the forward's output bound (2e-2 on the fp32-accumulated
value) plus half a bf16 step of the stored result; its hidden layer is
rounded to bf16 once, a relative 2^-9 on each hidden value whose effect on
an output is 2^-9 times the sum of |w2| |hidden| over the hidden width, well
inside that bound at these scales.
"""
import numpy as np
import pytest

from oracle import learned as LR
from long_context_dynamic_amd import inputs, nsa, workloads
from tests import gpu_util as U

TOL = 2e-2      # the compression's output bound
EXP_TOL = 1e-6  # the device exponential in the sigmoid

MLP_CASES = [
    ("8k shape T=L=1000 G2 dh192", dict(workloads.get("nsa_prefill_8k"), q_len=1000, kv_len=1000, n_groups=2), 192, True),
    ("d64 dh64 B2 ragged L=700 no bias", dict(workloads.get("nsa_prefill_8k"), batch=2, q_len=700, kv_len=700,
                                              n_groups=1, d_qk=64, d_v=64), 64, False),
    ("dh256 block 32", dict(workloads.get("nsa_prefill_8k"), q_len=640, kv_len=640, n_groups=1, block=32), 256, True),
]


def _dev(a, prob):
    return None if a is None else nsa.to_device(a, prob)


def _close(got, ref, bound, what):
    """got: the device result widened to float64; ref: the exact value (before
    any rounding); bound: the accumulation bound per entry."""
    tol = bound + U.half_ulp_bf16(np.maximum(np.abs(ref), np.abs(got))) + EXP_TOL
    err = np.abs(got - ref)
    print(f"[learned] {what}: max err {err.max():.3g} max |ref| {np.abs(ref).max():.3g} "
          f"worst err/tol {(err / tol).max():.3f}", flush=True)
    assert np.all(err <= tol), what


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(MLP_CASES)), ids=[c[0] for c in MLP_CASES])
def test_compress_mlp_matches_oracle(i):
    name, prob, dh, bias = MLP_CASES[i]
    print(f"[case] compress_mlp {name}", flush=True)
    x = inputs.generate(prob, want=("k", "v"))
    w = inputs.learned_weights(prob, dh, seed=i, bias=bias)
    rk, rv = LR.compress(prob, x["k"], x["v"], w["k"], w["v"], exact=True)
    bk = bv = TOL
    wk = {n: _dev(a, prob) for n, a in w["k"].items()}
    wv = {n: _dev(a, prob) for n, a in w["v"].items()}
    kc, vc = nsa.compress_mlp(prob, _dev(x["k"], prob), _dev(x["v"], prob), wk, wv)
    _close(U.widen_out(kc, prob), rk, bk, f"{name} k_cmp")
    _close(U.widen_out(vc, prob), rv, bv, f"{name} v_cmp")


GATE_CASES = [
    ("64 heads d_model 2560 T=1000 B2", dict(workloads.get("nsa_prefill_8k"), batch=2, q_len=1000, kv_len=1000), 2560, False),
    ("logits, 64 heads T=333", dict(workloads.get("nsa_prefill_8k"), q_len=333, kv_len=333), 2560, True),
    ("4 heads (12 outputs) d_model 96", dict(workloads.get("nsa_prefill_8k"), q_len=200, kv_len=200, n_groups=1,
                                             heads_per_group=4), 96, False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(GATE_CASES)), ids=[c[0] for c in GATE_CASES])
def test_gate_projection_matches_oracle(i):
    name, prob, dm, logits = GATE_CASES[i]
    print(f"[case] gate_proj {name}", flush=True)
    w = inputs.learned_weights(prob, 64, d_model=dm, seed=10 + i)
    ref = LR.gate_proj(w["x"], w["gate_w"], w["gate_b"], prob["dtype"], logits=logits)
    bound = LR.gate_proj_error_bound(w["x"], w["gate_w"], w["gate_b"], prob["dtype"], logits=logits)
    got = nsa.gate_proj(prob, _dev(w["x"], prob), _dev(w["gate_w"], prob), _dev(w["gate_b"], prob), logits=logits)
    _close(U.widen_out(got, prob), ref, bound, f"{name} gates")
