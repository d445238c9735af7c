"""nsa_forward_noalloc (GPU): the forward in the library's fixed device
scratch gives the same bits as nsa_forward with a caller workspace, on two
calls in a row with the second one smaller (the scratch then holds the first
call's leftovers), for the decoding path over a caller-held summary cache and
for a prefill path.  A call whose workspace exceeds the fixed scratch is
refused before anything is queued."""
import pytest
import torch

from long_context_dynamic_amd import inputs, nsa, workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _run_pair(prob, with_cmp):
    x = inputs.generate(prob)
    t = U.upload(x, prob)
    kc = vc = None
    if with_cmp:
        kc, vc = nsa.compress(prob, t["k"], t["v"])
    H = workloads.n_heads(prob)
    shape = (prob["batch"], prob["q_len"], H, prob["d_v"])
    want = nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"], k_cmp=kc, v_cmp=vc, out_f32=True)
    got = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    nsa.forward_noalloc(prob, t["q"], t["k"], t["v"], t["gates"], got, k_cmp=kc, v_cmp=vc, out_f32=True)
    torch.cuda.synchronize()
    return want, got


@pytest.mark.parametrize("name,big,small,with_cmp", [
    ("decode", dict(batch=64, kv_len=65536), dict(batch=5, kv_len=4096 + 17), True),
    ("decode, summaries in scratch", dict(batch=4, kv_len=20000), dict(batch=2, q_len=3, kv_len=3000), False),
    ("prefill", dict(q_len=300, kv_len=400), dict(q_len=120, kv_len=120), False),
])
def test_noalloc_matches_forward_on_two_calls(name, big, small, with_cmp):
    base = "nsa_decode_64x64k" if name.startswith("decode") else "nsa_prefill_8k"
    for over in (big, small):
        prob = workloads.get(base, **over)
        print(f"[noalloc] {name} {over} workspace {nsa.workspace_bytes(prob, with_cmp)} B", flush=True)
        assert nsa.workspace_bytes(prob, with_cmp) <= nsa.NOALLOC_SCRATCH_BYTES
        want, got = _run_pair(prob, with_cmp)
        assert torch.equal(want.view(torch.int32), got.view(torch.int32)), (name, over)


def test_noalloc_refuses_a_call_beyond_its_scratch():
    prob = workloads.get("nsa_prefill_8k")  # 8k prefill: a workspace of hundreds of MB
    assert nsa.workspace_bytes(prob) > nsa.NOALLOC_SCRATCH_BYTES
    x = {n: torch.empty(s, dtype=torch.bfloat16, device="cuda") for n, s in
         (("q", (1, 8192, 64, 192)), ("k", (1, 8192, 4, 192)), ("v", (1, 8192, 4, 128)), ("g", (1, 8192, 64, 3)))}
    out = torch.empty((1, 8192, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nsa.NsaError) as e:
        nsa.forward_noalloc(prob, x["q"], x["k"], x["v"], x["g"], out)
    assert e.value.code == 3  # NSA_ERR_WORKSPACE
