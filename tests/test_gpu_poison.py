"""Poisoned buffers (GPU): every output and scratch buffer a call is handed is
filled first with 0x00 bytes and then, in a second call, with 0xFF bytes
(a NaN in fp32 and bf16, -1 in int32).  Both calls must give bit-identical,
finite results: a kernel that reads an output before writing it, leaves part
of it unwritten, or reads workspace that no earlier kernel of the same call
wrote would pass the zero fill and fail the poisoned one.  Covered: the
forward on every path (generic fp32, matrix-core prefill with ragged and
decoupled blocks, the MoBA special case, the decode step), the separate
select_topk and sparse_attn calls, the training forward and the backward,
recomputing and from saved statistics."""
import pytest
import torch

from long_context_dynamic_amd import inputs, nsa, workloads
from tests import gpu_util as U
from tests.test_gpu_backward import CASES as BW_CASES

pytestmark = pytest.mark.gpu

FWD_CASES = [
    ("tiny fp32 ragged", workloads.get("nsa_tiny_fp32", q_len=700, kv_len=1000, window=100)),
    ("prefill bf16 ragged", workloads.get("nsa_prefill_8k", q_len=1000, kv_len=1300)),
    ("prefill two sequences", workloads.get("nsa_prefill_8k", batch=2, q_len=700, kv_len=800, n_groups=2)),
    ("prefill decoupled blocks", workloads.get("nsa_prefill_8k", q_len=600, kv_len=700, block=32, sel_block=64)),
    ("moba ragged", workloads.get("moba_32k", q_len=700, kv_len=3000)),
    ("decode ragged", workloads.get("nsa_decode_64x64k", batch=5, kv_len=4096 + 17)),
    ("decode long", workloads.get("nsa_decode_64x64k", batch=2, kv_len=40000, block=32, sel_block=64)),
    ("decode five tokens", workloads.get("nsa_decode_64x64k", batch=2, q_len=5, kv_len=4096 + 17)),
]


def _fill(ts, byte):
    for t in ts:
        if t is not None:
            t.view(torch.uint8).fill_(byte)


def _bits(t):
    return t.contiguous().view(torch.uint8).clone()


def _finite(t):
    return bool(torch.isfinite(t.float()).all().item()) if t.is_floating_point() else True


def _gates(prob, t):
    return t["gates"] if prob["use_cmp"] + prob["use_slc"] + prob["use_win"] > 1 else None


@pytest.mark.parametrize("name,prob", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_with_poisoned_output_and_workspace(name, prob):
    print(f"[case] poisoned forward {name}", flush=True)
    t = U.upload(inputs.generate(prob), prob)
    s = nsa._shapes(prob)
    out = torch.empty(s["out"], dtype=nsa.torch_dtype(prob), device="cuda")
    ws = nsa.alloc_workspace(prob)
    res = []
    for byte in (0x00, 0xFF):
        _fill((out, ws), byte)
        nsa.forward(prob, t["q"], t["k"], t["v"], _gates(prob, t), out=out, workspace=ws)
        torch.cuda.synchronize()
        assert _finite(out), byte
        res.append(_bits(out))
    assert torch.equal(res[0], res[1])


@pytest.mark.parametrize("name,prob", FWD_CASES[:4], ids=[c[0] for c in FWD_CASES[:4]])
def test_select_and_sparse_attention_with_poisoned_outputs(name, prob):
    print(f"[case] poisoned select_topk + sparse_attn {name}", flush=True)
    t = U.upload(inputs.generate(prob), prob)
    s = nsa._shapes(prob)
    kc, vc = nsa.compress(prob, t["k"], t["v"])
    idx = torch.empty(s["idx"], dtype=torch.int32, device="cuda")
    score = torch.empty(s["idx"], dtype=torch.float32, device="cuda")
    out = torch.empty(s["out"], dtype=nsa.torch_dtype(prob), device="cuda")
    lse = torch.empty(s["lse"], dtype=torch.float32, device="cuda")
    ws = nsa.alloc_workspace(prob, True)
    res = []
    for byte in (0x00, 0xFF):
        _fill((idx, score, out, lse, ws), byte)
        nsa.select_topk(prob, t["q"], kc, idx=idx, score=score, workspace=ws)
        nsa.sparse_attn(prob, t["q"], t["k"], t["v"], idx, out=out, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        assert _finite(out), byte
        assert not torch.isnan(score).any().item() and not torch.isnan(lse).any().item(), byte
        res.append([_bits(x) for x in (idx, score, out, lse)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("i", [0, 1, 4, 7], ids=[BW_CASES[i][0] for i in (0, 1, 4, 7)])
def test_training_forward_and_backward_with_poisoned_buffers(i):
    name, prob = BW_CASES[i]
    print(f"[case] poisoned training forward + backward {name}", flush=True)
    x = inputs.generate(prob, want=("q", "k", "v", "gates", "dout"))
    t = U.upload(x, prob)
    gates = _gates(prob, t)
    s = nsa._shapes(prob)
    f32 = torch.float32
    out = torch.empty(s["out"], dtype=nsa.torch_dtype(prob), device="cuda")
    idx = torch.empty(s["idx"], dtype=torch.int32, device="cuda")
    saved = torch.empty(max(nsa.train_saved_bytes(prob), 256), dtype=torch.uint8, device="cuda")
    fws = nsa.alloc_workspace(prob)
    grads = [torch.empty(s[k], dtype=f32, device="cuda") for k in ("q", "k", "v")]
    grads.append(torch.empty(s["gates"], dtype=f32, device="cuda") if gates is not None else None)
    bws = torch.empty(max(nsa.backward_workspace_bytes(prob), 256), dtype=torch.uint8, device="cuda")
    res = []
    for byte in (0x00, 0xFF):
        _fill((out, idx, saved, fws), byte)
        nsa.forward_train(prob, t["q"], t["k"], t["v"], gates, out=out, idx=idx, saved=saved, workspace=fws)
        got = [_bits(out), _bits(idx)] + [_bits(x) for x in nsa.saved_views(prob, saved)]  # not the padding
        for use_saved in (None, saved):
            _fill((*grads, bws), byte)
            nsa.backward(prob, t["q"], t["k"], t["v"], gates, idx, t["dout"], *grads, workspace=bws,
                         saved=use_saved)
            torch.cuda.synchronize()
            for g in grads:
                if g is not None:
                    assert _finite(g), (byte, use_saved is not None)
            got += [_bits(g) for g in grads if g is not None]
        assert _finite(out)
        res.append(got)
    for j, (a, b) in enumerate(zip(*res)):
        assert torch.equal(a, b), j
