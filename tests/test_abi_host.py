"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every call include/nsa.h declares, and rejects bad arguments synchronously,
before anything is queued (fake device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from long_context_dynamic_amd import nsa, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class _NoStream:
    cuda_stream = 0


def _declared():
    text = open(os.path.join(ROOT, "include", "nsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\**\s*(nsa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("nsa_compress", "nsa_select_topk", "nsa_sparse_attn", "nsa_forward",
              "nsa_workspace_bytes", "nsa_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = nsa.lib()
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings():
    lib = nsa.lib()
    seen = {lib.nsa_status_str(c).decode() for c in range(5)}
    assert len(seen) == 5
    assert lib.nsa_status_str(99).decode() == "unknown status"


FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation


def _p(prob, **kw):
    p = nsa.params(prob, stream=_NoStream, **{k: v for k, v in kw.items() if k in ("flags",)})
    for k, v in kw.items():
        if k != "flags":
            setattr(p, k, v)
    return p


def _forward(p, gates=FAKE, q=FAKE, out=FAKE):
    return nsa.lib().nsa_forward(q, FAKE, FAKE, gates, ctypes.byref(p), out)


BASE = workloads.get("nsa_prefill_8k", q_len=256, kv_len=256)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, 1), ("q_len", 0, 1), ("kv_len", 100, 1), ("n_kv_groups", 0, 1),
    ("heads_per_group", 0, 1), ("heads_per_group", 17, 2), ("d_qk", 0, 1), ("d_qk", 300, 2),
    ("d_v", 257, 2), ("block", 0, 1), ("block", 8192, 2), ("top_k", -1, 1), ("top_k", 1, 1),
    ("top_k", 65, 2), ("window", -1, 1), ("window", 20000, 2), ("dtype", 7, 1), ("flags", 1 << 9, 1),
    ("scale", -1.0, 1), ("scale", float("inf"), 1), ("scale", float("nan"), 1),
    ("sel_block", -64, 1), ("sel_block", 96, 1), ("sel_block", 8192, 2),
])
def test_bad_params_are_rejected_before_launch(field, value, code):
    p = _p(BASE)
    setattr(p, field, value)
    assert _forward(p) == code
    assert nsa.lib().nsa_workspace_bytes(ctypes.byref(p)) == 0


def test_huge_sizes_are_unsupported():
    # every int32 field at its largest: the grid-size checks must not overflow
    # (run under UndefinedBehaviorSanitizer by test_host_sanitizers.py)
    big = (1 << 31) - 1
    for b, t, g in ((big, big, big), (1, big, big), (big, 1, 1), (3, (1 << 30), 1), (1, 1 << 27, 16)):
        p = _p(BASE)
        p.batch, p.q_len, p.kv_len, p.n_kv_groups = b, t, t, g
        p.block, p.sel_block = 4096, 0
        assert _forward(p) == 2, (b, t, g)
        assert nsa.lib().nsa_workspace_bytes(ctypes.byref(p)) == 0
    p = _p(BASE)
    p.batch, p.q_len, p.kv_len, p.n_kv_groups = 1, 1 << 20, 1 << 20, 1024
    assert _forward(p) == 3        # 2^30 (b, t, g) rows fit: only the workspace is missing


def test_empty_summary_arrays_may_be_null():
    # no complete block: the summary arrays are empty, so NULL is accepted
    # (and nothing is launched); with complete blocks NULL stays invalid
    lib = nsa.lib()
    p = _p(workloads.get("nsa_prefill_8k", q_len=40, kv_len=40))
    assert lib.nsa_compress(FAKE, FAKE, 0, 0, ctypes.byref(p)) == 0
    assert lib.nsa_compress(FAKE, FAKE, 0, 0, ctypes.byref(_p(BASE))) == 1
    assert lib.nsa_select_topk(FAKE, 0, FAKE, 0, ctypes.byref(_p(BASE))) == 1
    w = nsa.MlpWeights()
    w.d_hidden = 192
    for n in ("k_w1", "k_w2", "v_w1", "v_w2"):
        setattr(w, n, FAKE)
    assert lib.nsa_compress_mlp(FAKE, FAKE, ctypes.byref(w), 0, 0, ctypes.byref(p)) == 0
    assert lib.nsa_compress_mlp(FAKE, FAKE, ctypes.byref(w), 0, 0, ctypes.byref(_p(BASE))) == 1


def test_pointer_and_flag_errors():
    lib = nsa.lib()
    p = _p(BASE)
    assert _forward(p, q=0) == 1                        # NULL q
    assert _forward(p, q=FAKE + 2) == 1                 # misaligned q
    assert _forward(p, gates=0) == 1                    # three branches need gates
    p0 = _p(BASE, flags=0)
    assert _forward(p0) == 1                            # no branch at all
    p1 = _p(BASE)
    p1.k_cmp = FAKE                                     # summaries: both or neither
    assert _forward(p1) == 1
    p2 = _p(BASE)
    p2.workspace, p2.workspace_bytes = FAKE, 16         # too small
    assert _forward(p2) == 3
    p3 = _p(BASE)
    assert _forward(p3) == 3                            # none given
    assert lib.nsa_compress(FAKE, FAKE, 0, FAKE, ctypes.byref(p)) == 1
    assert lib.nsa_select_topk(FAKE, FAKE, FAKE + 4, 0, ctypes.byref(p)) == 1
    assert lib.nsa_sparse_attn(FAKE, FAKE, FAKE, FAKE, 0, 0, ctypes.byref(p)) == 1
    assert lib.nsa_compress(FAKE, FAKE, FAKE, FAKE, None) == 1


def test_workspace_sizes():
    for name in workloads.WORKLOADS:
        prob = workloads.get(name)
        need = nsa.workspace_bytes(prob)
        assert need > 0, name
        assert need % 256 == 0
    # a caller-provided summary cache needs less room than computing it
    dec = workloads.get("nsa_decode_64x64k")
    assert nsa.workspace_bytes(dec, have_cmp=True) < nsa.workspace_bytes(dec)


def _backward(p, gates=FAKE, dout=FAKE, dgates=FAKE, saved=0):
    return nsa.lib().nsa_backward(FAKE, FAKE, FAKE, gates, FAKE, dout, saved, FAKE, FAKE, FAKE, dgates,
                                  ctypes.byref(p))


def _forward_train(p, gates=FAKE, idx=FAKE, saved=FAKE):
    return nsa.lib().nsa_forward_train(FAKE, FAKE, FAKE, gates, ctypes.byref(p), FAKE, idx, saved)


def test_backward_validation():
    lib = nsa.lib()
    p = _p(BASE)
    assert _backward(p, dout=0) == 1                          # NULL dout
    assert _backward(p, gates=0, dgates=0) == 1               # three branches need gates
    pw = _p(BASE, flags=nsa.F_SLC)
    assert _backward(pw, gates=0, dgates=FAKE) == 1           # dgates without gates
    assert _backward(p) == 3                                  # no workspace
    p.workspace, p.workspace_bytes = FAKE, 16
    assert _backward(p) == 3                                  # too small
    tiny = _p(workloads.get("nsa_tiny_fp32"))
    assert _backward(tiny) == 2                               # fp32: outside the kernels' limits
    assert lib.nsa_backward_workspace_bytes(ctypes.byref(tiny)) == 0
    odd = _p(workloads.get("nsa_prefill_8k", q_len=256, kv_len=256, block=32))
    assert _backward(odd) == 2                                # 32-token blocks
    need = nsa.backward_workspace_bytes(workloads.get("nsa_prefill_64k"))
    assert need > 0 and need % 256 == 0
    assert nsa.backward_phases(BASE) == ["bwd_images", "bwd_lists", "bwd_kv_selected_stats", "bwd_q",
                                         "bwd_kv_window", "bwd_kv_selected", "bwd_kv_compressed", "bwd_reduce"]


def test_learned_parts_validation():
    lib = nsa.lib()
    p = _p(BASE)
    w = nsa.MlpWeights()
    w.d_hidden = 192
    for n in ("k_w1", "k_w2", "v_w1", "v_w2"):
        setattr(w, n, FAKE)
    assert lib.nsa_compress_mlp(FAKE, FAKE, None, FAKE, FAKE, ctypes.byref(p)) == 1   # no weights
    w.k_w1 = 0
    assert lib.nsa_compress_mlp(FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, ctypes.byref(p)) == 1
    w.k_w1 = FAKE
    w.d_hidden = 100
    assert lib.nsa_compress_mlp(FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, ctypes.byref(p)) == 2
    tiny = _p(workloads.get("nsa_tiny_fp32"))
    w.d_hidden = 64
    assert lib.nsa_compress_mlp(FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, ctypes.byref(tiny)) == 2
    assert lib.nsa_gate_proj(0, 2560, FAKE, 0, FAKE, ctypes.byref(p)) == 1             # NULL x
    assert lib.nsa_gate_proj(FAKE, 100, FAKE, 0, FAKE, ctypes.byref(p)) == 2           # d_model % 32
    assert lib.nsa_gate_proj(FAKE, 2560, FAKE, 0, FAKE, ctypes.byref(tiny)) == 2       # fp32


def test_training_forward_validation():
    lib = nsa.lib()
    p = _p(BASE)
    assert _forward_train(p, idx=0) == 1                      # the selection goes to the caller
    assert _forward_train(p, saved=0) == 1                    # NULL statistics
    assert _forward_train(p, saved=FAKE + 8) == 1             # misaligned statistics
    assert _forward_train(p) == 3                             # no workspace
    pc = _p(BASE)
    pc.k_cmp = pc.v_cmp = FAKE                                # learned summaries: not what the backward pools
    assert _forward_train(pc) == 2
    tiny = _p(workloads.get("nsa_tiny_fp32"))
    assert _forward_train(tiny) == 2 and lib.nsa_train_saved_bytes(ctypes.byref(tiny)) == 0
    dec = workloads.get("nsa_decode_64x64k")
    pd = _p(dec)
    assert _forward_train(pd) == 2                            # decoding shapes keep no statistics
    assert lib.nsa_train_saved_bytes(ctypes.byref(pd)) == 0
    pd.workspace, pd.workspace_bytes = FAKE, 1 << 40
    assert _backward(pd, saved=FAKE) == 2                     # nor can the backward take them
    assert _backward(_p(BASE), saved=FAKE + 8) == 1
    B, T, H, dv = BASE["batch"], BASE["q_len"], BASE["n_groups"] * BASE["heads_per_group"], BASE["d_v"]
    lse_bytes = (3 * B * T * H * 4 + 255) // 256 * 256
    assert nsa.train_saved_bytes(BASE) == lse_bytes + 3 * B * T * H * dv * 2


def test_noalloc_forward_validates_like_forward_and_refuses_beyond_its_scratch():
    # the allocation-free forward checks its arguments as nsa_forward does and
    # refuses a call whose workspace exceeds its fixed scratch, both before
    # anything touches a device
    lib = nsa.lib()
    p = _p(BASE)
    p.batch = 0
    assert lib.nsa_forward_noalloc(FAKE, FAKE, FAKE, FAKE, ctypes.byref(p), FAKE) == 1
    big = workloads.get("nsa_prefill_8k")
    p = _p(big)
    assert lib.nsa_workspace_bytes(ctypes.byref(p)) > nsa.NOALLOC_SCRATCH_BYTES
    p.workspace, p.workspace_bytes = FAKE, 1 << 40  # ignored by this call
    assert lib.nsa_forward_noalloc(FAKE, FAKE, FAKE, FAKE, ctypes.byref(p), FAKE) == 3


def test_binding_knows_the_noalloc_scratch_size():
    text = open(os.path.join(ROOT, "include", "nsa.h")).read()
    m = re.search(r"#define NSA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == nsa.NOALLOC_SCRATCH_BYTES
