"""ctypes binding of libnsa.so (the C ABI in include/nsa.h).

Argument marshalling only: every step of the forward pass runs in the HIP
library.  torch provides device memory and the current stream.  There is no
fallback: if the library is not built, loading fails loudly.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnsa.so")

NSA_BF16, NSA_F32 = 0, 1
F_FORCE_FIRST, F_FORCE_CURRENT, F_CMP, F_SLC, F_WIN, F_GATE_LOGITS, F_OUT_F32 = 1, 2, 4, 8, 16, 32, 64

STATUS = {0: "NSA_OK", 1: "NSA_ERR_INVALID_ARG", 2: "NSA_ERR_UNSUPPORTED", 3: "NSA_ERR_WORKSPACE",
          4: "NSA_ERR_HIP"}

EXPORTS = ("nsa_compress", "nsa_select_topk", "nsa_sparse_attn", "nsa_forward",
           "nsa_forward_phases", "nsa_workspace_bytes", "nsa_backward", "nsa_backward_workspace_bytes",
           "nsa_backward_phases", "nsa_compress_mlp", "nsa_gate_proj", "nsa_forward_train",
           "nsa_train_saved_bytes", "nsa_status_str", "nsa_forward_noalloc")

NOALLOC_SCRATCH_BYTES = 64 << 20  # NSA_NOALLOC_SCRATCH_BYTES


class NsaError(RuntimeError):
    def __init__(self, call: str, code: int, text: str):
        super().__init__(f"{call}: {STATUS.get(code, code)} ({text})")
        self.code = code


class MlpWeights(ctypes.Structure):
    _fields_ = [("d_hidden", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("k_w1", "k_b1", "k_w2", "k_b2", "v_w1", "v_b1", "v_w2", "v_b2")]


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
        ("n_kv_groups", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("block", ctypes.c_int32), ("top_k", ctypes.c_int32), ("window", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("k_cmp", ctypes.c_void_p), ("v_cmp", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("phase_events", ctypes.POINTER(ctypes.c_void_p)), ("n_phase_events", ctypes.c_int32),
        ("sel_block", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libnsa.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: run `python -m long_context_dynamic_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER(Params)
        L.nsa_compress.argtypes = [vp, vp, vp, vp, P]
        L.nsa_select_topk.argtypes = [vp, vp, vp, vp, P]
        L.nsa_sparse_attn.argtypes = [vp, vp, vp, vp, vp, vp, P]
        L.nsa_forward.argtypes = [vp, vp, vp, vp, P, vp]
        L.nsa_forward_noalloc.argtypes = [vp, vp, vp, vp, P, vp]
        L.nsa_workspace_bytes.argtypes = [P]
        L.nsa_workspace_bytes.restype = ctypes.c_size_t
        L.nsa_forward_phases.argtypes = [P, ctypes.POINTER(ctypes.c_char_p), ctypes.c_int32]
        L.nsa_forward_phases.restype = ctypes.c_int32
        L.nsa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, P]
        L.nsa_forward_train.argtypes = [vp, vp, vp, vp, P, vp, vp, vp]
        L.nsa_train_saved_bytes.argtypes = [P]
        L.nsa_train_saved_bytes.restype = ctypes.c_size_t
        L.nsa_backward_workspace_bytes.argtypes = [P]
        L.nsa_backward_workspace_bytes.restype = ctypes.c_size_t
        L.nsa_backward_phases.argtypes = [P, ctypes.POINTER(ctypes.c_char_p), ctypes.c_int32]
        L.nsa_backward_phases.restype = ctypes.c_int32
        L.nsa_compress_mlp.argtypes = [vp, vp, ctypes.POINTER(MlpWeights), vp, vp, P]
        L.nsa_gate_proj.argtypes = [vp, ctypes.c_int32, vp, vp, vp, P]
        L.nsa_status_str.argtypes = [ctypes.c_int]
        L.nsa_status_str.restype = ctypes.c_char_p
        for name in ("nsa_compress", "nsa_select_topk", "nsa_sparse_attn", "nsa_forward", "nsa_forward_noalloc",
                     "nsa_backward",
                     "nsa_compress_mlp", "nsa_gate_proj", "nsa_forward_train"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def library_path() -> str:
    return _LIB_PATH


def flags_of(prob: dict, out_f32: bool = False) -> int:
    f = 0
    f |= F_FORCE_FIRST if prob["force_first"] else 0
    f |= F_FORCE_CURRENT if prob["force_current"] else 0
    f |= F_CMP if prob["use_cmp"] else 0
    f |= F_SLC if prob["use_slc"] else 0
    f |= F_WIN if prob["use_win"] else 0
    f |= F_GATE_LOGITS if prob.get("gate_logits") else 0
    f |= F_OUT_F32 if out_f32 else 0
    return f


def torch_dtype(prob: dict):
    return torch.bfloat16 if prob["dtype"] == "bf16" else torch.float32


def params(prob: dict, *, out_f32: bool = False, k_cmp=None, v_cmp=None, workspace=None,
           stream=None, flags=None) -> Params:
    p = Params()
    p.batch, p.q_len, p.kv_len = prob["batch"], prob["q_len"], prob["kv_len"]
    p.n_kv_groups, p.heads_per_group = prob["n_groups"], prob["heads_per_group"]
    p.d_qk, p.d_v = prob["d_qk"], prob["d_v"]
    p.block, p.top_k, p.window = prob["block"], prob["top_k"], prob["window"]
    p.sel_block = int(prob.get("sel_block", 0) or 0)
    p.flags = flags_of(prob, out_f32) if flags is None else flags
    p.dtype = NSA_BF16 if prob["dtype"] == "bf16" else NSA_F32
    p.scale = float(prob.get("scale") or 0.0)
    p.k_cmp = None if k_cmp is None else k_cmp.data_ptr()
    p.v_cmp = None if v_cmp is None else v_cmp.data_ptr()
    if workspace is not None:
        p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream()
    p.stream = stream.cuda_stream
    return p


def _on_stream(fn):
    """Run a wrapper with the caller's stream (keyword `stream`) current, so
    every tensor it allocates (outputs, workspace) belongs to the stream the
    library queues its kernels on: the caching allocator then cannot hand
    that memory to other work while those kernels still use it."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        ctx = contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)
        with ctx:
            return fn(*args, stream=stream, **kw)
    return run


def _call(name: str, *args) -> None:
    code = getattr(lib(), name)(*args)
    if code != 0:
        raise NsaError(name, code, lib().nsa_status_str(code).decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, shape, dtype, name: str) -> None:
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shapes(prob: dict) -> dict:
    B, T, L, G, hpg = prob["batch"], prob["q_len"], prob["kv_len"], prob["n_groups"], prob["heads_per_group"]
    H, dq, dv, nb, n = G * hpg, prob["d_qk"], prob["d_v"], L // prob["block"], prob["top_k"]
    return dict(q=(B, T, H, dq), k=(B, L, G, dq), v=(B, L, G, dv), gates=(B, T, H, 3),
                kc=(B, nb, G, dq), vc=(B, nb, G, dv), idx=(B, T, G, n), out=(B, T, H, dv),
                lse=(B, T, H))


def workspace_bytes(prob: dict, have_cmp: bool = False) -> int:
    p = params(prob, stream=_NoStream)
    p.k_cmp = p.v_cmp = (16 if have_cmp else None)  # only NULL / non-NULL matters here
    return int(lib().nsa_workspace_bytes(ctypes.byref(p)))


class _NoStream:
    cuda_stream = 0


def alloc_workspace(prob: dict, have_cmp: bool = False, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(prob, have_cmp), 256), dtype=torch.uint8, device=device)


@_on_stream
def compress(prob: dict, k: torch.Tensor, v: torch.Tensor, kc=None, vc=None, stream=None):
    s, dt = _shapes(prob), torch_dtype(prob)
    _check(k, s["k"], dt, "k")
    _check(v, s["v"], dt, "v")
    kc = torch.empty(s["kc"], dtype=dt, device=k.device) if kc is None else kc
    vc = torch.empty(s["vc"], dtype=dt, device=k.device) if vc is None else vc
    _check(kc, s["kc"], dt, "k_cmp")
    _check(vc, s["vc"], dt, "v_cmp")
    p = params(prob, stream=stream)
    _call("nsa_compress", k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), ctypes.byref(p))
    return kc, vc


@_on_stream
def select_topk(prob: dict, q: torch.Tensor, kc: torch.Tensor, idx=None, score=None, want_score=True,
                workspace=None, stream=None):
    s, dt = _shapes(prob), torch_dtype(prob)
    _check(q, s["q"], dt, "q")
    _check(kc, s["kc"], dt, "k_cmp")
    idx = torch.empty(s["idx"], dtype=torch.int32, device=q.device) if idx is None else idx
    if want_score and score is None:
        score = torch.empty(s["idx"], dtype=torch.float32, device=q.device)
    _check(idx, s["idx"], torch.int32, "idx")
    if workspace is None:
        workspace = alloc_workspace(prob, True, q.device)
    p = params(prob, workspace=workspace, stream=stream)
    _call("nsa_select_topk", q.data_ptr(), kc.data_ptr(), idx.data_ptr(), _ptr(score), ctypes.byref(p))
    return idx, score


@_on_stream
def sparse_attn(prob: dict, q, k, v, idx, out=None, lse=None, want_lse=True, out_f32=False,
                workspace=None, stream=None):
    s, dt = _shapes(prob), torch_dtype(prob)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, s[name], dt, name)
    _check(idx, s["idx"], torch.int32, "idx")
    odt = torch.float32 if out_f32 else dt
    out = torch.empty(s["out"], dtype=odt, device=q.device) if out is None else out
    _check(out, s["out"], odt, "out")
    if want_lse and lse is None:
        lse = torch.empty(s["lse"], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(prob, True, q.device)
    p = params(prob, out_f32=out_f32, workspace=workspace, stream=stream)
    _call("nsa_sparse_attn", q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), out.data_ptr(),
          _ptr(lse), ctypes.byref(p))
    return out, lse


def forward_phases(prob: dict, have_cmp: bool = False) -> list:
    """Names of the kernels nsa_forward launches for this problem, in order."""
    p = params(prob, stream=_NoStream)
    p.k_cmp = p.v_cmp = (16 if have_cmp else None)
    names = (ctypes.c_char_p * 64)()
    n = lib().nsa_forward_phases(ctypes.byref(p), names, 64)
    return [names[i].decode() for i in range(min(n, 64))]


@_on_stream
def forward(prob: dict, q, k, v, gates, out=None, k_cmp=None, v_cmp=None, out_f32=False,
            workspace=None, stream=None, events=None):
    s, dt = _shapes(prob), torch_dtype(prob)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, s[name], dt, name)
    if gates is not None:
        _check(gates, s["gates"], dt, "gates")
    if k_cmp is not None:
        _check(k_cmp, s["kc"], dt, "k_cmp")
        _check(v_cmp, s["vc"], dt, "v_cmp")
    odt = torch.float32 if out_f32 else dt
    out = torch.empty(s["out"], dtype=odt, device=q.device) if out is None else out
    _check(out, s["out"], odt, "out")
    if workspace is None:
        workspace = alloc_workspace(prob, k_cmp is not None, q.device)
    p = params(prob, out_f32=out_f32, k_cmp=k_cmp, v_cmp=v_cmp, workspace=workspace, stream=stream)
    if events is not None:  # torch.cuda.Event list: recorded around each kernel
        for e in events:
            if not e.cuda_event:  # torch creates the HIP event on first record
                e.record()
        handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        p.phase_events, p.n_phase_events = handles, len(events)
    _call("nsa_forward", q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(gates), ctypes.byref(p),
          out.data_ptr())
    return out


@_on_stream
def forward_noalloc(prob: dict, q, k, v, gates, out, k_cmp=None, v_cmp=None, out_f32=False, stream=None):
    """nsa_forward_noalloc: the forward in the library's fixed device scratch
    (no workspace); out must be given (nothing is allocated here either)."""
    s, dt = _shapes(prob), torch_dtype(prob)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, s[name], dt, name)
    if gates is not None:
        _check(gates, s["gates"], dt, "gates")
    if k_cmp is not None:
        _check(k_cmp, s["kc"], dt, "k_cmp")
        _check(v_cmp, s["vc"], dt, "v_cmp")
    _check(out, s["out"], torch.float32 if out_f32 else dt, "out")
    p = params(prob, out_f32=out_f32, k_cmp=k_cmp, v_cmp=v_cmp, stream=stream)
    _call("nsa_forward_noalloc", q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(gates), ctypes.byref(p),
          out.data_ptr())
    return out


def train_saved_bytes(prob: dict) -> int:
    p = params(prob, stream=_NoStream)
    return int(lib().nsa_train_saved_bytes(ctypes.byref(p)))


def saved_views(prob: dict, saved: torch.Tensor):
    """(lse fp32 [3, B, T, H], O bf16 [3, B, T, H, d_v]) views of a saved buffer."""
    B, T, H, dv = prob["batch"], prob["q_len"], prob["n_groups"] * prob["heads_per_group"], prob["d_v"]
    n = 3 * B * T * H
    lse_bytes = (n * 4 + 255) // 256 * 256
    lse = saved[:n * 4].view(torch.float32).view(3, B, T, H)
    o = saved[lse_bytes:lse_bytes + n * dv * 2].view(torch.bfloat16).view(3, B, T, H, dv)
    return lse, o


@_on_stream
def forward_train(prob: dict, q, k, v, gates, out=None, idx=None, saved=None, out_f32=False,
                  workspace=None, stream=None, events=None):
    """nsa_forward_train: (out, idx, saved) -- saved is the uint8 statistics buffer."""
    s, dt = _shapes(prob), torch_dtype(prob)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, s[name], dt, name)
    if gates is not None:
        _check(gates, s["gates"], dt, "gates")
    odt = torch.float32 if out_f32 else dt
    out = torch.empty(s["out"], dtype=odt, device=q.device) if out is None else out
    _check(out, s["out"], odt, "out")
    idx = torch.empty(s["idx"], dtype=torch.int32, device=q.device) if idx is None else idx
    _check(idx, s["idx"], torch.int32, "idx")
    need = train_saved_bytes(prob)
    if saved is None:
        saved = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(prob, False, q.device)
    p = params(prob, out_f32=out_f32, workspace=workspace, stream=stream)
    if events is not None:
        for e in events:
            if not e.cuda_event:
                e.record()
        handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        p.phase_events, p.n_phase_events = handles, len(events)
    _call("nsa_forward_train", q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(gates), ctypes.byref(p),
          out.data_ptr(), idx.data_ptr(), saved.data_ptr())
    return out, idx, saved


def backward_workspace_bytes(prob: dict) -> int:
    p = params(prob, stream=_NoStream)
    return int(lib().nsa_backward_workspace_bytes(ctypes.byref(p)))


def backward_phases(prob: dict) -> list:
    """Names of the kernel groups nsa_backward times, in order."""
    p = params(prob, stream=_NoStream)
    names = (ctypes.c_char_p * 64)()
    n = lib().nsa_backward_phases(ctypes.byref(p), names, 64)
    return [names[i].decode() for i in range(min(n, 64))]


@_on_stream
def backward(prob: dict, q, k, v, gates, idx, dout, dq=None, dk=None, dv=None, dgates=None,
             want_dgates=True, workspace=None, stream=None, events=None, saved=None):
    """Gradients of nsa_forward on the selection idx: (dq, dk, dv, dgates), fp32.
    saved: forward_train's statistics for the same inputs and idx, or None."""
    s, dt = _shapes(prob), torch_dtype(prob)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", dout)):
        _check(t, s[name], dt, "dout" if name == "out" else name)
    if gates is not None:
        _check(gates, s["gates"], dt, "gates")
    _check(idx, s["idx"], torch.int32, "idx")
    f32, dev = torch.float32, q.device
    dq = torch.empty(s["q"], dtype=f32, device=dev) if dq is None else dq
    dk = torch.empty(s["k"], dtype=f32, device=dev) if dk is None else dk
    dv = torch.empty(s["v"], dtype=f32, device=dev) if dv is None else dv
    if gates is not None and want_dgates and dgates is None:
        dgates = torch.empty(s["gates"], dtype=f32, device=dev)
    for name, t, shp in (("dq", dq, s["q"]), ("dk", dk, s["k"]), ("dv", dv, s["v"])):
        _check(t, shp, f32, name)
    if dgates is not None:
        _check(dgates, s["gates"], f32, "dgates")
    if workspace is None:
        workspace = torch.empty(max(backward_workspace_bytes(prob), 256), dtype=torch.uint8, device=dev)
    p = params(prob, workspace=workspace, stream=stream)
    if events is not None:  # torch.cuda.Event list: recorded around each kernel group
        for e in events:
            if not e.cuda_event:
                e.record()
        handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        p.phase_events, p.n_phase_events = handles, len(events)
    _call("nsa_backward", q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(gates), idx.data_ptr(),
          dout.data_ptr(), _ptr(saved), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _ptr(dgates),
          ctypes.byref(p))
    return dq, dk, dv, dgates


@_on_stream
def compress_mlp(prob: dict, k, v, wk: dict, wv: dict, kc=None, vc=None, stream=None):
    """Learned summaries: wk, wv hold device tensors w1, w2 and optional b1, b2."""
    s, dt = _shapes(prob), torch_dtype(prob)
    _check(k, s["k"], dt, "k")
    _check(v, s["v"], dt, "v")
    dh = wk["w1"].shape[0]
    for name, w, d in (("k", wk, prob["d_qk"]), ("v", wv, prob["d_v"])):
        _check(w["w1"], (dh, prob["block"] * d), dt, f"{name}_w1")
        _check(w["w2"], (d, dh), dt, f"{name}_w2")
        if w.get("b1") is not None:
            _check(w["b1"], (dh,), dt, f"{name}_b1")
        if w.get("b2") is not None:
            _check(w["b2"], (d,), dt, f"{name}_b2")
    kc = torch.empty(s["kc"], dtype=dt, device=k.device) if kc is None else kc
    vc = torch.empty(s["vc"], dtype=dt, device=k.device) if vc is None else vc
    _check(kc, s["kc"], dt, "k_cmp")
    _check(vc, s["vc"], dt, "v_cmp")
    mw = MlpWeights()
    mw.d_hidden = dh
    for pre, w in (("k_", wk), ("v_", wv)):
        for n in ("w1", "b1", "w2", "b2"):
            setattr(mw, pre + n, _ptr(w.get(n)))
    p = params(prob, stream=stream)
    _call("nsa_compress_mlp", k.data_ptr(), v.data_ptr(), ctypes.byref(mw), kc.data_ptr(), vc.data_ptr(),
          ctypes.byref(p))
    return kc, vc


@_on_stream
def gate_proj(prob: dict, x, w, bias=None, gates=None, logits=False, stream=None):
    """gates [B, T, H, 3] = sigmoid(x w^T + bias) (or the logits)."""
    s, dt = _shapes(prob), torch_dtype(prob)
    B, T, dm = x.shape
    _check(x, (prob["batch"], prob["q_len"], dm), dt, "x")
    _check(w, (3 * s["q"][2], dm), dt, "w")
    if bias is not None:
        _check(bias, (3 * s["q"][2],), dt, "bias")
    gates = torch.empty(s["gates"], dtype=dt, device=x.device) if gates is None else gates
    _check(gates, s["gates"], dt, "gates")
    flags = flags_of(prob) | (F_GATE_LOGITS if logits else 0)
    if not logits:
        flags &= ~F_GATE_LOGITS
    p = params(prob, stream=stream, flags=flags)
    _call("nsa_gate_proj", x.data_ptr(), dm, w.data_ptr(), _ptr(bias), gates.data_ptr(), ctypes.byref(p))
    return gates


def to_device(a, prob: dict, device="cuda") -> torch.Tensor:
    """Upload a numpy input (uint16 bf16 patterns or float32) as a device tensor."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def to_host_bits(t: torch.Tensor):
    """Download a device tensor as numpy (bf16 as uint16 patterns)."""
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.uint16).cpu().numpy()
    return t.detach().cpu().numpy()
