"""TEST INFRASTRUCTURE ONLY -- fp64 numpy statement of the learned parts
around the NSA forward: the block-compression MLP and the gate projection.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares nothing with the GPU library.

Sources ([P1] "Zhang Xiaojun Business Interviews #94" transcript, bidclub.ai):
  s4 "Inside Native Sparse Attention": each block of keys (and of values) is
     compressed into one learned representation; each branch's output is
     weighted by a gate the model learns from the token's input
     representation through a projection.
  s7 "Kimi Simplifies The Sparse Route": the earlier NSA work formed the
     block representation with an MLP, where MoBA takes the plain mean.

Readings where the pages leave the step open (the plainest that fits):
  * phi, the block MLP: one hidden layer over the block's keys flattened in
    token order, phi(X) = W2 relu(W1 vec(X) + b1) + b2, with
    vec(X)[i * d + c] = X[i, c] for token i < block and dim c < d; one phi
    for keys and one for values, shared by every block and KV group.
    Flattening in token order gives each position its own weights, so phi
    sees where in the block a token sits without a separate encoding.
  * gate projection: gates = sigmoid(x W^T + b) per token, x the token's
    hidden state [d_model], W [3H, d_model] (output features first), the
    three gates of head h at outputs 3h, 3h + 1, 3h + 2 (compressed,
    selected, window); with logits=True the sigmoid is left to the
    attention (its gate-logits mode).
Results are float64; compress() rounds the summaries once to the storage
type exactly as the mean pooling does, gate_proj() returns float64.
"""
from __future__ import annotations

import numpy as np


def _widen(a, dtype):
    a = np.asarray(a)
    if dtype == "bf16" and a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _round_store(x, dtype):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype != "bf16":
        return f
    u = f.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def mlp_rows(X, w1, b1, w2, b2):
    """phi over rows X [R, block * d] (float64): W2 relu(W1 x + b1) + b2."""
    h = X @ w1.T
    if b1 is not None:
        h = h + b1
    h = np.maximum(h, 0.0)
    y = h @ w2.T
    if b2 is not None:
        y = y + b2
    return y


def compress(prob, k, v, wk, wv, exact=False):
    """Learned block summaries kc [B, nb, G, d_qk], vc [B, nb, G, d_v] in the
    storage type (exact: float64, before that rounding).  wk, wv: dicts with
    w1 [dh, block * d], b1 [dh] or None, w2 [d, dh], b2 [d] or None (arrays
    in the storage type or float64)."""
    dt = prob["dtype"]
    B, L, G, bs = prob["batch"], prob["kv_len"], prob["n_groups"], prob["block"]
    nb = L // bs
    out = []
    for x, w in ((k, wk), (v, wv)):
        xx = _widen(x, dt)                               # [B, L, G, d]
        d = xx.shape[-1]
        blocks = xx[:, :nb * bs].reshape(B, nb, bs, G, d).transpose(0, 1, 3, 2, 4).reshape(B * nb * G, bs * d)
        W = {n: (None if w.get(n) is None else _widen(w[n], dt)) for n in ("w1", "b1", "w2", "b2")}
        y = mlp_rows(blocks, W["w1"], W["b1"], W["w2"], W["b2"]).reshape(B, nb, G, d)
        out.append(y if exact else _round_store(y, dt))
    return out[0], out[1]


def gate_proj(x, w, b, dtype, logits=False):
    """Gates [B, T, H, 3] (float64) from hidden states x [B, T, d_model],
    w [3H, d_model], b [3H] or None."""
    xx, ww = _widen(x, dtype), _widen(w, dtype)
    z = xx @ ww.T
    if b is not None:
        z = z + _widen(b, dtype)
    if not logits:
        z = 1.0 / (1.0 + np.exp(-z))
    return z.reshape(*xx.shape[:-1], -1, 3)


# ---- per-entry error bound of the gate projection (what the tests allow
# between gate_proj and a GPU's bf16-operand, fp32-accumulated result) ----
# Products of bf16 values are exact in fp32; a sum of n of them accumulated
# in fp32 in any order is within n 2^-24 times the sum of the products'
# absolute values of the exact sum (the worst case); the sigmoid's slope is
# at most 1/4.

_U32 = 2.0 ** -24


def gate_proj_error_bound(x, w, b, dtype, logits=False):
    """Per-entry bound (float64, gate_proj's shape, before the final rounding
    to the storage type) on |GPU - exact|."""
    xx, ww = _widen(x, dtype), _widen(w, dtype)
    n = xx.shape[-1]
    a = np.abs(xx) @ np.abs(ww).T
    if b is not None:
        a = a + np.abs(_widen(b, dtype))
    bound = (n + 1) * _U32 * a * (1.0 if logits else 0.25)
    return bound.reshape(*xx.shape[:-1], -1, 3)
