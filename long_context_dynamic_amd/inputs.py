"""Seeded synthetic inputs (no attention arithmetic here).

Recipe.  For batch element b, ``seq = SeedSequence(seed).spawn(B)[b]`` and
``seq.spawn(4)`` gives one stream per tensor (q, k, v, gates).  Each tensor
is drawn in chunks of CHUNK tokens; chunk c uses the c-th child of its
tensor's stream, ``Generator(PCG64(child))``, so chunks can be filled in
parallel and a shorter problem is a prefix of a longer one.  Values:

    q       ~ N(0, 1)       [T, H, d_qk]
    k       ~ N(0, 1)       [L, G, d_qk], plus a per-block offset
    offset  ~ N(0, std^2)   [ceil(L / block), G, d_qk] (std = key_offset_std),
                            drawn first from the k stream's last child and
                            added to every key of its block
    v       ~ N(0, 1)       [L, G, d_v]
    gates   ~ U(0, 1)       [T, H, 3]
    dout    ~ N(0, 1)       [T, H, d_v]  (the upstream gradient of a backward
                            pass; its stream is the fifth child, so the first
                            four tensors do not depend on whether it is drawn)

all float32, then stored as float32 or rounded to bf16 (nearest, ties to
even).  The per-block key offset gives blocks distinct summaries, so the
top-k choice is not a coin toss.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

CHUNK = 4096
_OFFSET_CHILD = 1 << 20  # child index reserved for the key offsets


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 22
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        flat_o[s:s + step] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
                              >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _child(ss: np.random.SeedSequence, c: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ss.entropy, spawn_key=ss.spawn_key + (c,))))


def _fill(out: np.ndarray, ss, rows: int, width_shape, dtype: str, kind: str, pool, offset=None, bs=1):
    """Fill out[rows, *width_shape] chunk by chunk."""
    def one(c):
        lo, hi = c * CHUNK, min(rows, (c + 1) * CHUNK)
        g = _child(ss, c)
        shape = (hi - lo,) + tuple(width_shape)
        x = g.standard_normal(shape, dtype=np.float32) if kind == "normal" else g.random(shape, dtype=np.float32)
        if offset is not None:
            blk = np.arange(lo, hi) // bs
            x += offset[blk]
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    list(pool.map(one, range(-(-rows // CHUNK))))


def generate_sequence(prob: dict, b: int, want=("q", "k", "v", "gates"), pool=None) -> dict:
    """Inputs of batch element b, each with a leading batch dimension of 1."""
    T, L = prob["q_len"], prob["kv_len"]
    G, hpg = prob["n_groups"], prob["heads_per_group"]
    H, dq, dv, bs = G * hpg, prob["d_qk"], prob["d_v"], prob["block"]
    dt = prob["dtype"]
    st = np.uint16 if dt == "bf16" else np.float32
    seq = np.random.SeedSequence(int(prob.get("seed", 0))).spawn(int(prob["batch"]))[b]
    s_q, s_k, s_v, s_g, s_d = seq.spawn(5)
    own = pool is None
    pool = pool or cf.ThreadPoolExecutor(_workers())
    try:
        out = {}
        if "q" in want:
            out["q"] = np.empty((1, T, H, dq), st)
            _fill(out["q"][0], s_q, T, (H, dq), dt, "normal", pool)
        if "k" in want:
            nbk = -(-L // bs)
            offset = _child(s_k, _OFFSET_CHILD).standard_normal((nbk, G, dq), dtype=np.float32)
            offset *= np.float32(prob.get("key_offset_std", 0.5))
            out["k"] = np.empty((1, L, G, dq), st)
            _fill(out["k"][0], s_k, L, (G, dq), dt, "normal", pool, offset=offset, bs=bs)
        if "v" in want:
            out["v"] = np.empty((1, L, G, dv), st)
            _fill(out["v"][0], s_v, L, (G, dv), dt, "normal", pool)
        if "gates" in want:
            out["gates"] = np.empty((1, T, H, 3), st)
            _fill(out["gates"][0], s_g, T, (H, 3), dt, "uniform", pool)
        if "dout" in want:
            out["dout"] = np.empty((1, T, H, dv), st)
            _fill(out["dout"][0], s_d, T, (H, dv), dt, "normal", pool)
        return out
    finally:
        if own:
            pool.shutdown()


def learned_weights(prob: dict, d_hidden: int, d_model: int = 2560, seed: int = 0, bias: bool = True) -> dict:
    """Random-initialised weights of the learned block compression and of the
    gate projection, plus hidden states x [B, T, d_model] ~ N(0, 1), stored
    like the other inputs.  Scales keep every layer's output near unit size:
    w1 ~ N(0, 1 / (block * d)), w2 ~ N(0, 1 / d_hidden), gate w ~ N(0, 1 /
    d_model), biases ~ N(0, 0.1^2).  Returns {"k": {w1, b1, w2, b2}, "v":
    {...}, "gate_w", "gate_b", "x"} (biases None when bias is False)."""
    dt = prob["dtype"]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 0x5EED])))
    H, bs = prob["n_groups"] * prob["heads_per_group"], prob["block"]

    def st(a):
        a = np.ascontiguousarray(a, dtype=np.float32)
        return f32_to_bf16_bits(a) if dt == "bf16" else a

    out = {}
    for name, d in (("k", prob["d_qk"]), ("v", prob["d_v"])):
        out[name] = {
            "w1": st(rng.standard_normal((d_hidden, bs * d), dtype=np.float32) / np.sqrt(bs * d)),
            "b1": st(0.1 * rng.standard_normal(d_hidden, dtype=np.float32)) if bias else None,
            "w2": st(rng.standard_normal((d, d_hidden), dtype=np.float32) / np.sqrt(d_hidden)),
            "b2": st(0.1 * rng.standard_normal(d, dtype=np.float32)) if bias else None,
        }
    out["gate_w"] = st(rng.standard_normal((3 * H, d_model), dtype=np.float32) / np.sqrt(d_model))
    out["gate_b"] = st(0.1 * rng.standard_normal(3 * H, dtype=np.float32)) if bias else None
    out["x"] = st(rng.standard_normal((prob["batch"], prob["q_len"], d_model), dtype=np.float32))
    return out


def generate(prob: dict, want=("q", "k", "v", "gates")) -> dict:
    """Inputs for every batch element, concatenated along the batch axis."""
    with cf.ThreadPoolExecutor(_workers()) as pool:
        parts = [generate_sequence(prob, b, want, pool) for b in range(prob["batch"])]
    if len(parts) == 1:
        return parts[0]
    return {name: np.concatenate([p[name] for p in parts], axis=0) for name in parts[0]}
