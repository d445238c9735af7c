"""Seeded synthetic inputs (no attention arithmetic here).

Recipe, per batch element b (its own stream, so sequences can be generated
one at a time): numpy ``Generator(PCG64(SeedSequence(seed).spawn(B)[b]))``
draws, in this order,

    q       ~ N(0, 1)       [T, H, d_qk]
    k       ~ N(0, 1)       [L, G, d_qk]
    offset  ~ N(0, std^2)   [ceil(L / block), G, d_qk], added to every key of its block
    v       ~ N(0, 1)       [L, G, d_v]
    gates   ~ U(0, 1)       [T, H, 3]

all in float32, then stored as float32 or rounded to bf16 (nearest, ties to
even).  The per-block key offset gives blocks distinct summaries, so the
top-k choice is not a coin toss.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        flat_o[s:s + step] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
                              >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def sequence_rng(prob: dict, b: int) -> np.random.Generator:
    seq = np.random.SeedSequence(int(prob.get("seed", 0))).spawn(int(prob["batch"]))[b]
    return np.random.Generator(np.random.PCG64(seq))


def generate_sequence(prob: dict, b: int, want=("q", "k", "v", "gates")) -> dict:
    """Inputs of batch element b, each with a leading batch dimension of 1."""
    rng = sequence_rng(prob, b)
    T, L = prob["q_len"], prob["kv_len"]
    G, hpg = prob["n_groups"], prob["heads_per_group"]
    H, dq, dv, bs = G * hpg, prob["d_qk"], prob["d_v"], prob["block"]
    dt = prob["dtype"]
    out = {}
    q = rng.standard_normal((T, H, dq), dtype=np.float32)
    if "q" in want:
        out["q"] = _store(q, dt)[None]
    del q
    k = rng.standard_normal((L, G, dq), dtype=np.float32)
    nbk = -(-L // bs)
    offset = rng.standard_normal((nbk, G, dq), dtype=np.float32) * np.float32(prob.get("key_offset_std", 0.5))
    for j in range(nbk):
        k[j * bs:(j + 1) * bs] += offset[j]
    if "k" in want:
        out["k"] = _store(k, dt)[None]
    del k
    v = rng.standard_normal((L, G, dv), dtype=np.float32)
    if "v" in want:
        out["v"] = _store(v, dt)[None]
    del v
    gates = rng.random((T, H, 3), dtype=np.float32)
    if "gates" in want:
        out["gates"] = _store(gates, dt)[None]
    return out


def generate(prob: dict, want=("q", "k", "v", "gates")) -> dict:
    """Inputs for every batch element, concatenated along the batch axis."""
    parts = [generate_sequence(prob, b, want) for b in range(prob["batch"])]
    return {name: np.concatenate([p[name] for p in parts], axis=0) for name in parts[0]}
