"""Shared test helpers: small problems, widening, library-routine references."""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

from long_context_dynamic_amd import inputs, workloads


def problem(**kw) -> dict:
    """A small problem: the tiny fp32 workload with fields replaced."""
    p = workloads.get("nsa_tiny_fp32")
    p.update(kw)
    return p


def make(prob: dict) -> dict:
    return inputs.generate(prob)


def widen(a: np.ndarray, prob_or_dtype) -> np.ndarray:
    dt = prob_or_dtype["dtype"] if isinstance(prob_or_dtype, dict) else prob_or_dtype
    if dt == "bf16":
        return inputs.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def store(x: np.ndarray, prob: dict) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float32)
    return inputs.f32_to_bf16_bits(x32) if prob["dtype"] == "bf16" else np.ascontiguousarray(x32)


def positions(prob: dict) -> np.ndarray:
    """Absolute position of every query row."""
    return prob["kv_len"] - prob["q_len"] + np.arange(prob["q_len"])


def sdpa(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    """torch's scaled_dot_product_attention in float64 on the CPU with a boolean
    mask [T, L] (True = attend).  Rows with no allowed key are returned as 0."""
    allowed = mask.any(axis=1)
    safe = mask.copy()
    safe[~allowed, 0] = True
    out = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], attn_mask=torch.from_numpy(safe)[None, None],
        scale=scale).numpy()[0, 0]
    out[~allowed] = 0.0
    return out


def softmax_probs(q: np.ndarray, k: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    """torch.softmax over masked logits in float64; fully masked rows give 0."""
    logits = torch.from_numpy(q) @ torch.from_numpy(k).T * scale
    logits = logits.masked_fill(~torch.from_numpy(mask), float("-inf"))
    probs = torch.softmax(logits, dim=-1)
    return torch.nan_to_num(probs, nan=0.0).numpy()


def default_scale(prob: dict) -> float:
    return prob["scale"] if prob.get("scale") else 1.0 / np.sqrt(prob["d_qk"])
