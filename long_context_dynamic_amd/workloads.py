"""Named problem descriptions (shapes and switches only, no arithmetic).

A problem is a plain dict that both the GPU binding and the test oracle
understand.  The named workloads are the shapes the pages discuss: NSA with
4 KV groups x 16 query heads, d_qk 192, 64-token blocks and top-16 ([P1] s5
"Hardware Makes Sparsity Work"; [P2] numbers table), MoBA with 512-token
blocks and top-3 ([P1] s7 "Kimi Simplifies The Sparse Route") at 32k, 128k
and 1M tokens (MoBA's evaluation reaches the million-token range: [P1] s7,
[P2] numbers table), and batched decoding over a 64k context ([P1] s6).
"""
from __future__ import annotations

import copy

_BASE = dict(
    batch=1, q_len=1024, kv_len=1024, n_groups=1, heads_per_group=4,
    d_qk=64, d_v=64, block=64, top_k=4, window=128,
    force_first=1, force_current=1, use_cmp=1, use_slc=1, use_win=1,
    gate_logits=0, dtype="f32", scale=0.0,
    sel_block=0,  # selection block size; 0: the compression block size
    key_offset_std=0.5, seed=0,
)

WORKLOADS = {
    # tiny fp32 NSA forward: 1 KV group x 4 heads, d 64, block 64, top-4, window 128
    "nsa_tiny_fp32": dict(_BASE),
    # NSA prefill at 8k: 4 groups x 16 heads, d_qk 192, d_v 128, block 64, top-16, window 512
    "nsa_prefill_8k": dict(_BASE, q_len=8192, kv_len=8192, n_groups=4, heads_per_group=16,
                           d_qk=192, d_v=128, block=64, top_k=16, window=512, dtype="bf16"),
    # the same at 64k tokens
    "nsa_prefill_64k": dict(_BASE, q_len=65536, kv_len=65536, n_groups=4, heads_per_group=16,
                            d_qk=192, d_v=128, block=64, top_k=16, window=512, dtype="bf16"),
    # the 64k prefill with 32-token summaries under 64-token selection blocks
    # (compression and selection block sizes decoupled)
    "nsa_prefill_64k_c32": dict(_BASE, q_len=65536, kv_len=65536, n_groups=4, heads_per_group=16,
                                d_qk=192, d_v=128, block=32, sel_block=64, top_k=16, window=512,
                                dtype="bf16"),
    # MoBA: 32 heads each with its own K/V, d 128, block 512, top-3 with the current
    # block always in, selected branch only, no gates
    "moba_32k": dict(_BASE, q_len=32768, kv_len=32768, n_groups=32, heads_per_group=1,
                     d_qk=128, d_v=128, block=512, top_k=3, window=0, force_first=0,
                     force_current=1, use_cmp=0, use_slc=1, use_win=0, dtype="bf16"),
    # MoBA at longer contexts: the same head layout and rule
    "moba_128k": dict(_BASE, q_len=131072, kv_len=131072, n_groups=32, heads_per_group=1,
                      d_qk=128, d_v=128, block=512, top_k=3, window=0, force_first=0,
                      force_current=1, use_cmp=0, use_slc=1, use_win=0, dtype="bf16"),
    "moba_1m": dict(_BASE, q_len=1048576, kv_len=1048576, n_groups=32, heads_per_group=1,
                    d_qk=128, d_v=128, block=512, top_k=3, window=0, force_first=0,
                    force_current=1, use_cmp=0, use_slc=1, use_win=0, dtype="bf16"),
    # NSA decode: 64 sequences, 65536-token cache each, one new query token
    "nsa_decode_64x64k": dict(_BASE, batch=64, q_len=1, kv_len=65536, n_groups=4,
                              heads_per_group=16, d_qk=192, d_v=128, block=64, top_k=16,
                              window=512, dtype="bf16"),
}


def get(name: str, **overrides) -> dict:
    """A copy of a named workload with some fields replaced."""
    prob = copy.deepcopy(WORKLOADS[name])
    prob.update(overrides)
    prob["name"] = name
    return prob


def n_heads(prob: dict) -> int:
    return prob["n_groups"] * prob["heads_per_group"]


def n_blocks(prob: dict) -> int:
    """Complete blocks in the KV sequence (rows of the pooled summaries)."""
    return prob["kv_len"] // prob["block"]
