"""Benchmark of the NSA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-moba] [--no-backward] [--no-cpu]

One step is one nsa_forward (pooling, selection, all three branches, gates)
over the 64k-token prefill workload (B=1, T=65536, 4 KV groups x 16 heads,
d_qk 192, d_v 128, block 64, top-16, window 512) with inputs resident in
HBM.  Prints ONE JSON line: tokens/s, per-kernel times from HIP events
recorded on the library's stream, the roofline of the dominant kernel, the
MoBA forward (32k tokens, 32 heads, 512-token blocks, top-3) with its own
roofline, the backward pass of the 64k workload (dq, dk, dv, dgates on its
selection) with its roofline, the batched-decode measurement (64 x 65536-token caches, % of HBM
peak) and the CPU oracle timed on a bounded sample of the 64k workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "NSA fwd tokens/s + % bf16 MFMA peak (64k prefill); decode % HBM peak"


# What the pages themselves report for this method, quoted as context: none
# of it is a measurement of this path or of this chip.
PAGE_CONTEXT = {
    "nsa_vs_flashattention_64k": "close to 10x faster than a FlashAttention kernel at 64k tokens, both "
                                 "written in Triton; hardware, precision and shapes not stated "
                                 "([P1] s6 'Why Sparse Attention Wins'; [P2] numbers table)",
    "shorter_sequences": "already faster at 8k-16k, the ratio growing with length; no numbers ([P1] s6, s7)",
    "decode": "memory-bound, set by the KV bytes read; a speed-up is expected but not quantified ([P1] s6)",
    "selection_granularity": "NSA: 64-token blocks, top-16; MoBA: 512-token blocks, top-3 ([P1] s7; [P2])",
    "model_shapes": "4 KV groups, 64 query heads, query head dim 192, hidden size 2560 ([P1] s5; [P2])",
    "matrix_vs_vector": "half-precision matrix units about 16x the vector ALUs at equal FLOPs, on A100 ([P1] s5)",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- counts --

def positions(prob):
    return prob["kv_len"] - prob["q_len"] + np.arange(prob["q_len"], dtype=np.int64)


def algorithmic_flops(prob):
    """Per-branch algorithmic FLOPs of one forward: 2 per multiply-add, over
    exactly the keys each branch attends to (masked work not counted)."""
    p = positions(prob)
    bc = prob["block"]                      # summaries
    bs = prob.get("sel_block", 0) or bc     # selection blocks
    n, w = prob["top_k"], prob["window"]
    H, dq, dv = prob["n_groups"] * prob["heads_per_group"], prob["d_qk"], prob["d_v"]
    per_key = 2.0 * (dq + dv) * H * prob["batch"]
    nvis_c = np.minimum((p + 1) // bc, prob["kv_len"] // bc)
    nvis = np.minimum((p + 1) // bs, prob["kv_len"] // bs)
    cur = p // bs
    first, current = bool(prob["force_first"]), bool(prob["force_current"])
    n_forced = np.full_like(p, int(first) + int(current))
    if first and current:
        n_forced[cur == 0] = 1
    forced_visible = (int(first) * (nvis >= 1)) + (int(current) * (cur < nvis))
    if first and current:
        forced_visible = np.where(cur == 0, (nvis >= 1).astype(np.int64), forced_visible)
    chosen = n_forced + np.minimum(n - n_forced, nvis - forced_visible)
    cur_in = np.full(p.shape, current) | ((cur == 0) & first)
    sel_keys = bs * chosen - np.where(cur_in, bs - (p % bs + 1), 0)
    win_keys = np.minimum(w, p + 1) if (prob["use_win"] and w > 0) else np.zeros_like(p)
    return {
        "cmp": per_key * float(nvis_c.sum()) if prob["use_cmp"] else 0.0,
        "slc": per_key * float(sel_keys.sum()),
        "win": per_key * float(win_keys.sum()),
    }


# ---------------------------------------------------------------- prefill --

def run_prefill(args, torch, nsa, workloads, inputs, workload=None):
    workload = workload or args.workload
    prob = workloads.get(workload)
    log(f"workload {workload}: generating inputs")
    t0 = time.time()
    x = inputs.generate(prob)
    log(f"inputs ready in {time.time() - t0:.1f}s; uploading")
    t = {k: nsa.to_device(a, prob) for k, a in x.items()}
    ws = nsa.alloc_workspace(prob)
    out = torch.empty((1, prob["q_len"], workloads.n_heads(prob), prob["d_v"]), dtype=torch.bfloat16, device="cuda")
    phases = nsa.forward_phases(prob)
    K, W = args.steps, args.warmup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(K)]
    for i in range(W):
        nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"], out=out, workspace=ws)
    torch.cuda.synchronize()
    log(f"warmup done ({W} steps); timing {K} steps")
    t0 = time.perf_counter()
    for i in range(K):
        nsa.forward(prob, t["q"], t["k"], t["v"], t["gates"], out=out, workspace=ws, events=ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_phase = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)]))
                 for j, name in enumerate(phases)}
    return prob, x, wall / K * 1e3, per_phase


def moba_kernel_flops(prob):
    """Algorithmic FLOPs of the two MoBA attention kernels: the chosen blocks
    before the query's own (whole blocks) and the own block (causal part)."""
    p = positions(prob)
    bs, n = prob["block"], prob["top_k"]
    H, dq, dv = prob["n_groups"] * prob["heads_per_group"], prob["d_qk"], prob["d_v"]
    per_key = 2.0 * (dq + dv) * H * prob["batch"]
    nvis = np.minimum((p + 1) // bs, prob["kv_len"] // bs)
    cur = p // bs
    first, current = bool(prob["force_first"]), bool(prob["force_current"])
    forced_earlier = np.where(first & (cur > 0), 1, 0)             # block 0 before the own block
    own = np.full(p.shape, current) | ((cur == 0) & first)
    cand = nvis - forced_earlier - np.where(current & (cur < nvis), 1, 0)
    earlier = forced_earlier + np.minimum(n - forced_earlier - own.astype(np.int64), cand)
    return {"moba_attn": per_key * bs * float(earlier.sum()),
            "moba_own_block": per_key * float(np.where(own, p % bs + 1, 0).sum())}


def load_traffic(kernel, workload):
    """Bytes per launch from the committed counter summary of this kernel and
    workload, or None when there is none or the kernel's sources changed."""
    from long_context_dynamic_amd import pmc
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != pmc.source_hash(kernel):
        log(f"{path}: kernel sources changed since the counters were taken; traffic not reported")
        return None
    return int(round(rec["traffic_bytes_per_launch"]))


def load_counters(kernel, workload):
    """The committed counter summary of this kernel and workload (matrix-op
    utilisation and FLOP, VALU busy, waits; mean per dispatch), or None when
    there is none or the kernel's sources changed since it was taken."""
    from long_context_dynamic_amd import pmc
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != pmc.source_hash(kernel):
        log(f"{path}: kernel sources changed since the counters were taken; counters not reported")
        return None
    out = {k: round(v, 4) for k, v in rec["counters"].items()}
    if "executed_over_algorithmic" in rec:
        out["mfma_flop_executed_over_algorithmic"] = round(rec["executed_over_algorithmic"], 4)
    return out


def roofline(kernel_flops, per_phase, workload):
    dominant = max((k for k in per_phase if k in kernel_flops), key=lambda k: per_phase[k])
    ms = per_phase[dominant]
    achieved = kernel_flops[dominant] / (ms * 1e-3) / 1e12
    return {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(dominant, workload), "traffic_unit": "HBM bytes per launch",
            "algorithmic_flop_per_launch": kernel_flops[dominant], "kernel_ms": round(ms, 4),
            "counters": load_counters(dominant, workload),
            "other_kernels_counters": {k: c for k in list(kernel_flops) + ["selected_merge"] if k != dominant
                                       for c in [load_counters(k, workload)] if c is not None},
            "other_kernels_traffic": {k: t for k in list(kernel_flops) + ["selected_merge"] if k != dominant
                                      for t in [load_traffic(k, workload)] if t is not None}}


def prefill_roofline(prob, per_phase, workload):
    fl = algorithmic_flops(prob)
    kernel_flops = {"selected": fl["slc"], "cmp_select_window": fl["cmp"] + fl["win"]}
    roof = roofline(kernel_flops, per_phase, workload)
    # the selected branch is two kernels: the per-stripe partials (the
    # dominant kernel above) and their merge with the gated sum
    if "selected_merge" in per_phase:
        ms = per_phase["selected"] + per_phase["selected_merge"]
        tf = fl["slc"] / (ms * 1e-3) / 1e12
        roof["selected_branch"] = {"kernels": ["selected", "selected_merge"], "ms": round(ms, 4),
                                   "achieved": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return roof, fl


def run_moba(args, torch, nsa, workloads, inputs, workload="moba_32k"):
    prob, x, ms, per_phase = run_prefill(args, torch, nsa, workloads, inputs, workload=workload)
    kf = moba_kernel_flops(prob)
    tokens = prob["batch"] * prob["q_len"]
    return {"workload": workload, "batch": prob["batch"], "seq_len": prob["q_len"],
            "heads": prob["n_groups"], "d": prob["d_qk"], "block": prob["block"], "top_k": prob["top_k"],
            "ms_per_step": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "phases_ms": {k: round(v, 4) for k, v in per_phase.items()},
            "algorithmic_tflop": {k: round(v / 1e12, 4) for k, v in kf.items()},
            "forward_mfma_frac": round(sum(kf.values()) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "roofline": roofline(kf, per_phase, workload)}


def run_side_leg(args, torch, nsa, workloads, inputs, workload, fn):
    """A further configuration measured the same way with fewer steps."""
    import copy
    a = copy.copy(args)
    a.steps, a.warmup = min(args.steps, 3), 1
    rec = fn(a, torch, nsa, workloads, inputs, workload)
    rec["steps"], rec["warmup"] = a.steps, a.warmup
    torch.cuda.empty_cache()
    return rec


def run_nsa_leg(args, torch, nsa, workloads, inputs, workload):
    prob, x, ms, per_phase = run_prefill(args, torch, nsa, workloads, inputs, workload=workload)
    roof, fl = prefill_roofline(prob, per_phase, workload)
    tokens = prob["batch"] * prob["q_len"]
    return {"workload": workload, "block": prob["block"], "sel_block": prob.get("sel_block", 0) or prob["block"],
            "ms_per_step": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "phases_ms": {k: round(v, 4) for k, v in per_phase.items()},
            "algorithmic_tflop": {k: round(v / 1e12, 4) for k, v in fl.items()},
            "forward_mfma_frac": round(sum(fl.values()) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "roofline": roof}


# --------------------------------------------------------------- backward --

def backward_kernel_flops(prob):
    """Algorithmic FLOPs of the backward per kernel group: five products per
    attended (key, head) -- S = q.k, dP = dout.v, dq, dk, dv -- over exactly
    the keys of each branch.  The query side (dq) is charged S, dP and dq;
    each branch's key side its dk and dv."""
    fl = algorithmic_flops(prob)  # 2 (dq + dv) per key and head
    dq, dv = prob["d_qk"], prob["d_v"]
    keys = {b: f / (2.0 * (dq + dv)) for b, f in fl.items()}  # key-head pairs per branch
    out = {"bwd_q": sum(keys.values()) * 2.0 * (2 * dq + dv)}
    for b, name in (("cmp", "bwd_kv_compressed"), ("slc", "bwd_kv_selected"), ("win", "bwd_kv_window")):
        if keys[b] > 0:
            out[name] = keys[b] * 2.0 * (dq + dv)
    return out


def run_backward(args, torch, nsa, workloads, inputs, workload="nsa_prefill_64k"):
    """nsa_backward on the workload's own selection (from nsa_select_topk)."""
    prob = workloads.get(workload)
    log(f"backward {workload}: generating inputs")
    x = inputs.generate(prob, want=("q", "k", "v", "gates", "dout"))
    t = {k: nsa.to_device(a, prob) for k, a in x.items()}
    del x
    kc, _ = nsa.compress(prob, t["k"], t["v"])
    idx, _ = nsa.select_topk(prob, t["q"], kc, want_score=False)
    del kc
    ws = torch.empty(nsa.backward_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    f32 = torch.float32
    B, T, L, G, H = prob["batch"], prob["q_len"], prob["kv_len"], prob["n_groups"], workloads.n_heads(prob)
    dq = torch.empty((B, T, H, prob["d_qk"]), dtype=f32, device="cuda")
    dk = torch.empty((B, L, G, prob["d_qk"]), dtype=f32, device="cuda")
    dv = torch.empty((B, L, G, prob["d_v"]), dtype=f32, device="cuda")
    dg = torch.empty((B, T, H, 3), dtype=f32, device="cuda")
    phases = nsa.backward_phases(prob)
    K, W = args.steps, args.warmup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(K)]

    def step(events=None):
        nsa.backward(prob, t["q"], t["k"], t["v"], t["gates"], idx, t["dout"], dq=dq, dk=dk, dv=dv, dgates=dg,
                     workspace=ws, events=events)
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(ev[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / K * 1e3
    per_phase = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)]))
                 for j, name in enumerate(phases)}
    kf = backward_kernel_flops(prob)
    tokens = B * T
    rec = {"workload": workload, "ms_per_step": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
           "steps": K, "warmup": W, "phases_ms": {k: round(v, 4) for k, v in per_phase.items()},
           "algorithmic_tflop": {k: round(v / 1e12, 4) for k, v in kf.items()},
           "backward_mfma_frac": round(sum(kf.values()) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "roofline": roofline(kf, per_phase, workload),
           "note": "gradients of the whole forward on its selection: dq, dk, dv (fp32), dgates"}
    del idx
    rec["training_step"] = run_training_step(args, torch, nsa, prob, t, ws, dq, dk, dv, dg, phases)
    del t, ws, dq, dk, dv, dg
    torch.cuda.empty_cache()
    return rec


def run_training_step(args, torch, nsa, prob, t, bws, dq, dk, dv, dg, phases):
    """One training step of the attention: nsa_forward_train (output,
    selection and the per-branch statistics) then nsa_backward reading those
    statistics, each timed with HIP events on the current stream."""
    B, T, H = prob["batch"], prob["q_len"], prob["n_groups"] * prob["heads_per_group"]
    out = torch.empty((B, T, H, prob["d_v"]), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, T, prob["n_groups"], prob["top_k"]), dtype=torch.int32, device="cuda")
    saved = torch.empty(nsa.train_saved_bytes(prob), dtype=torch.uint8, device="cuda")
    fws = nsa.alloc_workspace(prob)
    K, W = args.steps, args.warmup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(K)]
    fe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]

    def fwd():
        nsa.forward_train(prob, t["q"], t["k"], t["v"], t["gates"], out=out, idx=idx, saved=saved, workspace=fws)

    def bwd(events=None):
        nsa.backward(prob, t["q"], t["k"], t["v"], t["gates"], idx, t["dout"], dq=dq, dk=dk, dv=dv, dgates=dg,
                     workspace=bws, events=events, saved=saved)
    for _ in range(W):
        fwd()
        bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        fe[i][0].record()
        fwd()
        fe[i][1].record()
        bwd(ev[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / K * 1e3
    f_ms = float(np.mean([fe[i][0].elapsed_time(fe[i][1]) for i in range(K)]))
    per_phase = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)]))
                 for j, name in enumerate(phases)}
    b_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(K)]))
    del out, idx, saved, fws
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "forward_train_ms": round(f_ms, 4), "backward_from_saved_ms": round(b_ms, 4),
            "backward_phases_ms": {k: round(v, 4) for k, v in per_phase.items()},
            "saved_bytes": nsa.train_saved_bytes(prob),
            "note": "forward keeping per-branch log-sum-exp and bf16 outputs, backward reading them"}


# ---------------------------------------------------------------- learned --

def run_learned(args, torch, nsa, workloads, inputs, workload="nsa_prefill_64k", d_hidden=192, d_model=2560):
    """The learned block compression (MLP per 64-token block, hidden width
    d_hidden) and the gate projection (d_model 2560, the pages' hidden size)
    for the workload, each timed alone with HIP events."""
    prob = workloads.get(workload)
    x = inputs.generate(prob, want=("k", "v"))
    w = inputs.learned_weights(prob, d_hidden, d_model=d_model, seed=0)
    dev = lambda a: None if a is None else nsa.to_device(a, prob)
    k, v = dev(x["k"]), dev(x["v"])
    wk = {n: dev(a) for n, a in w["k"].items()}
    wv = {n: dev(a) for n, a in w["v"].items()}
    xs, gw, gb = dev(w["x"]), dev(w["gate_w"]), dev(w["gate_b"])
    del x, w
    kc, vc = nsa.compress_mlp(prob, k, v, wk, wv)
    gates = nsa.gate_proj(prob, xs, gw, gb)
    K = max(3, min(args.steps, 10))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K
    ms_mlp = timed(lambda: nsa.compress_mlp(prob, k, v, wk, wv, kc=kc, vc=vc))
    ms_gate = timed(lambda: nsa.gate_proj(prob, xs, gw, gb, gates=gates))
    B, L, G, bs, nb = prob["batch"], prob["kv_len"], prob["n_groups"], prob["block"], prob["kv_len"] // prob["block"]
    rows = B * nb * G
    fl_mlp = sum(2.0 * rows * (bs * d * d_hidden + d_hidden * d) for d in (prob["d_qk"], prob["d_v"]))
    M, N = B * prob["q_len"], 3 * workloads.n_heads(prob)
    fl_gate = 2.0 * M * d_model * N
    by_gate = 2.0 * (M * d_model + N * d_model + M * N)
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    del k, v, wk, wv, xs, gw, gb, kc, vc, gates
    torch.cuda.empty_cache()
    return {"workload": workload, "d_hidden": d_hidden, "d_model": d_model, "steps": K,
            "compress_mlp": {"ms": round(ms_mlp, 4), "algorithmic_gflop": round(fl_mlp / 1e9, 2),
                             "tflops": round(tf(fl_mlp, ms_mlp), 1),
                             "mfma_frac": round(tf(fl_mlp, ms_mlp) / PEAK_BF16_TFLOPS, 4)},
            "gate_proj": {"ms": round(ms_gate, 4), "algorithmic_gflop": round(fl_gate / 1e9, 2),
                          "tflops": round(tf(fl_gate, ms_gate), 1),
                          "mfma_frac": round(tf(fl_gate, ms_gate) / PEAK_BF16_TFLOPS, 4),
                          "hbm_gbs": round(by_gate / (ms_gate * 1e-3) / 1e9, 1),
                          "hbm_frac": round(by_gate / (ms_gate * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}


# ----------------------------------------------------------------- decode --

def run_decode(args, torch, nsa, workloads, inputs):
    import concurrent.futures as cf
    prob = workloads.get("nsa_decode_64x64k")
    B, L, G, dq, dv = prob["batch"], prob["kv_len"], prob["n_groups"], prob["d_qk"], prob["d_v"]
    H = workloads.n_heads(prob)
    log("decode: generating 64 x 65536-token caches")
    t0 = time.time()
    dev = {"q": torch.empty((B, 1, H, dq), dtype=torch.bfloat16, device="cuda"),
           "k": torch.empty((B, L, G, dq), dtype=torch.bfloat16, device="cuda"),
           "v": torch.empty((B, L, G, dv), dtype=torch.bfloat16, device="cuda"),
           "gates": torch.empty((B, 1, H, 3), dtype=torch.bfloat16, device="cuda")}
    with cf.ThreadPoolExecutor(16) as pool:
        for b in range(B):
            xs = inputs.generate_sequence(prob, b, pool=pool)
            for name, arr in xs.items():
                dev[name][b:b + 1].copy_(nsa.to_device(arr, prob))
    torch.cuda.synchronize()
    log(f"decode inputs ready in {time.time() - t0:.1f}s")
    kc, vc = nsa.compress(prob, dev["k"], dev["v"])
    ws = nsa.alloc_workspace(prob, have_cmp=True)
    out = torch.empty((B, 1, H, dv), dtype=torch.bfloat16, device="cuda")
    idx, _ = nsa.select_topk(prob, dev["q"], kc, want_score=False)
    # evicting the 256 MB last-level cache between steps: a read-only pass
    # over 512 MiB, so no dirty lines are left to be written back during the
    # timed step
    flush = torch.ones(128 * 2 ** 20, dtype=torch.int32, device="cuda")
    phases = nsa.forward_phases(prob, have_cmp=True)
    K = args.steps if args.only else max(args.steps, 10)
    times = []
    per_phase = {n: [] for n in phases}
    for i in range(args.warmup + K):
        flush.max()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
        nsa.forward(prob, dev["q"], dev["k"], dev["v"], dev["gates"], out=out, k_cmp=kc, v_cmp=vc,
                    workspace=ws, events=evs)
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(evs[0].elapsed_time(evs[-1]))
            for j, n in enumerate(phases):
                per_phase[n].append(evs[j].elapsed_time(evs[j + 1]))
    ms = float(np.median(times))
    # algorithmic bytes: summaries, the union of selected and window blocks, q, gates, out
    sel = idx.cpu().numpy()[:, 0]  # [B, G, n]
    p = L - 1
    win_blocks = set(range(max(0, p - prob["window"] + 1) // 64, p // 64 + 1))
    nblk = sum(len(set(int(j) for j in sel[b, g] if j >= 0) | win_blocks) for b in range(B) for g in range(G))
    nb = L // 64
    byts = (B * G * nb * (dq + dv) * 2 + nblk * 64 * (dq + dv) * 2 + B * H * (dq + 3 + dv) * 2)
    achieved = byts / (ms * 1e-3) / 1e9
    return {"workload": "nsa_decode_64x64k", "batch": B, "kv_len": L, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(B / (ms * 1e-3), 1),
            "phases_ms": {n: round(float(np.median(v)), 4) for n, v in per_phase.items()},
            "roofline": {"kernel": "whole decode step", "bound": "hbm", "achieved": round(achieved, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic("dec_step", "nsa_decode_64x64k"),
                         "traffic_unit": "HBM bytes per launch",
                         "algorithmic_bytes_per_step": int(byts),
                         "counters": load_counters("dec_step", "nsa_decode_64x64k")},
            "timing": "median of per-step HIP-event times; a 512 MiB read pass between steps evicts the last-level cache"}


def run_decode_variants(args, torch, nsa, workloads):
    """Where the decode step's time goes, from the public call alone: the
    64 x 64k step with branches switched off by their flags, at other batch
    sizes and cache lengths (seeded normal inputs; kernel time by HIP events,
    the last-level cache flushed before each step).  Printed, not part of
    the JSON line."""
    base = workloads.get("nsa_decode_64x64k")
    flush = torch.ones(128 * 2 ** 20, dtype=torch.int32, device="cuda")

    def timed(prob, steps):
        B, L, G, dq, dv = prob["batch"], prob["kv_len"], prob["n_groups"], prob["d_qk"], prob["d_v"]
        H = workloads.n_heads(prob)
        gen = torch.Generator(device="cuda").manual_seed(0)
        q = torch.randn((B, 1, H, dq), generator=gen, device="cuda").to(torch.bfloat16)
        k = torch.randn((B, L, G, dq), generator=gen, device="cuda").to(torch.bfloat16)
        v = torch.randn((B, L, G, dv), generator=gen, device="cuda").to(torch.bfloat16)
        gates = torch.rand((B, 1, H, 3), generator=gen, device="cuda").to(torch.bfloat16)
        kc, vc = nsa.compress(prob, k, v)
        ws = nsa.alloc_workspace(prob, have_cmp=True)
        out = torch.empty((B, 1, H, dv), dtype=torch.bfloat16, device="cuda")
        ts = []
        for i in range(steps + 3):
            flush.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            nsa.forward(prob, q, k, v, gates, out=out, k_cmp=kc, v_cmp=vc, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            if i >= 3:
                ts.append(e0.elapsed_time(e1) * 1e3)
        del q, k, v, kc, vc, ws, out
        torch.cuda.empty_cache()
        return round(float(np.median(ts)), 1)

    res = {}
    for label, kw in (("full", {}), ("no window", {"use_win": 0}), ("no selected", {"use_slc": 0}),
                      ("compressed only", {"use_win": 0, "use_slc": 0}), ("batch 32", {"batch": 32}),
                      ("batch 128", {"batch": 128}), ("top-4", {"top_k": 4}), ("top-8", {"top_k": 8})):
        res[label] = timed(dict(base, **kw), args.steps)
        log(f"decode {label}: {res[label]} us")
    for L in (16384, 32768, 131072):
        res[f"kv_len {L}"] = timed(dict(base, kv_len=L), args.steps)
        res[f"kv_len {L} compressed only"] = timed(dict(base, kv_len=L, use_win=0, use_slc=0), args.steps)
        log(f"decode kv_len {L}: {res[f'kv_len {L}']} us, compressed only {res[f'kv_len {L} compressed only']} us")
    return res


# -------------------------------------------------------------- cpu oracle --

def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo, as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(prob, x, target_s=15.0):
    import oracle
    T = prob["q_len"]
    t0 = time.perf_counter()
    kc, vc = oracle.pool(prob, x["k"], x["v"])
    t_pool = time.perf_counter() - t0

    def timed(rows):
        s = time.perf_counter()
        idx, _, ocmp = oracle.select(prob, x["q"], kc, vc, rows=rows, want_imp=False)
        oracle.attend(prob, x["q"], x["k"], x["v"], x["gates"], idx, ocmp, rows=rows)
        return time.perf_counter() - s

    probe = np.linspace(0, T - 1, 16).astype(np.int64)
    t_probe = timed(probe)
    n = int(np.clip(target_s / max(t_probe / len(probe), 1e-6), 16, T))
    rows = np.linspace(0, T - 1, n).astype(np.int64)
    t_rows = timed(rows)
    secs = t_rows + t_pool * n / T
    return {"value": round(n / secs, 2), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n} query rows evenly spaced over the {T}-token sequence (all 64 heads each); "
                      f"pooling of the whole sequence ({t_pool:.2f}s) prorated by {n}/{T}",
            "seconds": round(t_rows + t_pool, 2)}


# ---------------------------------------------------------------- ceilings --

def run_ceilings(torch):
    """Reference rates measured on this chip: a 1 GiB device copy, and random
    whole 40 KiB block gathers (the selected branch's access pattern: K and V
    of 64 keys at d 192 / 128) with ordinary loads from tables of 2.5 MiB
    (fits each XCD's 4 MB L2), 10 MiB, 40 MiB (one group's K and V at 64k),
    160 MiB (fits the 256 MB last-level cache) and 1.25 GiB (does not), and
    with non-temporal loads from 1.25 GiB."""
    probe = _probe_lib()
    res = {}
    a = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    res["copy_1GiB_GBps"] = round(2 * 2 ** 30 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    stream = torch.cuda.current_stream().cuda_stream
    waves, per_wave = 262144, 4
    out = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    gen = torch.Generator().manual_seed(0)
    for nblk, label, nt in ((64, "2.5MiB", 0), (256, "10MiB", 0), (1024, "40MiB", 0), (4096, "160MiB", 0),
                            (32768, "1280MiB", 0), (32768, "1280MiB_nontemporal", 1)):
        table = torch.ones(nblk * 40960 // 4, dtype=torch.int32, device="cuda")
        pick = torch.randint(0, nblk, (2 ** 20,), generator=gen, dtype=torch.int32).cuda()
        args = (table.data_ptr(), pick.data_ptr(), pick.numel(), out.data_ptr(), waves, per_wave, nt, stream)
        if probe.nsa_probe_gather(*args) != 0:
            raise RuntimeError("gather probe launch failed")
        e0.record()
        if probe.nsa_probe_gather(*args) != 0:
            raise RuntimeError("gather probe launch failed")
        e1.record()
        torch.cuda.synchronize()
        res[f"gather_40KiB_blocks_{label}_TBps"] = round(waves * per_wave * 40960 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 2)
        del table, pick
    return res


GATHER_CAL = {"blocks": 32768, "waves": 262144, "per_wave": 4}  # 1.25 GiB table: read from HBM


def _probe_lib():
    import ctypes
    from long_context_dynamic_amd import build as nsa_build
    if not os.path.exists(nsa_build.PROBE_LIB):
        raise RuntimeError(f"{nsa_build.PROBE_LIB} is not built (python -m long_context_dynamic_amd.build)")
    probe = ctypes.CDLL(nsa_build.PROBE_LIB)
    probe.nsa_probe_gather.restype = ctypes.c_int
    probe.nsa_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return probe


def run_gather_calibration(torch, launches):
    """Launches of the read-only block gather over a 1.25 GiB table (larger
    than the last-level cache): a kernel whose HBM read bytes are known
    (waves x blocks per wave x 40 KiB, nothing written but 256 bytes per
    wave) and whose access pattern is the selected branch's and the decode's
    -- whole 40 KiB blocks at random -- so its FETCH_SIZE counter calibrates
    theirs.  Returns the bytes read per launch."""
    probe = _probe_lib()
    c = GATHER_CAL
    table = torch.ones(c["blocks"] * 40960 // 4, dtype=torch.int32, device="cuda")
    gen = torch.Generator().manual_seed(0)
    pick = torch.randint(0, c["blocks"], (2 ** 20,), generator=gen, dtype=torch.int32).cuda()
    out = torch.empty(c["waves"] * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(max(1, launches)):
        if probe.nsa_probe_gather(table.data_ptr(), pick.data_ptr(), pick.numel(), out.data_ptr(), c["waves"],
                                  c["per_wave"], 0, stream) != 0:
            raise RuntimeError("gather probe launch failed")
    torch.cuda.synchronize()
    return c["waves"] * c["per_wave"] * 40960


# ------------------------------------------------------- profiling legs --

def run_only(args, torch, nsa, workloads, inputs):
    """One leg for a profiler: prefill or decode steps, or a plain 1 GiB
    device copy whose byte counters calibrate the others'."""
    if args.only == "ceilings":
        log(f"ceilings {run_ceilings(torch)}")
    elif args.only == "decode_variants":
        log(f"decode variants (us) {run_decode_variants(args, torch, nsa, workloads)}")
    elif args.only == "gather":
        log(f"gathered {run_gather_calibration(torch, args.steps)} bytes per launch")
    elif args.only == "copy":
        a = torch.empty(2 ** 30, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied 1 GiB x {args.steps}")
    elif args.only == "learned":
        log(f"learned {run_learned(args, torch, nsa, workloads, inputs, args.workload)}")
    elif args.only == "backward":
        rec = run_backward(args, torch, nsa, workloads, inputs, args.workload)
        log(f"backward {rec['ms_per_step']} ms/step {rec['phases_ms']}")
        log(f"training step {rec['training_step']}")
    elif args.only == "prefill":
        args.steps, args.warmup = max(1, args.steps), args.warmup
        _, _, ms, per_phase = run_prefill(args, torch, nsa, workloads, inputs)
        log(f"prefill {ms:.3f} ms/step {per_phase}")
    else:
        rec = run_decode(args, torch, nsa, workloads, inputs)
        log(f"decode {rec['ms_per_step']} ms/step {rec['phases_ms']}")


# ------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="nsa_prefill_64k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-moba", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip MoBA 128k/1M and the decoupled-block 64k legs")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "decode_variants", "copy", "gather", "ceilings",
                                       "backward", "learned"],
                    default=None,
                    help="profiling runs: one leg only, no JSON contract line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path runs on a single "
              "MI355X and its multi-GPU sharding is a design note, not a measured mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_dynamic_amd import inputs, nsa, workloads
    torch.cuda.set_device(0)
    nsa.lib()
    if args.only:
        run_only(args, torch, nsa, workloads, inputs)
        return

    prob, x, ms, per_phase = run_prefill(args, torch, nsa, workloads, inputs)
    roof, fl = prefill_roofline(prob, per_phase, args.workload)
    f_tot = fl["cmp"] + fl["slc"] + fl["win"]
    tokens = prob["batch"] * prob["q_len"]
    rec = {
        "metric": METRIC, "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64: q,k,v ~ N(0,1), per-block key offset N(0,0.5^2), gates ~ U(0,1))",
        "config": {"workload": args.workload, "batch": prob["batch"], "seq_len": prob["q_len"],
                   "kv_groups": prob["n_groups"], "heads_per_group": prob["heads_per_group"],
                   "d_qk": prob["d_qk"], "d_v": prob["d_v"], "block": prob["block"], "top_k": prob["top_k"],
                   "window": prob["window"]},
        "phases_ms": {k: round(v, 4) for k, v in per_phase.items()},
        "algorithmic_tflop": {k: round(v / 1e12, 4) for k, v in fl.items()},
        "forward_mfma_frac": round(f_tot / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "context_from_pages": PAGE_CONTEXT,
    }
    log(f"prefill: {ms:.3f} ms/step, phases {rec['phases_ms']}")
    del x  # host inputs of the 64k workload; made again for the CPU baseline
    torch.cuda.empty_cache()
    if not args.no_moba:
        rec["moba"] = run_moba(args, torch, nsa, workloads, inputs)
        log(f"moba: {rec['moba']['ms_per_step']} ms/step, phases {rec['moba']['phases_ms']}")
        torch.cuda.empty_cache()
    if not args.no_extra:
        # MoBA at longer contexts, and the 64k prefill with decoupled block sizes
        for wl, fn in (("nsa_prefill_8k", run_nsa_leg), ("moba_128k", run_moba), ("moba_1m", run_moba),
                       ("nsa_prefill_64k_c32", run_nsa_leg)):
            rec.setdefault("more_configs", {})[wl] = run_side_leg(args, torch, nsa, workloads, inputs, wl, fn)
            log(f"{wl}: {rec['more_configs'][wl]['ms_per_step']} ms/step")
    if not args.no_backward:
        a = __import__("copy").copy(args)
        a.steps, a.warmup = min(args.steps, 3), 1
        rec["backward"] = run_backward(a, torch, nsa, workloads, inputs, args.workload)
        log(f"backward: {rec['backward']['ms_per_step']} ms/step, phases {rec['backward']['phases_ms']}")
    if not args.no_backward:
        rec["learned"] = run_learned(args, torch, nsa, workloads, inputs, args.workload)
        log(f"learned: {rec['learned']}")
    if not args.no_decode:
        rec["decode"] = run_decode(args, torch, nsa, workloads, inputs)
        log(f"decode: {rec['decode']['ms_per_step']} ms/step")
        torch.cuda.empty_cache()
    rec["measured_ceilings"] = run_ceilings(torch)
    log(f"ceilings: {rec['measured_ceilings']}")
    if not args.no_cpu:
        log("cpu baseline: timing the oracle on a sample")
        rec["cpu_baseline"] = run_cpu_baseline(prob, inputs.generate(prob))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
