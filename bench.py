"""Benchmark of the hybrid-attention hot path on one MI355X.

Step (the timed unit, the headline): the Gemma-4-31B global-layer prefill of one 8192-token
sequence (32 q / 4 KV heads, head dim 512, one tensor as K and V, full causal): the q/k
prologue (RMSNorm + partial p-RoPE, out of place) followed by the attention kernel. The
JSON line's `value` is masked attention TFLOP/s of the whole step (4 * Hq * D * visible
pairs per second); `roofline` is the attention kernel alone, timed with HIP events on its
stream. The same run measures, under "extra": the sliding-layer step (2 x 4096), chunked
and image prefill, decode against prologue-filled KV caches (64 sequences, context lengths
uniform in [1024, 32768]) on both layer types, and the two prefills with peaked scores.
Inputs are synthetic (seeded N(0,1) bf16, norm weights N(1, 0.1)).

CPU baselines: the float64 numpy oracle, timed on the host cores on a bounded sample of
each workload (named in each `sample`), credited with the same algorithmic numerator.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# Chunk size (keys) of the split-form measurements of the global layer: prefill and decode
# must share it for their rows to agree. Of 4096 / 5120 / 6144 / 7168 / 8192, 6144 gives the
# fastest 64-sequence decode and, of the sizes that split an 8192-token prompt at all, the
# second-fastest prefill (two chunks, a quarter of the rows merged).
SPLIT_KEYS = 6144
KERNEL_SOURCES = ["global_gqa_attention_amd/csrc/attention.hip", "global_gqa_attention_amd/csrc/tile.hpp"]


def masked_pairs(L: int, window: int) -> int:
    if window <= 0 or window >= L:
        return L * (L + 1) // 2
    return window * (window + 1) // 2 + (L - window) * window


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name: str):
    """Per-launch HBM bytes of the attention kernel from a committed counter summary,
    if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def per_pass(bytes_per_launch, launches):
    return None if bytes_per_launch is None else bytes_per_launch * launches


class KernelTimer:
    """HIP events around every launch of one kernel on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.a = self.torch.cuda.Event(enable_timing=True)
        self.b = self.torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.pairs.append((self.a, self.b))

    def times_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]

    def mean_ms(self) -> float:
        return sum(self.times_ms()) / max(1, len(self.pairs))

    def spread(self) -> dict:
        """Median and minimum of the timed launches (ms), beside the mean the rates use."""
        t = sorted(self.times_ms())
        if not t:
            return {}
        mid = len(t) // 2
        med = t[mid] if len(t) % 2 else 0.5 * (t[mid - 1] + t[mid])
        return {"kernel_ms_median": round(med, 4), "kernel_ms_min": round(t[0], 4)}


def cpu_info():
    """(CPU model, threads the oracle's BLAS uses) of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    return model, cores


def prefill_step(args, torch, g, W, dev, spec, lens, seed, split_keys=0):
    """The prologue + attention step of one prefill workload: wall time per step over the
    timed steps (synchronised on both sides) and the attention kernel's HIP-event times.
    split_keys > 0: the split form (chunk work-groups and the merge, both inside the timed
    attention call)."""
    case = W.prefill_case(spec, lens, seed=seed, device=dev)
    layer = g.make_layer(spec)
    q, k = torch.empty_like(case.q), torch.empty_like(case.k)
    out = torch.empty_like(case.q)
    v = None if spec.k_eq_v else case.v
    # a layer with a value norm forms V in the prologue from the raw projection (the real
    # model's global layer: the k projection serves as both)
    v_raw = case.k if spec.v_norm else None
    if v_raw is not None:
        v = torch.empty_like(case.k)
    maxlen = max(lens)
    flops = 4.0 * spec.num_q_heads * spec.head_dim * sum(masked_pairs(L, spec.window) for L in lens)
    t = KernelTimer(torch)
    ws = None
    if split_keys:
        nbytes = g.g4attn_split_workspace_bytes(layer, len(lens), maxlen, maxlen, split_keys)
        ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=dev)

    def attend(provenance=False):
        if split_keys:
            return g.g4attn_prefill_split(layer, q, k, v, out, case.seq_start, case.seq_len, maxlen, split_keys, ws,
                                          provenance=provenance)
        return g.g4attn_prefill(layer, q, k, v, out, case.seq_start, case.seq_len, maxlen, provenance=provenance)

    def step(timer=None):
        g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions, v_in=v_raw,
                             v_out=v if v_raw is not None else None)
        if timer is None:
            attend()
        else:
            with timer:
                attend()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(t)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    prov = attend(provenance=True)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    return {"step_ms": step_ms, "value": flops / (step_ms * 1e-3) / 1e12, "flops": flops,
            "kernel": prov["kernel_id"], "kernel_ms": ms, "spread": t.spread(),
            "achieved": flops / (ms * 1e-3) / 1e12}


def run(args):
    import numpy as np
    import torch

    import global_gqa_attention_amd as g
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    torch.backends.cuda.matmul.allow_tf32 = False

    # ------------- the step: global-layer prefill, 1 x 8192, prologue + attention -------------
    spec = W.GLOBAL_31B
    st = prefill_step(args, torch, g, W, dev, spec, [8192], seed=2)
    log(f"global 1x8192 step: {st['step_ms']:.4f} ms, attention {st['kernel_ms']:.4f} ms")

    extra = {}
    if not args.skip_extra:
        extra = run_extra(args, torch, np, g, W, dev, headline=st)

    cpu = None if args.skip_cpu else cpu_baseline_global(np, W)
    line = {
        "metric": "prefill attention TFLOP/s (masked) + decode KV GB/s, % of MI355X roofline",
        "value": round(st["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gemma4-31b global-layer prefill: q/k prologue + attention, batch 1 x seq 8192, "
                               "32 q / 4 kv heads, head dim 512, K=V, full causal, p-RoPE on 128 of 512 dims",
                   "global_batch": 1, "seq_len": 8192, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(st["achieved"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(st["achieved"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile("prefill_global_1x8192_traffic.txt"),
                     "kernel": st["kernel"], "kernel_ms": round(st["kernel_ms"], 4), **st["spread"],
                     "algorithmic_flop_per_launch": st["flops"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def log(msg: str) -> None:
    """Progress on stderr (stdout carries the one JSON line)."""
    print(msg, file=sys.stderr, flush=True)


def measure_sliding_step(args, torch, np, g, W, dev):
    """Sliding-layer prefill step, 2 x 4096 packed: prologue + attention."""
    spec = W.SLIDING_31B
    st = prefill_step(args, torch, g, W, dev, spec, [4096, 4096], seed=1)
    res = {"value": round(st["value"], 2), "unit": "TFLOP/s", "ms_per_step": round(st["step_ms"], 4),
           "kernel_ms": round(st["kernel_ms"], 4), **st["spread"],
           "roofline": {"bound": "mfma", "achieved": round(st["achieved"], 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(st["achieved"] / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_from_profile("prefill_sliding_2x4096_traffic.txt"),
                        "kernel": st["kernel"]},
           "algorithmic_flop_per_launch": st["flops"]}
    return res, st


def measure_global_v_step(args, torch, np, g, W, dev):
    """The global-layer step (1 x 8192) with separate K and V as the real model forms them:
    the prologue turns the one raw projection into K (normed, rotated) and V (unit RMS
    norm), then the 512-dim attention over separate K and V (the split-ring kernel)."""
    spec = W.GLOBAL_31B_V
    st = prefill_step(args, torch, g, W, dev, spec, [8192], seed=2)
    return {"value": round(st["value"], 2), "unit": "TFLOP/s", "ms_per_step": round(st["step_ms"], 4),
            "kernel_ms": round(st["kernel_ms"], 4), **st["spread"],
            "roofline": {"bound": "mfma", "achieved": round(st["achieved"], 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(st["achieved"] / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profile("prefill_global_v_1x8192_traffic.txt"),
                         "kernel": st["kernel"]},
            "algorithmic_flop_per_launch": st["flops"]}


def measure_backward(args, torch, np, g, W, dev, which):
    """The deterministic attention backward (dq, dk, dv, lse, delta: the call's two
    launches, timed together with HIP events) on the prefill workload's inputs after the
    prologue, the forward's output and an N(0,1) output gradient. Credited with 2.5 x the
    forward's masked FLOPs (the five products over the visible pairs: the scores again,
    dO V^T, P^T dO, dS^T q and dS k)."""
    if which == "sliding":
        spec, lens, seed = W.SLIDING_31B, [4096, 4096], 1
    else:
        spec, lens, seed = W.GLOBAL_31B, [8192], 2
    case = W.prefill_case(spec, lens, seed=seed, device=dev)
    layer = g.make_layer(spec)
    q, k = torch.empty_like(case.q), torch.empty_like(case.k)
    g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions)
    v = None if spec.k_eq_v else case.v
    maxlen = max(lens)
    out = torch.empty_like(q)
    g.g4attn_prefill(layer, q, k, v, out, case.seq_start, case.seq_len, maxlen)
    dout = W.bf16_normal(W.make_generator(seed + 100, dev), q.shape, device=dev)
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv = None if spec.k_eq_v else torch.empty_like(k)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    flops = 2.5 * 4.0 * spec.num_q_heads * spec.head_dim * sum(masked_pairs(L, spec.window) for L in lens)
    t = KernelTimer(torch)
    reps = max(3, args.steps // 4)
    for _ in range(max(3, args.warmup // 4)):
        g.g4attn_prefill_backward(layer, q, k, v, out, dout, dq, dk, dv, lse, delta, case.seq_start, case.seq_len, maxlen)
    for _ in range(reps):
        with t:
            g.g4attn_prefill_backward(layer, q, k, v, out, dout, dq, dk, dv, lse, delta, case.seq_start, case.seq_len,
                                      maxlen)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    tf = flops / (ms * 1e-3) / 1e12
    res = {"value": round(tf, 2), "unit": "TFLOP/s", "ms_per_call": round(ms, 4), **t.spread(),
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
           "algorithmic_flop_per_call": flops}
    if not args.skip_cpu and which == "global":
        res["cpu_baseline"] = cpu_baseline_backward(np, W)
    return res


def fill_decode_cache(torch, g, case):
    """The decode caches of a workloads.DecodeCase, filled as a serving engine fills them:
    the q/k prologue of every cached position writes k (and the raw v) into its cache row
    (kv_dst_row), and the new tokens' q go through the prologue at position ctx - 1.
    Returns (q, k_cache, v_cache) device tensors."""
    spec = case.spec
    dev = case.k_raw.device
    layer = g.make_layer(spec)
    Hk, D = spec.num_kv_heads, spec.head_dim
    kc = torch.zeros((case.cache_rows, Hk, D), dtype=torch.bfloat16, device=dev)
    vc = None if spec.k_eq_v else torch.zeros_like(kc)
    g.g4attn_qk_prologue(layer, None, None, case.k_raw, kc, None, case.wk, case.positions, v_in=case.v_raw, v_out=vc,
                         kv_dst_row=case.dst_row)
    qd = torch.empty_like(case.q_raw)
    qpos = torch.from_numpy(case.ctx - 1).to(dev)
    g.g4attn_qk_prologue(layer, case.q_raw, qd, None, None, case.wq, None, qpos)
    return qd, kc, vc


def decode_kv_bytes(spec, ctx, key_lo) -> int:
    """Algorithmic KV bytes of one decode launch: each visible key of every KV head read
    once, K and V (or the one K=V tensor)."""
    keys = int((ctx.astype("int64") - key_lo).sum())
    return keys * spec.num_kv_heads * spec.head_dim * 2 * (1 if spec.k_eq_v else 2)


def measure_decode(args, torch, np, g, W, dev, spec, split_keys=0):
    """Decode of 64 sequences (context lengths uniform in [1024, 32768], seed 3) against
    a sliding ring of 1024 slots (K and V) or a linear K=V cache, the caches filled by the
    prologue at the keys' true positions; KV-read GB/s. split_keys > 0: the split form
    (chunk work-groups and the merge, both inside each timed call)."""
    B = 64
    case = W.decode_case(spec, B, 1024, 32768, seed=3, device=dev)
    order = np.argsort(-case.ctx, kind="stable").astype(np.int32)
    layer = g.make_layer(spec)
    qd, kc, vc = fill_decode_cache(torch, g, case)
    od = torch.empty_like(qd)
    kv_bytes = decode_kv_bytes(spec, case.ctx, case.key_lo)
    row0_t = torch.from_numpy(case.row0).to(dev)
    ctx_t = torch.from_numpy(case.ctx).to(dev)
    sched = torch.from_numpy(order).to(dev)
    maxctx = int(case.ctx.max())
    ws = None
    if split_keys:
        nbytes = g.g4attn_split_workspace_bytes(layer, B, 1, maxctx, split_keys)
        ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=dev)

    def call():
        if split_keys:
            g.g4attn_decode_split(layer, qd, kc, vc, row0_t, ctx_t, case.slots, od, maxctx, split_keys, ws,
                                  schedule=sched)
        else:
            g.g4attn_decode(layer, qd, kc, vc, row0_t, ctx_t, case.slots, od, maxctx, schedule=sched)

    t = KernelTimer(torch)
    for _ in range(args.warmup):
        call()
    for _ in range(args.steps):
        with t:
            call()
    torch.cuda.synchronize()
    ms = t.mean_ms()
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    name = "decode_sliding_64seq" if spec.window > 0 else "decode_global_v_64seq" if spec.v_norm else \
        "decode_global_64seq"
    if split_keys:
        name += f"_split{split_keys}"
    res = {"value": round(gbs, 1), "unit": "GB/s", "kernel_ms": round(ms, 4), **t.spread(), "kv_bytes": kv_bytes,
           "caches": "filled by the q/k prologue at the keys' true positions",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": traffic_from_profile(name + "_traffic.txt")}}
    del kc, vc
    torch.cuda.empty_cache()
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_baseline_decode(np, W, case, split_keys=split_keys)
    return name, res


RESCALE_THRESHOLD = 64.0  # log2 units: a row's offset moves only past this (the kernels' lazy rule)


def rerun_fraction(torch, spec, q, k, lens, starts, scale, rows_per_group):
    """Estimated share of prefill work-groups that run their second pass. A row's exponent
    offset (log2 units) is set by its first visible 32-key block and moves only when a
    later block's largest visible score exceeds it by more than RESCALE_THRESHOLD; a
    work-group runs the second pass when any of its rows moves after holding keys. Scores
    come from an fp32 product of the same bf16 inputs, so rows right at the threshold may
    go the other way in the kernel's MFMA sums."""
    import math

    G = spec.group
    c = scale / math.log(2.0)
    groups = rerun = 0
    for s0, L in zip(starts, lens):
        nblk = (L + 31) // 32
        i = torch.arange(L, device=q.device)[:, None]
        j = torch.arange(nblk * 32, device=q.device)[None, :]
        hide = j > i
        if spec.window > 0:
            hide |= (i - j) >= spec.window
        ppg = rows_per_group // G
        for gk in range(spec.num_kv_heads):
            kk = torch.zeros((nblk * 32, spec.head_dim), device=q.device)
            kk[:L] = k[s0:s0 + L, gk].float()
            moved_pos = torch.zeros(L, dtype=torch.bool, device=q.device)
            for h in range(gk * G, (gk + 1) * G):
                s = (q[s0:s0 + L, h].float() @ kk.T) * c
                s.masked_fill_(hide, float("-inf"))
                bm = s.view(L, nblk, 32).amax(-1)
                del s
                m = torch.full((L,), float("-inf"), device=q.device)
                moved = torch.zeros(L, dtype=torch.bool, device=q.device)
                for jb in range(nblk):
                    t = bm[:, jb]
                    mv = t > m + RESCALE_THRESHOLD
                    moved |= mv & torch.isfinite(m)
                    m = torch.where(mv, t, m)
                moved_pos |= moved
            nq = (L + ppg - 1) // ppg
            pad = torch.zeros(nq * ppg, dtype=torch.bool, device=q.device)
            pad[:L] = moved_pos
            groups += nq
            rerun += int(pad.view(nq, ppg).any(1).sum().item())
    return rerun / groups


def measure_peaked(args, torch, np, g, W, dev, which, mode, plain_ms):
    """A prefill with peaked scores: the queries after the prologue multiplied by 24
    ("q24"), or the softmax scale 1.0 in place of 1/sqrt(D) ("scale1", the scale of
    transformers' Gemma 4 attention); attention kernel alone, masked FLOPs."""
    if which == "sliding":
        spec, lens, seed = W.SLIDING_31B, [4096, 4096], 1
    else:
        spec, lens, seed = W.GLOBAL_31B, [8192], 2
    case = W.prefill_case(spec, lens, seed=seed, device=dev)
    layer = g.make_layer(spec)
    scale = spec.softmax_scale
    if mode == "scale1":
        layer.softmax_scale = 1.0
        scale = 1.0
    q, k = torch.empty_like(case.q), torch.empty_like(case.k)
    g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions)
    if mode == "q24":
        q = (q.float() * 24.0).to(torch.bfloat16)
    out = torch.empty_like(q)
    v = None if spec.k_eq_v else case.v
    maxlen = max(lens)
    flops = 4.0 * spec.num_q_heads * spec.head_dim * sum(masked_pairs(L, spec.window) for L in lens)
    t = KernelTimer(torch)
    for _ in range(args.warmup):
        g.g4attn_prefill(layer, q, k, v, out, case.seq_start, case.seq_len, maxlen)
    for _ in range(args.steps):
        with t:
            g.g4attn_prefill(layer, q, k, v, out, case.seq_start, case.seq_len, maxlen)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    tf = flops / (ms * 1e-3) / 1e12
    rows = 128 if spec.head_dim >= 512 else 256
    frac = rerun_fraction(torch, spec, q, k, lens, case.seq_start.tolist(), scale, rows)
    return {"value": round(tf, 2), "unit": "TFLOP/s", "kernel_ms": round(ms, 4), **t.spread(),
            "slowdown_vs_plain": round(ms / plain_ms, 3), "workgroups_rerun_est": round(frac, 4),
            "inputs": "the plain measurement's inputs, " + ("queries x 24 after the prologue" if mode == "q24"
                                                             else "softmax scale 1.0"),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
            "algorithmic_flop_per_launch": flops}


def image_pairs(np, seq_lens, images, window: int) -> int:
    """Visible (query, key) pairs with per-row last keys: row i of a sequence sees keys
    max(0, i - window + 1) .. max(i, last_i) (an image's rows see up to its last row)."""
    tot = 0
    for L, imgs in zip(seq_lens, images):
        i = np.arange(L)
        last = np.full(L, -1)
        for a, n in imgs:
            last[a:a + n] = a + n - 1
        lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros(L, np.int64)
        tot += int((np.maximum(i, last) - lo + 1).sum())
    return tot


def measure_images(args, torch, np, g, W, dev):
    """The step's sliding-layer prefill (2 x 4096, same inputs) with images: four 256-row
    images per sequence at seeded positions (seed 5), whose rows see the whole image
    (g4attn_prefill_masked); attention kernel alone, masked FLOPs."""
    spec = W.SLIDING_31B
    lens = [4096, 4096]
    case = W.prefill_case(spec, lens, seed=1, device=dev)
    images = W.image_spans(lens, 256, 4, seed=5)
    last_key = W.image_last_keys(case.seq_start.cpu(), case.seq_len.cpu(), images, case.num_tokens).to(dev)
    layer = g.make_layer(spec)
    q, k = torch.empty_like(case.q), torch.empty_like(case.k)
    out = torch.empty_like(case.q)
    g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions)
    flops = 4.0 * spec.num_q_heads * spec.head_dim * image_pairs(np, lens, images, spec.window)
    t = KernelTimer(torch)
    for _ in range(args.warmup):
        g.g4attn_prefill_masked(layer, q, k, case.v, out, case.seq_start, case.seq_len, last_key, 4096)
    for _ in range(args.steps):
        with t:
            g.g4attn_prefill_masked(layer, q, k, case.v, out, case.seq_start, case.seq_len, last_key, 4096)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    tf = flops / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "kernel_ms": round(ms, 4), **t.spread(),
            "images": "4 per sequence, 256 rows each (seed 5)",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profile("prefill_sliding_2x4096_images_traffic.txt")},
            "algorithmic_flop_per_launch": flops}


def measure_chunked(args, torch, np, g, W, dev):
    """Chunked prefill of the step's workload (sliding layer, 2 x 4096 tokens) in 512-row
    chunks through a ring of window + 512 slots per sequence: per chunk the q/k prologue
    scatters the chunk's keys into the ring (untimed), then g4attn_prefill_cached runs the
    chunk's attention (timed with HIP events). TFLOP/s = the whole prefill's masked FLOP
    over the summed attention time of the 8 chunk calls."""
    spec = W.SLIDING_31B
    lens, C = [4096, 4096], 512
    case = W.prefill_case(spec, lens, seed=1, device=dev)
    layer = g.make_layer(spec)
    H, Hk, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    slots = spec.window + C
    kc = torch.zeros((2 * slots, Hk, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    row0 = torch.tensor([0, slots], dtype=torch.int64, device=dev)
    starts = case.seq_start.tolist()
    chunks = []
    for c in range(lens[0] // C):
        rows = torch.cat([torch.arange(s + c * C, s + (c + 1) * C, device=dev) for s in starts])
        pos = torch.arange(c * C, (c + 1) * C, dtype=torch.int32, device=dev).repeat(2)
        dst = torch.cat([r0 + torch.arange(c * C, (c + 1) * C, device=dev) % slots for r0 in (0, slots)])
        chunks.append(dict(q=case.q[rows].contiguous(), k=case.k[rows].contiguous(), v=case.v[rows].contiguous(),
                           pos=pos, dst=dst.to(torch.int64), qc=torch.empty((2 * C, H, D), dtype=torch.bfloat16,
                                                                            device=dev),
                           qr=torch.tensor([0, C], dtype=torch.int32, device=dev),
                           qp=torch.tensor([c * C, c * C], dtype=torch.int32, device=dev),
                           cl=torch.tensor([C, C], dtype=torch.int32, device=dev), key_len=(c + 1) * C))
    out = torch.empty((2 * C, H, D), dtype=torch.bfloat16, device=dev)
    t = KernelTimer(torch)

    def one_pass(timer=None):
        for ch in chunks:
            g.g4attn_qk_prologue(layer, ch["q"], ch["qc"], ch["k"], kc, case.wq, case.wk, ch["pos"], v_in=ch["v"],
                                 v_out=vc, kv_dst_row=ch["dst"])
            if timer is None:
                g.g4attn_prefill_cached(layer, ch["qc"], kc, vc, out, ch["qr"], ch["qp"], ch["cl"], row0, slots, C,
                                        ch["key_len"])
            else:
                with timer:
                    g.g4attn_prefill_cached(layer, ch["qc"], kc, vc, out, ch["qr"], ch["qp"], ch["cl"], row0, slots,
                                            C, ch["key_len"])

    passes_w = max(1, args.warmup // len(chunks))
    passes_t = max(1, args.steps // len(chunks))
    for _ in range(passes_w):
        one_pass()
    for _ in range(passes_t):
        one_pass(t)
    torch.cuda.synchronize()
    ms = t.mean_ms() * len(chunks)  # attention time of one chunked pass over the workload
    flops = 4.0 * spec.num_q_heads * spec.head_dim * sum(masked_pairs(L, spec.window) for L in lens)
    tf = flops / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "attention_ms_per_pass": round(ms, 4), "chunk_rows": C,
            "chunks_per_pass": len(chunks),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": per_pass(traffic_from_profile("chunked_prefill_sliding_512_traffic.txt"),
                                             len(chunks))},
            "algorithmic_flop_per_pass": flops}


def run_extra(args, torch, np, g, W, dev, headline):
    res = {}
    sl, sl_st = measure_sliding_step(args, torch, np, g, W, dev)
    log(f"sliding 2x4096 step: {sl['ms_per_step']} ms, attention {sl['kernel_ms']} ms")
    if not args.skip_cpu:
        sl["cpu_baseline"] = cpu_baseline_sliding(np, W)
    res["sliding_step_2x4096"] = sl
    res["chunked_prefill_sliding_2x4096_by_512"] = measure_chunked(args, torch, np, g, W, dev)
    res["prefill_sliding_2x4096_images"] = measure_images(args, torch, np, g, W, dev)
    log("chunked and image prefill done")
    for spec in (W.SLIDING_31B, W.GLOBAL_31B, W.GLOBAL_31B_V):
        name, r = measure_decode(args, torch, np, g, W, dev, spec)
        res[name] = r
        log(f"{name}: {r['kernel_ms']} ms")
    # the split form of the global layer (contract-fixed key chunks merged in order)
    name, r = measure_decode(args, torch, np, g, W, dev, W.GLOBAL_31B, split_keys=args.split_keys)
    res[name] = r
    log(f"{name}: {r['kernel_ms']} ms")
    st = prefill_step(args, torch, g, W, dev, W.GLOBAL_31B, [8192], seed=2, split_keys=args.split_keys)
    res[f"prefill_global_1x8192_split{args.split_keys}"] = {
        "value": round(st["achieved"], 2), "unit": "TFLOP/s", "kernel_ms": round(st["kernel_ms"], 4),
        **st["spread"], "kernel": st["kernel"],
        "roofline": {"bound": "mfma", "achieved": round(st["achieved"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(st["achieved"] / PEAK_BF16_TFLOPS, 4), "traffic": None}}
    log(f"prefill global split {args.split_keys}: {st['kernel_ms']:.4f} ms")
    res["global_v_step_1x8192"] = measure_global_v_step(args, torch, np, g, W, dev)
    for which in ("global", "sliding"):
        r = measure_backward(args, torch, np, g, W, dev, which)
        res[f"backward_{which}"] = r
        log(f"backward {which}: {r['ms_per_call']} ms")
    log(f"global step with separate K and V: {res['global_v_step_1x8192']['kernel_ms']} ms")
    if not args.skip_peaked:
        for which, plain in (("sliding", sl_st["kernel_ms"]), ("global", headline["kernel_ms"])):
            for mode in ("q24", "scale1"):
                r = measure_peaked(args, torch, np, g, W, dev, which, mode, plain)
                res[f"peaked_{which}_{mode}"] = r
                log(f"peaked {which} {mode}: {r['kernel_ms']} ms, rerun {r['workgroups_rerun_est']}")
    return res


COPY_BYTES = 512 * 1024 * 1024  # bytes read (and written) by one launch of the calibration copy


def run_copy(torch):
    """Calibration for the HBM byte counters: an elementwise negation of 512 MiB of bf16
    into another 512 MiB buffer (one plain read and one plain write of COPY_BYTES)."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def _counter_rows(path, kernel_substr, counter):
    import csv

    vals = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for a kernel containing {kernel_substr!r}")
    return vals


def write_traffic_summary(args):
    """profiles/NAME: mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the kernel, the same
    counters on the calibration copy, and the scaled HBM bytes per launch."""
    name, kernel, f_csv, w_csv, cf_csv, cw_csv = args.traffic_summary
    fetch = _counter_rows(f_csv, kernel, "FETCH_SIZE")
    write = _counter_rows(w_csv, kernel, "WRITE_SIZE")
    cfetch = _counter_rows(cf_csv, "neg", "FETCH_SIZE")
    cwrite = _counter_rows(cw_csv, "neg", "WRITE_SIZE")
    mf, mw = sum(fetch) / len(fetch), sum(write) / len(write)
    cf, cw = sum(cfetch) / len(cfetch), sum(cwrite) / len(cwrite)
    fscale = COPY_BYTES / (cf * 1024.0)
    wscale = COPY_BYTES / (cw * 1024.0)
    hbm = mf * 1024.0 * fscale + mw * 1024.0 * wscale
    lines = [
        f"# HBM traffic per launch of the kernel whose name contains '{kernel}'",
        "# Counters: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch, separate runs);",
        "# each scaled by the ratio of the known bytes of the calibration copy (bench.py --only copy:",
        f"# {COPY_BYTES} bytes read and {COPY_BYTES} bytes written per launch) to what the same counter reads for it.",
        f"command: {args.command}",
        f"kernel: {kernel}",
        f"dispatches_fetch: {len(fetch)}",
        f"dispatches_write: {len(write)}",
        f"fetch_kib_per_dispatch: {mf:.1f}",
        f"write_kib_per_dispatch: {mw:.1f}",
        f"copy_fetch_kib_per_dispatch: {cf:.1f}",
        f"copy_write_kib_per_dispatch: {cw:.1f}",
        f"fetch_scale: {fscale:.4f}",
        f"write_scale: {wscale:.4f}",
        f"fetch_bytes_per_launch: {mf * 1024.0 * fscale:.0f}",
        f"write_bytes_per_launch: {mw * 1024.0 * wscale:.0f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
        f"kernel_source_sha256_16: {source_hash()}",
    ]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", name), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_counter_summary(args):
    """profiles/NAME: the mean per dispatch of every counter a rocprofv3 --pmc pass recorded
    for the kernel (raw counters and rocprofv3's derived metrics, e.g. MfmaUtil = 100 x
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), LdsBankConflict = bank-conflict
    cycles per cycle of LDS index activity)."""
    import csv

    name, kernel, csv_path = args.counter_summary
    vals = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if kernel in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{csv_path}: no rows for a kernel containing {kernel!r}")
    lines = [f"# rocprofv3 --pmc counters of the kernel whose name contains '{kernel}' (mean per dispatch)",
             f"command: {args.command}", f"kernel: {kernel}",
             f"dispatches: {max(len(v) for v in vals.values())}"]
    for k in sorted(vals):
        v = vals[k]
        lines.append(f"{k}: {sum(v) / len(v):.6g}")
    lines.append(f"kernel_source_sha256_16: {source_hash()}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", name), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def run_only(args):
    """One measurement alone (kernel profiling): prints its numbers as one JSON line."""
    import numpy as np
    import torch

    import global_gqa_attention_amd as g
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    args.skip_cpu = True
    if args.only == "copy":
        run_copy(torch)
        return
    if args.only == "step":
        args.skip_extra = True
        run(args)
        return
    if args.only == "sliding":
        res = {"sliding_step_2x4096": measure_sliding_step(args, torch, np, g, W, dev)[0]}
    elif args.only == "chunked":
        res = {"chunked_prefill_sliding_2x4096_by_512": measure_chunked(args, torch, np, g, W, dev)}
    elif args.only == "images":
        res = {"prefill_sliding_2x4096_images": measure_images(args, torch, np, g, W, dev)}
    elif args.only in ("backward_global", "backward_sliding"):
        res = {args.only: measure_backward(args, torch, np, g, W, dev, args.only.split("_")[1])}
    elif args.only == "global_v":
        res = {"global_v_step_1x8192": measure_global_v_step(args, torch, np, g, W, dev)}
    elif args.only.startswith("peaked_"):
        _, which, mode = args.only.split("_")
        res = {args.only: measure_peaked(args, torch, np, g, W, dev, which, mode, float("nan"))}
    elif args.only == "prefill_global_split":
        st = prefill_step(args, torch, g, W, dev, W.GLOBAL_31B, [8192], seed=2, split_keys=args.split_keys)
        res = {f"prefill_global_1x8192_split{args.split_keys}": st}
    else:
        spec = {"decode_sliding": W.SLIDING_31B, "decode_global": W.GLOBAL_31B, "decode_global_split": W.GLOBAL_31B,
                "decode_global_v": W.GLOBAL_31B_V}[args.only]
        name, r = measure_decode(args, torch, np, g, W, dev, spec,
                                 split_keys=args.split_keys if args.only.endswith("_split") else 0)
        res = {name: r}
    print(json.dumps(res), flush=True)


def _oracle_result(value, unit, sec, sample):
    model, cores = cpu_info()
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "seconds": round(sec, 2),
            "cpu_model": model, "sample": sample}


def cpu_baseline_global(np, W):
    """The oracle on a bounded sample of the headline workload: the 8192-token global-layer
    sequence's KV head 0 (query heads 0..7 over their shared K=V head), prologue and
    dense-mask float64 attention; credited with that sample's masked FLOPs."""
    from oracle.attention import attention
    from oracle.bf16 import bf16_bits_to_f64
    from oracle.prologue import qk_prologue

    spec = W.GLOBAL_31B
    L = 8192
    case = W.prefill_case(spec, [L], seed=2)  # the step's recipe, drawn by the CPU generator
    G = spec.group
    kw = dict(rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta, eps=spec.rms_eps)
    pos = case.positions.numpy()
    qb, kb = W.bits(case.q[:, :G]), W.bits(case.k[:, :1])
    t0 = time.perf_counter()
    _, q1 = qk_prologue(qb, W.bits(case.wq), pos, **kw)
    _, k1 = qk_prologue(kb, W.bits(case.wk), pos, **kw)
    kf = bf16_bits_to_f64(k1)
    attention(bf16_bits_to_f64(q1), kf, kf, np.array([0]), np.array([L]), 1, 0, spec.softmax_scale)
    sec = time.perf_counter() - t0
    flops = 4.0 * G * spec.head_dim * masked_pairs(L, 0)
    log(f"cpu oracle, global sample: {sec:.2f} s")
    return _oracle_result(round(flops / sec / 1e12, 6), "TFLOP/s", sec,
                          "KV head 0 of the 1 x 8192 global-layer step (8 of 32 query heads, 1 of 4 KV heads): "
                          "float64 prologue + dense-mask attention, credited with the sample's masked FLOPs")


def cpu_baseline_sliding(np, W):
    """The oracle on the sliding step's whole workload (both 4096-token sequences, all 32
    query heads): prologue and attention, float64 numpy with dense masks."""
    from oracle.attention import attention
    from oracle.bf16 import bf16_bits_to_f64
    from oracle.prologue import qk_prologue

    spec = W.SLIDING_31B
    lens = [4096, 4096]
    case = W.prefill_case(spec, lens, seed=1)  # the step's recipe, drawn by the CPU generator
    kw = dict(rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta, eps=spec.rms_eps)
    pos = case.positions.numpy()
    t0 = time.perf_counter()
    _, q1 = qk_prologue(W.bits(case.q), W.bits(case.wq), pos, **kw)
    _, k1 = qk_prologue(W.bits(case.k), W.bits(case.wk), pos, **kw)
    attention(bf16_bits_to_f64(q1), bf16_bits_to_f64(k1), bf16_bits_to_f64(W.bits(case.v)), case.seq_start.numpy(),
              case.seq_len.numpy(), spec.num_kv_heads, spec.window, spec.softmax_scale)
    sec = time.perf_counter() - t0
    flops = 4.0 * spec.num_q_heads * spec.head_dim * sum(masked_pairs(L, spec.window) for L in lens)
    log(f"cpu oracle, sliding step: {sec:.2f} s")
    return _oracle_result(round(flops / sec / 1e12, 6), "TFLOP/s", sec,
                          "the whole sliding step once (2 x 4096 tokens, 32 q / 16 kv heads): float64 prologue + "
                          "dense-mask attention, credited with the masked FLOPs only")


def cpu_baseline_backward(np, W):
    """The oracle's attention backward on a bounded sample of the global backward workload:
    the first 4096 positions of KV head 0 (8 query heads) of the 1 x 8192 global layer
    (float64 dense masks), credited with 2.5 x that sample's masked FLOPs."""
    from oracle.attention import attention
    from oracle.backward import attention_backward

    spec = W.GLOBAL_31B
    L = 4096
    gen = W.make_generator(22)
    q = W.bf16_normal(gen, (L, spec.group, spec.head_dim)).double().numpy()
    k = W.bf16_normal(gen, (L, 1, spec.head_dim)).double().numpy()
    dout = W.bf16_normal(gen, (L, spec.group, spec.head_dim)).double().numpy()
    st, ln = np.array([0]), np.array([L])
    out = attention(q, k, k, st, ln, 1, 0, spec.softmax_scale)
    t0 = time.perf_counter()
    attention_backward(q, k, None, out, dout, st, ln, 1, 0, spec.softmax_scale, k_eq_v=True)
    sec = time.perf_counter() - t0
    flops = 2.5 * 4.0 * spec.group * spec.head_dim * masked_pairs(L, 0)
    log(f"cpu oracle, backward sample: {sec:.2f} s")
    return _oracle_result(round(flops / sec / 1e12, 6), "TFLOP/s", sec,
                          "KV head 0 (8 query heads) of the first 4096 positions of a global-layer sequence: float64 "
                          "dense-mask backward, credited with 2.5 x the sample's masked FLOPs")


def cpu_baseline_decode(np, W, case, sample=8, split_keys=0):
    """The oracle on the first `sample` sequences of a decode workload (the same inputs, copied
    to the host): the prologue of each sequence's cached keys and of its new token, then the
    token's attention over its visible keys (split_keys > 0: the oracle's split form);
    credited with those sequences' KV bytes."""
    from oracle.attention import decode_rows
    from oracle.split import split_decode_rows
    from oracle.bf16 import bf16_bits_to_f64
    from oracle.prologue import qk_prologue, v_prologue

    spec = case.spec
    kw = dict(rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim, theta=spec.rope_theta, eps=spec.rms_eps)
    wq, wk = W.bits(case.wq), W.bits(case.wk)
    qb = W.bits(case.q_raw[:sample])
    kb, vb = [], []
    for b in range(sample):
        a, n = int(case.key_start[b]), int(case.ctx[b] - case.key_lo[b])
        kb.append(W.bits(case.k_raw[a:a + n]))
        vb.append(None if spec.k_eq_v else W.bits(case.v_raw[a:a + n]))
    t0 = time.perf_counter()
    _, q1 = qk_prologue(qb, wq, case.ctx[:sample] - 1, **kw)
    qf = bf16_bits_to_f64(q1)
    for b in range(sample):
        lo, L = int(case.key_lo[b]), int(case.ctx[b])
        _, k1 = qk_prologue(kb[b], wk, np.arange(lo, L), **kw)
        keys = bf16_bits_to_f64(k1)
        if spec.k_eq_v:
            vals = keys
        elif spec.v_norm:
            vals = bf16_bits_to_f64(v_prologue(vb[b], eps=spec.rms_eps)[1])
        else:
            vals = bf16_bits_to_f64(vb[b])
        if split_keys:
            split_decode_rows(qf[b:b + 1], [keys], [vals], [lo], [L], spec.window, spec.softmax_scale, split_keys)
        else:
            decode_rows(qf[b:b + 1], [keys], [vals], [lo], [L], spec.window, spec.softmax_scale)
    sec = time.perf_counter() - t0
    kv = decode_kv_bytes(spec, case.ctx[:sample], case.key_lo[:sample])
    log(f"cpu oracle, decode sample ({spec.name}): {sec:.2f} s")
    return _oracle_result(round(kv / sec / 1e9, 4), "GB/s", sec,
                          f"sequences 0..{sample - 1} of the 64 ({kv} bytes of KV): float64 prologue of their cached "
                          "keys and new tokens, then the new tokens' attention; credited with their KV bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU takes a few hundred launches (~0.1 s of work) to reach its steady clock:
    # the default warm-up covers that, so the timed steps measure the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--skip-extra", action="store_true", help="omit every measurement but the headline step")
    ap.add_argument("--skip-peaked", action="store_true", help="omit the peaked-score prefill measurements")
    ap.add_argument("--only", choices=["step", "sliding", "chunked", "images", "decode_sliding", "decode_global",
                                       "global_v", "decode_global_v", "backward_global", "backward_sliding",
                                       "peaked_sliding_q24", "peaked_sliding_scale1", "peaked_global_q24",
                                       "peaked_global_scale1", "decode_global_split", "prefill_global_split",
                                       "copy"],
                    default=None,
                    help="run one measurement alone (for kernel profiling; prints that part's numbers only); "
                         "'copy' runs the plain copy that calibrates the HBM byte counters")
    ap.add_argument("--traffic-summary", nargs=6, default=None,
                    metavar=("NAME", "KERNEL", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/NAME from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of the "
                         "kernel (name containing KERNEL) and of the calibration copy; no GPU needed")
    ap.add_argument("--counter-summary", nargs=3, default=None, metavar=("NAME", "KERNEL", "CSV"),
                    help="write profiles/NAME from a rocprofv3 --pmc counter CSV of the kernel (name containing "
                         "KERNEL); no GPU needed")
    ap.add_argument("--split-keys", type=int, default=SPLIT_KEYS,
                    help="chunk size of the split-form measurements (a multiple of 256)")
    ap.add_argument("--command", default="", help="the profiling command, recorded in the summary")
    args = ap.parse_args()
    if args.traffic_summary is not None:
        write_traffic_summary(args)
        return
    if args.counter_summary is not None:
        write_counter_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (single-GPU build)", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)
    if args.only is not None:
        run_only(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
