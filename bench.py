"""Benchmark of the hybrid-attention hot path on one MI355X.

Step (the timed unit): the Gemma-4-31B sliding-layer prefill of a packed batch of
2 x 4096 tokens (32 q / 16 KV heads, head dim 256, window 1024): the q/k prologue
(RMSNorm + RoPE, out of place) followed by the attention kernel. The JSON line's
`value` is masked attention TFLOP/s of the whole step (4 * Hq * D * visible pairs
per second); `roofline` is the attention kernel alone, timed with HIP events on its
stream. The same run also measures the global-layer 8k prefill and decode against
KV caches (64 sequences, context lengths uniform in [1024, 32768]) and reports them
under "extra". Inputs are synthetic (seeded N(0,1) bf16, norm weights N(1, 0.1)).

CPU baseline: the float64 numpy oracle on a bounded sample of the step's workload.
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


def run(args):
    import numpy as np
    import torch

    import global_gqa_attention_amd as g
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    torch.backends.cuda.matmul.allow_tf32 = False

    # ---------------- step workload: sliding-layer prefill, 2 x 4096 -----------------
    spec = W.SLIDING_31B
    lens = [4096, 4096]
    case = W.prefill_case(spec, lens, seed=1, device=dev)
    layer = g.make_layer(spec)
    q_raw, k_raw, v = case.q, case.k, case.v
    q, k = torch.empty_like(q_raw), torch.empty_like(k_raw)
    out = torch.empty_like(q_raw)
    pairs = sum(masked_pairs(L, spec.window) for L in lens)
    flops = 4.0 * spec.num_q_heads * spec.head_dim * pairs
    attn_t = KernelTimer(torch)

    def step(timer=None):
        g.g4attn_qk_prologue(layer, q_raw, q, k_raw, k, case.wq, case.wk, case.positions)
        if timer is None:
            g.g4attn_prefill(layer, q, k, v, out, case.seq_start, case.seq_len, 4096)
        else:
            with timer:
                g.g4attn_prefill(layer, q, k, v, out, case.seq_start, case.seq_len, 4096)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(attn_t)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    attn_ms = attn_t.mean_ms()
    value = flops / (step_ms * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    prov = g.g4attn_prefill(layer, q, k, v, out, case.seq_start, case.seq_len, 4096, provenance=True)
    torch.cuda.synchronize()
    traffic = traffic_from_profile("prefill_sliding_2x4096_traffic.txt")

    extra = {}
    if not args.skip_extra:
        extra = run_extra(args, torch, np, g, W, dev)

    cpu = None if args.skip_cpu else cpu_baseline(np, W)
    line = {
        "metric": "prefill attention TFLOP/s (masked) + decode KV GB/s, % of MI355X roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gemma4-31b sliding-layer prefill: q/k prologue + attention, batch 2 x seq 4096 "
                               "packed (8192 tokens), 32 q / 16 kv heads, head dim 256, window 1024",
                   "global_batch": 2, "seq_len": 4096, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": prov["kernel_id"], "kernel_ms": round(attn_ms, 4), **attn_t.spread(),
                     "algorithmic_flop_per_launch": flops},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def measure_global_prefill(args, torch, np, g, W, dev):
    """Global-layer prefill, 1 x 8192, K=V, head dim 512: attention kernel alone."""
    spec = W.GLOBAL_31B
    case = W.prefill_case(spec, [8192], seed=2, device=dev)
    layer = g.make_layer(spec)
    q, k = torch.empty_like(case.q), torch.empty_like(case.k)
    out = torch.empty_like(case.q)
    g.g4attn_qk_prologue(layer, case.q, q, case.k, k, case.wq, case.wk, case.positions)
    flops = 4.0 * spec.num_q_heads * spec.head_dim * masked_pairs(8192, 0)
    t = KernelTimer(torch)
    for _ in range(args.warmup):
        g.g4attn_prefill(layer, q, k, None, out, case.seq_start, case.seq_len, 8192)
    for _ in range(args.steps):
        with t:
            g.g4attn_prefill(layer, q, k, None, out, case.seq_start, case.seq_len, 8192)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    tf = flops / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "kernel_ms": round(ms, 4), **t.spread(),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profile("prefill_global_1x8192_traffic.txt")},
            "algorithmic_flop_per_launch": flops}


def measure_decode(args, torch, np, g, W, dev, spec):
    """Decode of 64 sequences (context lengths uniform in [1024, 32768], seed 3) against
    a sliding ring of 1024 slots (K and V) or a linear K=V cache; KV-read GB/s."""
    B = 64
    ctx = W.decode_ctx_lens(B, 1024, 32768, seed=3)
    order = np.argsort(-ctx, kind="stable").astype(np.int32)
    gen = W.make_generator(3 if spec.window > 0 else 13, dev)
    layer = g.make_layer(spec)
    Hk, D = spec.num_kv_heads, spec.head_dim
    if spec.window > 0:
        C = spec.window
        region = [C] * B
        kv_bytes = sum(min(int(L), C) for L in ctx) * Hk * D * 2 * 2
    else:
        C = int(ctx.max())
        region = [int(L) for L in ctx]
        kv_bytes = int(ctx.sum()) * Hk * D * 2
    row0 = np.concatenate([[0], np.cumsum(region)[:-1]]).astype(np.int64)
    rows = int(sum(region))
    kc = W.bf16_normal(gen, (rows, Hk, D), device=dev)
    vc = None if spec.k_eq_v else W.bf16_normal(gen, (rows, Hk, D), device=dev)
    qd = W.bf16_normal(gen, (B, spec.num_q_heads, D), device=dev)
    od = torch.empty_like(qd)
    row0_t = torch.from_numpy(row0).to(dev)
    ctx_t = torch.from_numpy(ctx).to(dev)
    sched = torch.from_numpy(order).to(dev)
    t = KernelTimer(torch)
    for _ in range(args.warmup):
        g.g4attn_decode(layer, qd, kc, vc, row0_t, ctx_t, C, od, int(ctx.max()), schedule=sched)
    for _ in range(args.steps):
        with t:
            g.g4attn_decode(layer, qd, kc, vc, row0_t, ctx_t, C, od, int(ctx.max()), schedule=sched)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    name = "decode_sliding_64seq" if spec.window > 0 else "decode_global_64seq"
    res = {"value": round(gbs, 1), "unit": "GB/s", "kernel_ms": round(ms, 4), **t.spread(), "kv_bytes": kv_bytes,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": traffic_from_profile(name + "_traffic.txt")}}
    del kc, vc
    torch.cuda.empty_cache()
    return name, res


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


def run_extra(args, torch, np, g, W, dev):
    res = {"global_prefill_1x8192": measure_global_prefill(args, torch, np, g, W, dev),
           "chunked_prefill_sliding_2x4096_by_512": measure_chunked(args, torch, np, g, W, dev),
           "prefill_sliding_2x4096_images": measure_images(args, torch, np, g, W, dev)}
    for spec in (W.SLIDING_31B, W.GLOBAL_31B):
        name, r = measure_decode(args, torch, np, g, W, dev, spec)
        res[name] = r
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


def run_only(args):
    """One measurement alone (kernel profiling): prints its numbers as one JSON line."""
    import numpy as np
    import torch

    import global_gqa_attention_amd as g
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    if args.only == "copy":
        run_copy(torch)
        return
    if args.only == "step":
        args.skip_extra = True
        args.skip_cpu = True
        run(args)
        return
    if args.only == "global":
        res = {"global_prefill_1x8192": measure_global_prefill(args, torch, np, g, W, dev)}
    elif args.only == "chunked":
        res = {"chunked_prefill_sliding_2x4096_by_512": measure_chunked(args, torch, np, g, W, dev)}
    elif args.only == "images":
        res = {"prefill_sliding_2x4096_images": measure_images(args, torch, np, g, W, dev)}
    else:
        spec = W.SLIDING_31B if args.only == "decode_sliding" else W.GLOBAL_31B
        name, r = measure_decode(args, torch, np, g, W, dev, spec)
        res = {name: r}
    print(json.dumps(res), flush=True)


def cpu_baseline(np, W):
    """The oracle on the step's workload (both 4096-token sequences, all 32 query heads):
    prologue and attention, float64 numpy with dense masks. About 10 s on 16 host cores."""
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
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(sec, 2),
            "sample": "the whole step workload once (2 x 4096 tokens, 32 q / 16 kv heads): float64 prologue + "
                      "dense-mask attention, credited with the masked FLOPs only"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU takes a few hundred launches (~0.1 s of work) to reach its steady clock:
    # the default warm-up covers that, so the timed steps measure the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--skip-extra", action="store_true", help="omit the global prefill and decode measurements")
    ap.add_argument("--only", choices=["step", "global", "chunked", "images", "decode_sliding", "decode_global", "copy"],
                    default=None,
                    help="run one measurement alone (for kernel profiling; prints that part's numbers only); "
                         "'copy' runs the plain copy that calibrates the HBM byte counters")
    ap.add_argument("--traffic-summary", nargs=6, default=None,
                    metavar=("NAME", "KERNEL", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/NAME from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of the "
                         "kernel (name containing KERNEL) and of the calibration copy; no GPU needed")
    ap.add_argument("--command", default="", help="the profiling command, recorded in the traffic summary")
    args = ap.parse_args()
    if args.traffic_summary is not None:
        write_traffic_summary(args)
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
