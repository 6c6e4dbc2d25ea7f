#!/usr/bin/env python3
"""Decode-step benchmark of the ResidualQuant KV path on one MI355X.

A step is one pass of the whole hot path over a synthetic Ouro-1.4B-like
cache (24 layers x 4 loops, 16 heads x 128, 8192 tokens, batch 4): for every
loop and layer, fused decode attention of one query token per (batch row,
head) over the packed INT4-anchor / INT2-residual cache, then the quantize-
append of the new token's K/V for all loops and layers.  Inputs are resident
in HBM before timing starts.

Prints one JSON line (stdout).  Progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu] [--no-bf16]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X published HBM3E bandwidth
PROFILES = os.path.join(ROOT, "profiles")
# the sources the dominant kernel's code and launch depend on, and the build
# script that sets its compiler flags
DECODE_SRCS = [os.path.join(ROOT, "decode_attention_int4_amd", "csrc", f)
               for f in ("rq_decode.hip", "rq_stage.h", "rq_api.hip", "rq_layout.h", "rq_kernels.h",
                         "rq_device.h")] + [os.path.join(ROOT, "decode_attention_int4_amd", "build.py")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_sha(paths=DECODE_SRCS) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(config: str):
    """HBM bytes per dominant-kernel launch from committed rocprofv3 counter
    runs, or None when missing or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"decode_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != src_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def trace_from_profile(config: str):
    """The dominant kernel's average dispatch duration in the committed
    rocprofv3 kernel trace of this benchmark (profiles/), or None when missing
    or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"decode_{config}_kernel_trace.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != src_sha():
        return None
    return t.get("dominant_avg_us")


def time_steps(step, steps: int, torch):
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    for _ in range(steps):
        step()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / steps, wall


def graphed(fn, torch):
    """Captures fn's launches (made on the current stream) into one HIP graph,
    after one warm call on a side stream as graph capture requires."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def dominant_calls(run):
    """The decode-attention calls of the dominant kind in step order (the
    residual loops of a residual cache, the INT4 anchor loops of a direct
    one); every call reads a different (loop, layer) of the cache."""
    w = run.w
    P = w.loops_per_group
    return [(loop, layer) for loop in range(w.loops) for layer in range(w.layers)
            if (loop % P != P - 1) == (w.mode != 1)]


def kernel_name(w) -> str:
    """The dominant call's kernel as the profiler names it."""
    two = w.mode != 1
    if w.q_heads > w.kv_heads:
        return (f"gqa_kernel<{w.head_dim},{w.anchor_bits},{w.residual_bits if two else 0},"
                f"{str(w.page_tokens > 0).lower()}>")
    # waves per workgroup: 8 at d = 128 (residual calls, and anchor calls on
    # a contiguous cache) unless a chained loop reads several residual planes
    # (then 4), else 4
    waves = 8 if (w.head_dim == 128 and (w.page_tokens == 0 or two)) else 4
    return (f"decode_kernel<{w.head_dim},{w.anchor_bits},{w.residual_bits if two else 0},"
            f"{'NR' if w.mode == 2 else 1},{str(w.page_tokens > 0).lower()},"
            f"{'W' if w.mode == 2 and waves == 8 else waves}>")


def dominant_roofline(run, steps: int, torch, use_graph: bool) -> dict:
    """Roofline figures of a workload's dominant decode call: algorithmic
    bytes per launch over the event-timed average launch (see
    dominant_kernel_ms)."""
    dom_ms, n_launch = dominant_kernel_ms(run, steps, torch, use_graph)
    calls = dominant_calls(run)
    # bytes per dominant call (chained mode: the calls read 1 to P-1 residual planes)
    dom_bytes = sum(run.call_bytes(loop) for loop, _ in calls) // len(calls)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "kernel": kernel_name(run.w),
            "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_ms * 1e3, 2),
            "launches_timed": n_launch}


def dominant_kernel_ms(run, steps: int, torch, use_graph: bool):
    """Average duration of one dominant call (one decode kernel launch, which
    also merges its splits), from events on the stream the kernel runs on
    around `steps` back-to-back passes over all dominant calls of a step."""
    calls = dominant_calls(run)

    def once():
        for loop, layer in calls:
            run.attend(loop, layer)

    g = graphed(once, torch) if use_graph else None
    fn = g.replay if use_graph else once
    fn()
    ms, _ = time_steps(fn, steps, torch)
    return ms / len(calls), steps * len(calls)


def read_peak(torch, rq, call_bytes: int, nbytes=8 << 30, reps=5):
    """The library's streaming-read probe: GB/s over one 8 GiB read, and the
    time to read `call_bytes` per launch in back-to-back launches over
    distinct parts of the buffer (the floor for a decode call of that size)."""
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(7)
    sink = torch.zeros(rq.read_probe_sink_words(), dtype=torch.int32, device="cuda")
    rq.read_probe(buf, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        rq.read_probe(buf, sink)
    e.record()
    torch.cuda.synchronize()
    gbps = nbytes / (s.elapsed_time(e) / reps * 1e-3) / 1e9
    words = call_bytes // 16 * 4                     # int32 words, 16-byte multiple
    parts = [buf[i * words:(i + 1) * words] for i in range(min(40, buf.numel() // words))]
    for p in parts:
        rq.read_probe(p, sink)
    torch.cuda.synchronize()
    s.record()
    for p in parts:
        rq.read_probe(p, sink)
    e.record()
    torch.cuda.synchronize()
    call_us = s.elapsed_time(e) / len(parts) * 1e3
    del buf, parts
    torch.cuda.empty_cache()
    return gbps, call_us


def cpu_threads():
    """Host cores this process may run on, and the threads the oracle uses:
    all of them, up to 16 (the host share of a one-GPU machine)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return usable, max(1, min(16, usable))


def cpu_baseline(run, budget_s: float = 12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same step:
    attention calls of sampled (batch row, layer, head) slices for every loop,
    plus encoding of sampled new-token loop groups, both spread over the host
    threads (the oracle's C calls release the GIL); extrapolated to one full
    step (every loop x layer x batch row x head, and the whole append)."""
    import numpy as np

    import oracle as O
    from decode_attention_int4_amd.synth import rotation_signs

    w = run.w
    usable, cores = cpu_threads()
    p = O.Params(d=w.head_dim, P=w.loops_per_group, anchor_bits=w.anchor_bits,
                 residual_bits=w.residual_bits, mode=w.mode, alpha_mode=w.alpha_mode,
                 rotate=1 if (w.rotation == 1 and w.mode != 1) else 0)
    signs = rotation_signs(w).numpy()

    def bits(t):
        return t.contiguous().cpu().view(__import__("torch").int16).numpy().view(np.uint16)

    encs = []
    for key, kept in run.kept.items():
        b, layer, head = key
        HK, HV = signs[0, layer].copy(), signs[1, layer].copy()
        encs.append((key, O.encode_slice(p, bits(kept[0]), HK), O.encode_slice(p, bits(kept[1]), HV),
                     HK, HV))
    jobs = [(e, loop) for e in encs for loop in range(w.loops)]
    qbits = {(e[0], loop): bits(run.q[loop, e[0][1], e[0][0], e[0][2]]) for e, loop in jobs}

    def attn(job):
        (key, ek, ev, HK, HV), loop = job
        return O.attention_slice(p, ek, ev, HK, HV, qbits[(key, loop)], loop, run.N,
                                 w.softmax_scale)

    # append: encode new-token loop groups (one per kv, batch row, layer, head, group)
    new = run.new_kv  # [2, B, loops, layers, H, 1, d]
    groups = [(kv, b, layer, head, k) for kv in range(2) for b in range(w.batch)
              for layer in range(w.layers) for head in range(w.kv_heads)
              for k in range(w.loops // w.loops_per_group)]
    rng = np.random.default_rng(0)
    sample = [groups[i] for i in rng.choice(len(groups), size=min(1024, len(groups)), replace=False)]
    P = w.loops_per_group
    xs = [(O.bf16_decode(bits(new[kv, b, k * P:(k + 1) * P, layer, head, 0])), signs[kv, layer].copy())
          for kv, b, layer, head, k in sample]

    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        n_calls = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s * 0.8:
            reps = max(1, cores // len(jobs))
            list(ex.map(attn, jobs * reps))
            n_calls += len(jobs) * reps
        t_attn = time.perf_counter() - t0
        t1 = time.perf_counter()
        list(ex.map(lambda xh: O.encode_group(p, xh[0], xh[1]), xs))
        t_enc = (time.perf_counter() - t1) / len(xs)     # wall time per encode, all threads
    calls_per_s = n_calls / t_attn

    step_calls = w.loops * w.layers * w.batch * w.q_heads
    step_s = step_calls / calls_per_s + t_enc * len(groups)
    return {
        "value": w.batch / step_s,
        "unit": "tokens/s",
        "cores": cores,
        "host_cores": usable,
        "kind": "oracle",
        "sample": (f"{n_calls} fp64 attention calls (n={run.N}) on {len(encs)} sampled "
                   f"(batch,layer,head) slices x {w.loops} loops ({calls_per_s:.1f} calls/s) + "
                   f"{len(xs)} new-token loop-group encodes ({t_enc * 1e6:.1f} us wall each), on "
                   f"{cores} threads of {usable} host cores; extrapolated to {step_calls} calls "
                   f"and {len(groups)} encodes per step = {step_s:.1f} s/step"),
    }


def capacity_sweep(args, torch, rq, WORKLOADS, RQDecode, BF16Decode):
    """Batch doubling 1, 2, 4, ... on the configured shapes, for the packed
    cache and for BF16, while each cache fits in device memory (with a margin
    for the step's workspace and generation chunks).  One JSON line per batch."""
    base = WORKLOADS[args.config]
    margin = 8 << 30
    b = 1
    while b <= 1024:
        w = base.with_(batch=b, name=f"{base.name}_batch{b}")
        rec = {"sweep": "capacity", "workload": base.name, "batch": b}
        for kind in ("rq", "bf16"):
            torch.cuda.empty_cache()
            free, _ = torch.cuda.mem_get_info()
            if kind == "rq":
                from decode_attention_int4_amd.workload import desc_for
                need = rq.cache_bytes(desc_for(w, w.n_tokens + 1))
            else:
                need = 2 * w.batch * w.loops * w.layers * w.kv_heads * (w.n_tokens + 1) * w.head_dim * 2
            if need + margin > free:
                rec[kind] = {"fits": False, "cache_gb": round(need / 1e9, 1)}
                continue
            run = RQDecode(w) if kind == "rq" else BF16Decode(w)
            run.step()
            g = graphed(run.step, torch)
            for _ in range(args.warmup):
                g.replay()
            ms, _ = time_steps(g.replay, args.steps, torch)
            rec[kind] = {"fits": True, "cache_gb": round(need / 1e9, 1), "ms_per_step": round(ms, 4),
                         "tokens_per_s": round(b / (ms * 1e-3), 1),
                         "hbm_gbps": round(run.step_bytes() / (ms * 1e-3) / 1e9, 1)}
            del g, run
        print(json.dumps(rec), flush=True)
        log(f"[sweep] batch {b}: " + ", ".join(
            f"{k} " + (f"{rec[k]['tokens_per_s']} tok/s ({rec[k]['cache_gb']} GB)" if rec[k]["fits"]
                       else f"does not fit ({rec[k]['cache_gb']} GB)") for k in ("rq", "bf16")))
        if not rec["rq"]["fits"] and not rec["bf16"]["fits"]:
            break
        b *= 2


def pages_sweep(args, torch, rq, WORKLOADS, RQDecode):
    """The configured shapes on a contiguous cache and in paged pools of the
    given block sizes (blocks in random pool order): step time, dominant call
    and pool bytes, one JSON line per cache."""
    base = WORKLOADS[args.config]
    for pt in [0] + [int(x) for x in args.pages.split(",") if x]:
        w = base.with_(page_tokens=pt, name=f"{base.name}_pages{pt}" if pt else base.name)
        run = RQDecode(w)
        run.step()
        g = graphed(run.step, torch)
        for _ in range(args.warmup):
            g.replay()
        ms, _ = time_steps(g.replay, args.steps, torch)
        roof = dominant_roofline(run, args.steps, torch, True)
        rec = {"sweep": "pages", "workload": base.name, "block_tokens": pt or None,
               "ms_per_step": round(ms, 4), "tokens_per_s": round(w.batch / (ms * 1e-3), 1),
               "dominant_call_us": roof["avg_launch_us"], "kernel": roof["kernel"],
               "pool_gb": round(rq.cache_bytes(run.desc) / 1e9, 3)}
        print(json.dumps(rec), flush=True)
        del g, run
        torch.cuda.empty_cache()


def launch_gap(args, torch):
    """Per-launch time of 72 back-to-back trivial kernels (one 256 x 512
    element add each) replayed from a HIP graph: the floor that the graph's
    launch sequencing puts under every decode call's event-timed duration."""
    y = torch.zeros(256 * 512, device="cuda")

    def once():
        for _ in range(72):
            y.add_(1.0)
    g = graphed(once, torch)
    for _ in range(args.warmup):
        g.replay()
    ms, _ = time_steps(g.replay, args.steps, torch)
    print(json.dumps({"launch_gap_us": round(ms * 1e3 / 72, 3), "launches": 72 * args.steps}), flush=True)


def measure_variant(w, keep, args, torch, rq, RQDecode):
    """Cache size, step bytes and throughput of one workload's packed cache, the
    relative L2 error of its K and V reconstructions (first 128 tokens) against
    the BF16 originals, of the slice queries' logits over those keys, and of
    its decode-attention outputs against fp32 attention over the BF16
    originals (every loop of the `keep` slices)."""
    n_rec = min(128, w.n_tokens)

    def rel(a, b):
        return ((a - b).norm() / b.norm()).item()

    torch.cuda.empty_cache()
    run = RQDecode(w, keep=keep)
    run.step()
    torch.cuda.synchronize()
    att = []
    for (b, layer, head) in keep:
        kv = run.kept[(b, layer, head)].float().cuda()            # [2, loops, N, d]
        for loop in range(w.loops):
            q = run.q[loop, layer][b, head].float()
            p = torch.softmax((kv[0, loop] @ q) * w.softmax_scale, dim=0)
            att.append(rel(run.out[loop, layer, b, head], p @ kv[1, loop]))
    rec = rq.reconstruct(run.desc, run.cache, run.signs, 0, n_rec, out_dtype=torch.bfloat16)
    kerr, verr, lerr, lmax = [], [], [], []
    for (b, layer, head) in keep:
        orig = run.kept[(b, layer, head)][:, :, :n_rec].float().cuda()
        got = rec[:, b, :, layer, head].float()
        qh = head * (w.q_heads // w.kv_heads)
        for loop in range(w.loops):
            kerr.append(rel(got[0, loop], orig[0, loop]))
            verr.append(rel(got[1, loop], orig[1, loop]))
            # logits of the slice's query over the reconstructed keys: the
            # key error as attention sees it, before the softmax (whose
            # outlier channels make it nearly one-hot on these shapes)
            q = run.q[loop, layer][b, qh].float()
            lg_ref, lg = (orig[0, loop] @ q) * w.softmax_scale, (got[0, loop] @ q) * w.softmax_scale
            lerr.append(rel(lg, lg_ref))
            lmax.append((lg - lg_ref).abs().max().item())
    del rec
    g = graphed(run.step, torch)
    for _ in range(args.warmup):
        g.replay()
    ms, _ = time_steps(g.replay, args.steps, torch)
    out = {"cache_gb": round(rq.cache_bytes(run.desc) / 1e9, 2), "step_gb": round(run.step_bytes() / 1e9, 2),
           "ms_per_step": round(ms, 4), "tokens_per_s": round(w.batch / (ms * 1e-3), 1),
           "k_rel_l2": round(sum(kerr) / len(kerr), 5), "v_rel_l2": round(sum(verr) / len(verr), 5),
           "logit_rel_l2": round(sum(lerr) / len(lerr), 5), "logit_max_abs": round(max(lmax), 4),
           "attn_rel_l2_mean": round(sum(att) / len(att), 5), "attn_rel_l2_max": round(max(att), 5)}
    del g, run
    return out


def quant_timing(args, torch, rq, WORKLOADS):
    """Quantize-append on the configured shapes: one fill chunk of the size the
    cache fill uses, and the one-token append of a decode step.  Bytes are the
    BF16 input read plus the codes, FP8 scale/offset pairs and alphas written
    (the kernel reads each input once and writes each output once)."""
    from decode_attention_int4_amd.synth import kv_chunk, rotation_signs
    from decode_attention_int4_amd.workload import default_chunk, desc_for
    w = WORKLOADS[args.config]
    d, P, G = w.head_dim, w.loops_per_group, w.loops // w.loops_per_group
    for T in (default_chunk(w), 1):
        desc = desc_for(w, max(T, 64))
        cache = rq.alloc_cache(desc)
        x = kv_chunk(w, 0, T, "cuda")
        signs = rotation_signs(w).cuda()
        rq.quantize_append(desc, cache, x, 0, signs)
        reps = max(args.steps, 5)
        torch.cuda.synchronize()
        ms, _ = time_steps(lambda: rq.quantize_append(desc, cache, x, 0, signs), reps, torch)
        items = 2 * w.batch * w.layers * w.kv_heads * G * T
        out_b = items * (d * w.anchor_bits // 8 + 2 * (d // 16) + (P - 1) * (
            d * w.residual_bits // 8 + 2 * (d // 16) + (2 if w.mode != 1 else 0)))
        in_b = x.numel() * 2
        gbps = (in_b + out_b) / (ms * 1e-3) / 1e9
        print(json.dumps({"workload": w.name, "t_new": T, "us_per_call": round(ms * 1e3, 2),
                          "bytes_in": in_b, "bytes_out": out_b, "gbps": round(gbps, 1),
                          "frac_of_8tbs": round(gbps / PEAK_HBM_GBPS, 4)}), flush=True)
        del cache, x


def study_keep(w):
    return [(0, 0, 0), (w.batch // 2, w.layers // 2, w.kv_heads // 2),
            (w.batch - 1, w.layers - 1, w.kv_heads - 1)]


def variants_study(args, torch, rq, WORKLOADS, RQDecode, BF16Decode):
    """Accuracy and cost of the method's variants on one workload's shapes:
    bit widths, the alpha rule, the rotation, the chained anchor, and the
    direct per-loop quantization the method improves on (one JSON line each,
    see measure_variant), then loop groups of 4, 8 and 16 loops in residual
    mode with the bytes a chained previous-loop anchor would read (computed:
    the kernel reads at most three residual planes, groups of up to 4), and a
    last line timing the BF16 cache."""
    base = WORKLOADS[args.config]
    variants = [
        ("INT4 anchor + INT2 residual, LS alpha, Hadamard", {}),
        ("uniform INT4 (INT4 residual)", dict(residual_bits=4)),
        ("uniform INT2 (INT2 anchor)", dict(anchor_bits=2)),
        ("norm-ratio alpha", dict(alpha_mode=1)),
        ("alpha = 1", dict(alpha_mode=2)),
        ("rotation off", dict(rotation=0)),
        ("chained previous-loop anchor", dict(mode=2)),
        ("direct: INT4 anchor position, INT2 other loops", dict(mode=1)),
        ("direct: INT4 every loop", dict(mode=1, residual_bits=4)),
    ]
    keep = study_keep(base)
    for label, kw in variants:
        w = base.with_(name=f"{base.name}_variant", **kw)
        rec = {"variant": label, "workload": base.name, "settings": kw,
               **measure_variant(w, keep, args, torch, rq, RQDecode)}
        print(json.dumps(rec), flush=True)
        log(f"[variants] {label}: {rec['tokens_per_s']} tok/s, step {rec['step_gb']} GB, "
            f"K/V rel-L2 {rec['k_rel_l2']:.4f}/{rec['v_rel_l2']:.4f}, "
            f"logit rel-L2 {rec['logit_rel_l2']:.4f} (max abs {rec['logit_max_abs']:.3f}), "
            f"attention rel-L2 {rec['attn_rel_l2_mean']:.4f} (max {rec['attn_rel_l2_max']:.4f})")
    # loop groups: P loops per group, noise ramp 0.3 .. 0.1 towards the anchor
    d, ng = base.head_dim, base.head_dim // 16
    for P in (4, 8, 16):
        sig = tuple(round(0.1 + 0.2 * (P - 2 - j) / (P - 2), 4) for j in range(P - 1))
        w = base.with_(name=f"{base.name}_group{P}", loops=P, loops_per_group=P, sigmas=sig)
        anchor_b = d * w.anchor_bits // 8 + 2 * ng
        resid_b = d * w.residual_bits // 8 + 2 * ng + 2
        rows = 2 * w.batch * w.kv_heads * w.n_tokens * w.layers
        chained = rows * sum(anchor_b + (P - 1 - j) * resid_b for j in range(P - 1)) + rows * anchor_b
        rec = {"variant": f"loop group {P}", "workload": base.name, "settings": {"loops": P, "loops_per_group": P},
               **measure_variant(w, study_keep(w), args, torch, rq, RQDecode),
               "chained_step_gb_computed": round(chained / 1e9, 2)}
        print(json.dumps(rec), flush=True)
        log(f"[variants] loop group {P}: {rec['tokens_per_s']} tok/s, step {rec['step_gb']} GB "
            f"(chained anchor would read {rec['chained_step_gb_computed']} GB), "
            f"K/V rel-L2 {rec['k_rel_l2']:.4f}/{rec['v_rel_l2']:.4f}")
    torch.cuda.empty_cache()
    run = BF16Decode(base)
    run.step()
    g = graphed(run.step, torch)
    for _ in range(args.warmup):
        g.replay()
    ms, _ = time_steps(g.replay, args.steps, torch)
    print(json.dumps({"variant": "BF16 cache", "workload": base.name,
                      "cache_gb": round(2 * base.batch * base.loops * base.layers * base.kv_heads
                                        * base.n_tokens * base.head_dim * 2 / 1e9, 2),
                      "step_gb": round(run.step_bytes() / 1e9, 2), "ms_per_step": round(ms, 4),
                      "tokens_per_s": round(base.batch / (ms * 1e-3), 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="ouro8k_b4")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--also", default="ouro16k_b4,huginn8k_b2",
                    help="comma-separated workloads whose dominant decode call is also timed "
                         "(roofline only; empty to skip)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from Python instead of replaying a HIP graph of the step")
    ap.add_argument("--sweep", action="store_true",
                    help="batch-capacity sweep (batch 1, 2, 4, ... while caches fit) instead of the "
                         "single benchmark line")
    ap.add_argument("--pages", default="",
                    help="comma-separated paged block sizes: time the configured shapes on a "
                         "contiguous cache and in pools of these blocks (JSON lines) instead of "
                         "the single benchmark line")
    ap.add_argument("--launch-gap", action="store_true",
                    help="only time back-to-back trivial kernels replayed from a HIP graph "
                         "(the per-launch floor under every event-timed call)")
    ap.add_argument("--variants", action="store_true",
                    help="accuracy and cost of the method's variants on the configured shapes "
                         "(one JSON line per variant) instead of the single benchmark line")
    ap.add_argument("--quant", action="store_true",
                    help="only time quantize-append on the configured shapes: one fill chunk "
                         "and the one-token append (JSON lines)")
    ap.add_argument("--calibrate-counters", action="store_true",
                    help="only run a 1 GiB device copy and a 1 GiB read (known byte counts) "
                         "to calibrate FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (batch, head) pair is independent; see the design notes on sharding).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_int4_amd import rq
    from decode_attention_int4_amd.synth import WORKLOADS
    from decode_attention_int4_amd.workload import BF16Decode, RQDecode

    if args.calibrate_counters:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        sink = torch.zeros(rq.read_probe_sink_words(), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)                       # reads and writes exactly 1 GiB
        rq.read_probe(src, sink)             # reads exactly 1 GiB
        torch.cuda.synchronize()
        print(json.dumps({"calibration_bytes": n}), flush=True)
        return

    if args.quant:
        quant_timing(args, torch, rq, WORKLOADS)
        return
    if args.sweep:
        capacity_sweep(args, torch, rq, WORKLOADS, RQDecode, BF16Decode)
        return
    if args.pages:
        pages_sweep(args, torch, rq, WORKLOADS, RQDecode)
        return
    if args.launch_gap:
        launch_gap(args, torch)
        return
    if args.variants:
        variants_study(args, torch, rq, WORKLOADS, RQDecode, BF16Decode)
        return

    w = WORKLOADS[args.config]
    log(f"[bench] {w}")
    t = time.perf_counter()
    keep = [(0, 0, 0), (w.batch - 1, w.layers - 1, w.kv_heads - 1)]
    run = RQDecode(w, keep=keep)
    torch.cuda.synchronize()
    log(f"[bench] packed cache {rq.cache_bytes(run.desc) / 1e9:.2f} GB filled in "
        f"{time.perf_counter() - t:.1f} s")

    use_graph = not args.eager
    for _ in range(args.warmup):
        run.step()
    step_graph = graphed(run.step, torch) if use_graph else None
    step_fn = step_graph.replay if use_graph else run.step
    for _ in range(args.warmup):
        step_fn()
    ms, wall = time_steps(step_fn, args.steps, torch)
    tok_s = w.batch / (ms * 1e-3)
    step_bytes = run.step_bytes()
    log(f"[bench] {ms:.3f} ms/step, {tok_s:.1f} tokens/s, {step_bytes / (ms * 1e-3) / 1e9:.0f} GB/s")

    roof = dominant_roofline(run, args.steps, torch, use_graph)
    achieved, dom_bytes = roof["achieved"], roof["algorithmic_bytes_per_launch"]
    log(f"[bench] dominant call ({roof['kernel']}): {roof['avg_launch_us']} us/launch over "
        f"{roof['launches_timed']} launches, {achieved:.0f} GB/s, {roof['frac']:.3f} of 8 TB/s")
    trace_us = trace_from_profile(args.config)
    if trace_us:
        roof["trace_avg_launch_us"] = trace_us
        roof["trace_frac"] = round(dom_bytes / (trace_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)

    extra = {}
    if not args.no_probe:
        peak, call_us = read_peak(torch, rq, dom_bytes)
        extra["measured_read_peak_gbps"] = round(peak, 1)
        extra["frac_of_measured_read_peak"] = round(achieved / peak, 4)
        extra["read_probe"] = {"gbps_8gib": round(peak, 1), "call_bytes": dom_bytes,
                               "us_per_call_bytes": round(call_us, 2),
                               "gbps_call_bytes": round(dom_bytes / (call_us * 1e-6) / 1e9, 1)}
        log(f"[bench] streaming-read probe: {peak:.0f} GB/s over 8 GiB; one call's "
            f"{dom_bytes / 1e6:.0f} MB in {call_us:.1f} us per launch")

    others = [o for o in args.also.split(",") if o and o != args.config]
    if others:
        extra["roofline_other_workloads"] = {}
    for name in others:
        ow = WORKLOADS[name]
        orun = RQDecode(ow)
        for _ in range(args.warmup):
            orun.step()
        oroof = dominant_roofline(orun, args.steps, torch, use_graph)
        extra["roofline_other_workloads"][name] = oroof
        log(f"[bench] {name} dominant call ({oroof['kernel']}): {oroof['avg_launch_us']} us/launch, "
            f"{oroof['achieved']:.0f} GB/s, {oroof['frac']:.3f} of 8 TB/s")
        del orun
        torch.cuda.empty_cache()

    if not args.no_bf16:
        base = BF16Decode(w)
        for _ in range(args.warmup):
            base.step()
        base_graph = graphed(base.step, torch) if use_graph else None
        base_fn = base_graph.replay if use_graph else base.step
        bms, _ = time_steps(base_fn, args.steps, torch)
        extra["bf16_baseline"] = {
            "ms_per_step": round(bms, 4), "tokens_per_s": round(w.batch / (bms * 1e-3), 2),
            "hbm_gbps": round(base.step_bytes() / (bms * 1e-3) / 1e9, 1),
            "speedup_of_residual": round(bms / ms, 3)}
        log(f"[bench] bf16 baseline: {bms:.3f} ms/step, {w.batch / (bms * 1e-3):.1f} tokens/s")
        del base, base_graph, base_fn
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(run)
        log(f"[bench] oracle: {cpu['value']:.4f} tokens/s ({cpu['sample']})")

    traffic = traffic_from_profile(args.config)
    line = {
        "metric": "decode-attn tokens/s + achieved HBM GB/s on INT4/INT2 residual KV, 8k/16k",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "loops": w.loops, "layers": w.layers,
                   "kv_heads": w.kv_heads, "q_heads": w.q_heads, "head_dim": w.head_dim,
                   "context_tokens": w.n_tokens, "anchor_bits": w.anchor_bits,
                   "residual_bits": w.residual_bits, "group": 16,
                   "mode": {0: "residual", 1: "direct", 2: "chained"}[w.mode],
                   "cache": (f"paged, {w.page_tokens}-token blocks in random pool order"
                             if w.page_tokens else "contiguous"),
                   "launch": "hip graph of one step" if use_graph else "eager"},
        "hbm_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "step_algorithmic_bytes": step_bytes,
        "roofline": {**roof, "traffic": traffic},
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
