"""Benchmark: K2V2 decode attention over the packed OmniKVQuant cache on one MI355X.

One step = one decode step of the whole batch: the split-KV partial pass and the
merge + batched inverse value rotation (omnikv_decode_partial then
omnikv_decode_combine) over every cached token of every sequence.  The packed
caches are built before timing by the library's own write path (keys and values
of synthetic drifting K/V, quantized in prefill-sized chunks), and several
independent caches are cycled so that a step never finds its cache in the 256 MB
Infinity Cache: the timed bytes come from HBM.

Timing.  The K timed steps are captured in one HIP graph (two short kernels per step
would otherwise wait on Python launch overhead).  The headline is one replay of that
graph between two synchronisations: exactly K steps.  The spread (median / p10 / p90
per step) comes from further replays of the same graph, each bracketed by events; the
per-kernel figures from graphs of K partial-only and K combine-only launches, replayed
the same way.  The write path is timed separately on one prefill chunk per sequence.

Prints one JSON line: the headline (effective KV GB/s of the decode step), the
roofline of the partial kernel, the write-path timings, the other configurations
(configs 4 and 5 at K2V2 and K4V4, the write path at K4V4 and with fp32 inputs, and the
config-5 prefill write path at both widths) and a CPU-oracle
baseline on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_attention_fwht_amd import binding, synth  # noqa: E402

METRIC = "K2V2 decode-attention µs/step + effective KV HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20


def mx_record_bytes(d):
    """Bytes of one window's MXFP4 key-metadata record (one vector): d/2 code bytes,
    d/32 exponent bytes, padded to 16 (the storage format of include/omnikv.h)."""
    return (d // 2 + d // 32 + 15) // 16 * 16


def algorithmic_bytes(cfg, kbits, vbits, lens, key_meta="fp16"):
    """Bytes one decode step must read: packed codes, window metadata, value
    scales and modality tags of every cached token (queries/outputs excluded)."""
    d, H = cfg.head_dim, cfg.kv_heads
    meta = 2 * 2 * d / 32 if key_meta == "fp16" else 2 * mx_record_bytes(d) / 32
    per_token_head = d * kbits / 8 + d * vbits / 8 + meta + 2
    total = 0.0
    for L in lens:
        nwin = math.ceil(L / 32)
        total += nwin * 32 * (H * per_token_head + 1)
    return total


def build_caches(ctx, cfg, nbuf, kbits, vbits, chunk=4096, seed=0):
    import torch
    T = cfg.context
    caches = []
    tags_np = synth.modality_layout(cfg, seed, T)
    for k in range(nbuf):
        c = ctx.alloc_cache(cfg.batch, T)
        c["modality"].copy_(torch.from_numpy(tags_np))
        for t0 in range(0, T, chunk):
            n = min(chunk, T - t0)
            kk = synth.drifting_tensor_device(cfg, tags_np, seed + 17 * k, 0, t0, n)
            vv = synth.drifting_tensor_device(cfg, tags_np, seed + 17 * k, 1, t0, n)
            ctx.quantize_keys(kk, t0, c)
            ctx.quantize_values(vv, t0, c)
            del kk, vv
        caches.append(c)
    torch.cuda.synchronize()
    return caches, tags_np


def time_write_path(ctx, cfg, tags_np, reps=20, seed=3):
    """Time omnikv_quantize_keys / _values on one prefill chunk per sequence.  Several
    input chunks (together over 2.5x the Infinity Cache) are cycled, so the inputs are read
    from HBM as a prefill's freshly computed keys and values would be."""
    import torch
    n = cfg.prefill if cfg.prefill else 4096
    c = ctx.alloc_cache(cfg.batch, n)
    c["modality"].copy_(torch.from_numpy(tags_np[:, :n]))
    chunk_bytes = cfg.batch * n * cfg.kv_heads * cfg.head_dim * (4 if cfg.fp32_inputs else 2)
    nbuf = max(2, math.ceil(2.5 * MALL_BYTES / chunk_bytes))
    ks = [synth.drifting_tensor_device(cfg, tags_np, seed + 31 * i, 0, 0, n) for i in range(nbuf)]
    vs = [synth.drifting_tensor_device(cfg, tags_np, seed + 31 * i, 1, 0, n) for i in range(nbuf)]
    for i in range(3):
        ctx.quantize_keys(ks[i % nbuf], 0, c)
        ctx.quantize_values(vs[i % nbuf], 0, c)
    torch.cuda.synchronize()
    res = {}
    for name, fn, xs in (("keys", ctx.quantize_keys, ks), ("values", ctx.quantize_values, vs)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            fn(xs[r % nbuf], 0, c)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[name] = {"us_per_call": round(us, 2), "input_GBps": round(chunk_bytes / us / 1e3, 1)}
    res["chunk"] = {"tokens_per_sequence": n, "batch": cfg.batch, "dtype": "fp32" if cfg.fp32_inputs else "bf16",
                    "input_buffers": nbuf}
    del ks, vs
    return res


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_16x32k_k2v2_hbm_traffic.txt")
DECODE_SOURCE = os.path.join(ROOT, "decode_attention_fwht_amd", "csrc", "decode.hip")


def decode_code_sha256(path: str = None) -> str:
    """sha256 of the decode source with comments and blank lines removed, and of its build
    flags: a change to the kernel's code or to how it is compiled changes it, a change to
    its comments does not."""
    import hashlib
    import re
    from decode_attention_fwht_amd import build as _build
    text = open(path or DECODE_SOURCE).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    # the flags without the include directories (their absolute paths depend on the checkout)
    flags = " ".join(f for f in _build.FLAGS + _build.EXTRA.get("decode.hip", []) if f != "-I" and "/" not in f)
    return hashlib.sha256((code + "\n" + flags).encode()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode_partial launch from the committed FETCH_SIZE / WRITE_SIZE
    summary, scaled by the copy reference; None unless the summary was taken on this
    workload with the current kernel code."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.lstrip().startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("decode_code_sha256") != decode_code_sha256() or kv.get("workload") != workload:
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(cfg, kbits, vbits, budget_s=15.0, seed=11):
    """The CPU oracle (float64 brute force over the dequantized cache) on a bounded
    sample of the same workload: whole (sequence, KV head) units of a synthetic
    packed cache of this configuration's shape, until the time budget is spent."""
    from oracle import omnikv_oracle as O
    cores = len(os.sched_getaffinity(0))   # the host cores this process may run on
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    d = cfg.head_dim
    signs = synth.rademacher_signs(d, seed)
    U = synth.value_rotations(d, seed)
    lv = O.value_codebook_f16(vbits)
    one = synth.Config(**{**cfg.__dict__, "batch": 1})
    q = synth.queries(cfg, seed)
    done_units, done_bytes, t_used = 0, 0.0, 0.0
    k = 0
    while t_used < budget_s and done_units < cfg.batch * cfg.kv_heads:
        cache = synth.random_packed_cache(one, seed + k, key_bits=kbits, value_bits=vbits)
        b = k % cfg.batch
        lens = np.array([cfg.context], np.int32)
        for kv in range(cfg.kv_heads):
            rows = [(0, kv * cfg.group + h) for h in range(cfg.group)]
            t0 = time.perf_counter()
            O.decode_attention(q[b:b + 1], lens, cache, signs, U, lv, rows=rows)
            t_used += time.perf_counter() - t0
            done_units += 1
            done_bytes += algorithmic_bytes(synth.Config(**{**cfg.__dict__, "batch": 1, "kv_heads": 1}),
                                            kbits, vbits, lens)
            if t_used >= budget_s:
                break
        k += 1
    gbs = done_bytes / t_used / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done_units} of {cfg.batch * cfg.kv_heads} (sequence, KV head) units at "
                      f"{cfg.context} tokens, {cfg.group} query heads each, float64 brute force "
                      f"({t_used:.1f} s; numpy, its BLAS on {blas_threads} threads)"}


def _graph(fn, n):
    """One HIP graph holding fn(0) .. fn(n - 1)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    return g


def _replay_ms(g, reps):
    """Milliseconds of each of `reps` replays of g, each bracketed by events on the stream the
    graph runs on (the current stream)."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for r in range(reps):
        g.replay()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]


def time_stream_append(ctx, cfg, cache, rings, n0, steps=128, reps=10):
    """omnikv_stream_append for the whole batch in lockstep: `steps` consecutive tokens from
    length n0, so the 32-token value windows and the 128-token key groups cross their
    thresholds as in generation (each crossing is one flush launch for the batch).  The
    calls are captured in one graph; microseconds per append call, from its replays."""
    import torch
    B, H, d = cfg.batch, cfg.kv_heads, cfg.head_dim
    g = torch.Generator(device="cuda").manual_seed(7)
    k_new = torch.randn(B, H, d, device="cuda", generator=g).to(torch.bfloat16)
    v_new = torch.randn(B, H, d, device="cuda", generator=g).to(torch.bfloat16)
    t_new = torch.zeros(B, dtype=torch.uint8, device="cuda")
    lens_dev = [torch.full((B,), n0 + i, dtype=torch.int32, device="cuda") for i in range(steps)]
    lens_host = [[n0 + i] * B for i in range(steps)]
    graph = _graph(lambda i: ctx.stream_append(k_new, v_new, t_new, lens_dev[i], lens_host[i], cache, rings), steps)
    graph.replay()
    torch.cuda.synchronize()
    us = [ms * 1e3 / steps for ms in _replay_ms(graph, reps)]
    del graph
    kp = [binding.Context.stream_packed_lengths(n0 + i) for i in range(steps + 1)]
    # a call launches at most one key flush and one value flush, whatever the batch; these count
    # the calls (of `tokens`) that did
    key_flushes = sum(kp[i + 1][0] > kp[i][0] for i in range(steps))
    value_flushes = sum(kp[i + 1][1] > kp[i][1] for i in range(steps))
    return {"append_us": _spread(us), "tokens": steps, "from_length": n0, "batch": B,
            "calls_with_key_flush": int(key_flushes), "calls_with_value_flush": int(value_flushes)}


def _spread(us):
    a = np.asarray(us, np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "samples": int(a.size)}


def time_decode(ctx, cfg, caches, alg, steps, warmup, replays, splits=0):
    """Decode-step timings over the cycled caches.  One step = omnikv_decode_attention over
    every cached token of the batch: the split-KV kernel, then the merge of the splits with
    the batched inverse value rotation.

    warm-up: exactly `warmup` untimed steps, as replays of the step graph (warmup // steps of
    them, then the rest eagerly): a replay bracketed by synchronizations approaches the
    back-to-back replay time only after ~20 ms of back-to-back work (48, 45, 44, ... 41.5 µs
    per step over its first eight replays at config 3, against 40.6 back to back), and eager
    steps launched from Python leave the GPU idle between launches.  head: one replay of the graph of `steps` steps, bracketed by
    synchronizations (the headline timed region: exactly `steps` steps).  spread: `replays`
    further replays of the same graph, each timed by events; a sample is the replay's time /
    steps.  partial / combine: graphs of `steps` launches of one kernel each
    (omnikv_decode_partial, omnikv_decode_combine), replayed `replays` times, medians per
    launch."""
    import torch
    nbuf = len(caches)
    B, T, d = cfg.batch, cfg.context, cfg.head_dim
    q = torch.from_numpy(synth.queries(cfg, 1)).cuda()
    lens = torch.from_numpy(np.full(B, T, np.int32)).cuda()
    ws = torch.empty(ctx.workspace_size(B, T, splits), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, cfg.q_heads, d), dtype=torch.float32, device="cuda")

    def step(i):
        ctx.decode(q, lens, T, caches[i % nbuf], out=out, workspace=ws, num_splits=splits)

    warm_replays, warm_rest = divmod(warmup, steps)
    g_step = _graph(lambda i: step(i), steps)
    g_part = _graph(lambda i: ctx.decode_partial(q, lens, T, caches[i % nbuf], ws, num_splits=splits), steps)
    g_comb = _graph(lambda i: ctx.decode_combine(lens, B, T, ws, out, num_splits=splits), steps)
    torch.cuda.synchronize()
    for i in range(warm_rest):
        step(i)
    for _ in range(warm_replays):
        g_step.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    g_step.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    head_ms = e0.elapsed_time(e1)
    spread = [ms * 1e3 / steps for ms in _replay_ms(g_step, replays)]
    part = [ms * 1e3 / steps for ms in _replay_ms(g_part, replays)]
    comb = [ms * 1e3 / steps for ms in _replay_ms(g_comb, replays)]
    del g_step, g_part, g_comb
    us_head = head_ms * 1e3 / steps
    us_med = float(np.median(spread))
    return {
        "head_ms": head_ms, "wall_s": wall, "us_per_step": us_head,
        "step_us": _spread(spread),
        "GBps_median": round(alg / (us_med * 1e-6) / 1e9, 1),
        "pct_of_hbm_peak_median": round(100 * alg / (us_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "kernels_us": {"decode_partial": _spread(part), "decode_combine": _spread(comb)},
        "partial_frac_of_peak": round(alg / (float(np.median(part)) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "partial_us_median": float(np.median(part)),
        "q": q, "lens": lens, "ws": ws, "out": out,
    }


def decode_config(cid, kbits, vbits, key_meta, steps, warmup, replays, buffers=0):
    """Build this configuration's caches with the write path and time its decode step."""
    import torch
    cfg = synth.CONFIGS[cid]
    d = cfg.head_dim
    ctx = binding.Context(d, cfg.q_heads, cfg.kv_heads, kbits, vbits, synth.rademacher_signs(d, 0),
                          synth.value_rotations(d, 0), key_meta=key_meta)
    lens_np = np.full(cfg.batch, cfg.context, np.int32)
    alg = algorithmic_bytes(cfg, kbits, vbits, lens_np, key_meta)
    nbuf = buffers or max(2, math.ceil(2.5 * MALL_BYTES / alg))
    caches, _ = build_caches(ctx, cfg, nbuf, kbits, vbits)
    r = time_decode(ctx, cfg, caches, alg, steps, warmup, replays)
    res = {"workload": f"{cfg.name} decode step (config {cid})", "codec": f"K{kbits}V{vbits}",
           "key_meta": key_meta, "batch": cfg.batch, "q_heads": cfg.q_heads, "kv_heads": cfg.kv_heads,
           "context": cfg.context, "algorithmic_bytes_per_step": int(alg), "cache_buffers": nbuf,
           "step_us": r["step_us"], "GBps_median": r["GBps_median"],
           "pct_of_hbm_peak_median": r["pct_of_hbm_peak_median"], "kernels_us": r["kernels_us"],
           "partial_frac_of_peak": r["partial_frac_of_peak"]}
    del caches, r
    ctx.close()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--replays", type=int, default=30, help="timed replays of the step graph for the spread")
    ap.add_argument("--config", type=int, default=3, help="workload id (default 3: 16 x 32k, 16Q/2KV/d128)")
    ap.add_argument("--kbits", type=int, default=2)
    ap.add_argument("--vbits", type=int, default=2)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--buffers", type=int, default=0, help="independent caches cycled (0: enough to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other configurations (configs 4 and 5, K2V2 and K4V4, and the 4-bit and config-5 write paths)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-reference-mib", type=int, default=0,
                    help="also run a plain device copy (out = 1 * in, fp32) of this many MiB, the "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(one GPU holds one shard of the KV heads; no collective is implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.config]
    d = cfg.head_dim
    signs = synth.rademacher_signs(d, 0)
    U = synth.value_rotations(d, 0)
    ctx = binding.Context(d, cfg.q_heads, cfg.kv_heads, args.kbits, args.vbits, signs, U)

    lens_np = np.full(cfg.batch, cfg.context, np.int32)
    alg = algorithmic_bytes(cfg, args.kbits, args.vbits, lens_np)
    nbuf = args.buffers or max(2, math.ceil(2.5 * MALL_BYTES / alg))
    caches, tags_np = build_caches(ctx, cfg, nbuf, args.kbits, args.vbits)
    write_path = time_write_path(ctx, cfg, tags_np)
    T = cfg.context

    r = time_decode(ctx, cfg, caches, alg, args.steps, args.warmup, args.replays, args.splits)
    q, lens, ws, out = r["q"], r["lens"], r["ws"], r["out"]

    # the same step for streamed sequences: the last stream_value_packed tokens (the
    # 128-token sliding value window) come from rings of recent tokens
    rings = ctx.alloc_rings(cfg.batch, 256)
    rings["k"].normal_()
    rings["v"].normal_()
    g_stream = _graph(lambda i: ctx.decode_streaming(q, lens, T, caches[i % nbuf], rings, out=out, workspace=ws,
                                                     num_splits=args.splits), args.steps)
    g_stream.replay()
    torch.cuda.synchronize()
    stream_us = [ms * 1e3 / args.steps for ms in _replay_ms(g_stream, max(5, args.replays // 3))]
    del g_stream
    append = time_stream_append(ctx, cfg, caches[0], rings, T - 192)

    # the same step with MXFP4 key metadata (the paper's default format): its own context
    # and caches, enough of them to exceed the MALL
    mx = decode_config(args.config, args.kbits, args.vbits, "mxfp4", args.steps, args.warmup,
                       max(5, args.replays // 3), args.buffers)
    kp, vp = binding.Context.stream_packed_lengths(T)
    ms_per_step = r["head_ms"] / args.steps
    kern_avg_s = r["partial_us_median"] * 1e-6
    value = alg / (ms_per_step / 1e3) / 1e9
    achieved = alg / kern_avg_s / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name} decode step (config {cfg.cid})",
            "batch": cfg.batch, "q_heads": cfg.q_heads, "kv_heads": cfg.kv_heads, "head_dim": d,
            "context": cfg.context, "codec": f"K{args.kbits}V{args.vbits}", "key_meta": "fp16", "window": 32,
            "cache_buffers": nbuf, "algorithmic_bytes_per_step": int(alg),
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "step_us": r["step_us"],
        "wall_s_timed_region": round(r["wall_s"], 6),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels_us": r["kernels_us"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{cfg.name} K{args.kbits}V{args.vbits} splits {args.splits}")},
        "write_path": write_path,
        "streaming": {"step_us": _spread(stream_us), "recent_tokens_per_sequence": T - vp, "packed_key_tokens": kp,
                      "append": append},
        "key_meta_mxfp4": mx,
    }
    del caches, rings, r, q, lens, ws, out
    ctx.close()
    torch.cuda.empty_cache()
    if not args.no_other_configs:
        others = {}
        for cid, kb, vb in ((4, 2, 2), (4, 4, 4), (5, 2, 2), (5, 4, 4)):
            others[f"config{cid}_K{kb}V{vb}"] = decode_config(cid, kb, vb, "fp16", 10, 20, 10)
        # the write path at 4 bits: this configuration's chunk, and the config-5 prefill at both widths
        ctx4 = binding.Context(d, cfg.q_heads, cfg.kv_heads, 4, 4, signs, U)
        others[f"config{cfg.cid}_write_K4V4"] = time_write_path(
            ctx4, cfg, synth.modality_layout(cfg, 0, max(cfg.context, cfg.prefill or 4096)), reps=20)
        ctx4.close()
        # the same chunk handed over as fp32 (both codecs' matrix-core paths take fp32 too)
        cfg32 = synth.Config(**{**cfg.__dict__, "fp32_inputs": True})
        ctx2 = binding.Context(d, cfg.q_heads, cfg.kv_heads, 2, 2, signs, U)
        others[f"config{cfg.cid}_write_fp32_K2V2"] = time_write_path(
            ctx2, cfg32, synth.modality_layout(cfg, 0, max(cfg.context, cfg.prefill or 4096)), reps=20)
        ctx2.close()
        torch.cuda.empty_cache()
        cfg5 = synth.CONFIGS[5]
        tags5 = synth.modality_layout(cfg5, 0, cfg5.prefill)
        for bits in (2, 4):
            ctx5 = binding.Context(cfg5.head_dim, cfg5.q_heads, cfg5.kv_heads, bits, bits, signs, U)
            others[f"config5_prefill_write_K{bits}V{bits}"] = time_write_path(ctx5, cfg5, tags5, reps=10)
            ctx5.close()
            torch.cuda.empty_cache()
        res["configs"] = others
    if args.copy_reference_mib:
        n = args.copy_reference_mib * (1 << 20) // 4
        src = torch.rand(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        res["copy_reference_mib"] = args.copy_reference_mib
        del src, dst
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.kbits, args.vbits, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
