"""Benchmark: K2V2 decode attention over the packed OmniKVQuant cache on one MI355X.

One step = one decode step of the whole batch: the split-KV partial pass and the
merge + batched inverse value rotation (omnikv_decode_partial then
omnikv_decode_combine) over every cached token of every sequence.  The packed
caches are built before timing by the library's own write path (keys and values
of synthetic drifting K/V, quantized in prefill-sized chunks), and several
independent caches are cycled so that a step never finds its cache in the 256 MB
Infinity Cache: the timed bytes come from HBM.  The K timed steps are captured in
one HIP graph and replayed once between two synchronisations (two short kernels per
step would otherwise wait on Python launch overhead); the per-kernel averages come
from graphs of K partial-only and K combine-only launches.  The write path itself is
timed separately on one prefill chunk per sequence and reported under "write_path".

Prints one JSON line: the headline (effective KV GB/s of the decode step), the
roofline of the partial kernel, the write-path timings and a CPU-oracle
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
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
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
                      f"({t_used:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload id (default 3: 16 x 32k, 16Q/2KV/d128)")
    ap.add_argument("--kbits", type=int, default=2)
    ap.add_argument("--vbits", type=int, default=2)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--buffers", type=int, default=0, help="independent caches cycled (0: enough to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    q = torch.from_numpy(synth.queries(cfg, 1)).cuda()
    lens = torch.from_numpy(lens_np).cuda()
    T = cfg.context
    ws = torch.empty(ctx.workspace_size(cfg.batch, T, args.splits), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.batch, cfg.q_heads, d), dtype=torch.float32, device="cuda")

    def step(i):
        c = caches[i % nbuf]
        ctx.decode_partial(q, lens, T, c, ws, num_splits=args.splits)
        ctx.decode_combine(lens, cfg.batch, T, ws, out, num_splits=args.splits)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed work is replayed from HIP graphs: one decode step is two short kernels, and
    # launching them one by one from Python would leave the GPU waiting for the host.
    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    def timed_replay(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), time.perf_counter() - t0

    g_step = capture(lambda i: step(args.warmup + i), args.steps)
    g_part = capture(lambda i: ctx.decode_partial(q, lens, T, caches[i % nbuf], ws, num_splits=args.splits),
                     args.steps)
    g_comb = capture(lambda i: ctx.decode_combine(lens, cfg.batch, T, ws, out, num_splits=args.splits),
                     args.steps)
    # the same step for streamed sequences: the last stream_value_packed tokens (the
    # 128-token sliding value window) come from rings of recent tokens
    rings = ctx.alloc_rings(cfg.batch, 256)
    rings["k"].normal_()
    rings["v"].normal_()
    g_stream = capture(lambda i: ctx.decode_streaming(q, lens, T, caches[i % nbuf], rings, out=out, workspace=ws,
                                                      num_splits=args.splits), args.steps)
    g_step.replay()  # untimed first replay
    g_stream.replay()
    torch.cuda.synchronize()
    step_ms, wall = timed_replay(g_step)
    part_ms, _ = timed_replay(g_part)
    comb_ms, _ = timed_replay(g_comb)
    stream_ms, _ = timed_replay(g_stream)

    # the same step with MXFP4 key metadata (the paper's default format): its own context
    # and caches, enough of them to exceed the MALL
    ctx_mx = binding.Context(d, cfg.q_heads, cfg.kv_heads, args.kbits, args.vbits, signs, U, key_meta="mxfp4")
    alg_mx = algorithmic_bytes(cfg, args.kbits, args.vbits, lens_np, key_meta="mxfp4")
    nbuf_mx = args.buffers or max(2, math.ceil(2.5 * MALL_BYTES / alg_mx))
    caches_mx, _ = build_caches(ctx_mx, cfg, nbuf_mx, args.kbits, args.vbits)
    ws_mx = torch.empty(ctx_mx.workspace_size(cfg.batch, T, args.splits), dtype=torch.uint8, device="cuda")

    def step_mx(i):
        c = caches_mx[i % nbuf_mx]
        ctx_mx.decode_partial(q, lens, T, c, ws_mx, num_splits=args.splits)
        ctx_mx.decode_combine(lens, cfg.batch, T, ws_mx, out, num_splits=args.splits)

    for i in range(args.warmup):
        step_mx(i)
    g_mx = capture(lambda i: step_mx(args.warmup + i), args.steps)
    g_mx_part = capture(lambda i: ctx_mx.decode_partial(q, lens, T, caches_mx[i % nbuf_mx], ws_mx,
                                                        num_splits=args.splits), args.steps)
    g_mx.replay()
    torch.cuda.synchronize()
    mx_ms, _ = timed_replay(g_mx)
    mx_part_ms, _ = timed_replay(g_mx_part)
    del caches_mx, g_mx, g_mx_part
    ctx_mx.close()
    kp, vp = binding.Context.stream_packed_lengths(T)
    ms_per_step = step_ms / args.steps
    us_step_med = ms_per_step * 1e3
    part_avg_s = part_ms / args.steps / 1e3

    value = alg / (ms_per_step / 1e3) / 1e9
    achieved = alg / part_avg_s / 1e9
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
            "context": cfg.context, "codec": f"K{args.kbits}V{args.vbits}", "window": 32,
            "cache_buffers": nbuf, "algorithmic_bytes_per_step": int(alg),
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "wall_s_timed_region": round(wall, 6),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels_us": {"decode_partial_avg": round(part_avg_s * 1e6, 2),
                       "decode_combine_avg": round(comb_ms / args.steps * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{cfg.name} K{args.kbits}V{args.vbits} splits {args.splits}")},
        "write_path": write_path,
        "streaming": {"us_per_step": round(stream_ms / args.steps * 1e3, 2),
                      "recent_tokens_per_sequence": T - vp, "packed_key_tokens": kp},
        "key_meta_mxfp4": {"us_per_step": round(mx_ms / args.steps * 1e3, 2),
                           "decode_partial_avg_us": round(mx_part_ms / args.steps * 1e3, 2),
                           "algorithmic_bytes_per_step": int(alg_mx),
                           "GBps": round(alg_mx / (mx_ms / args.steps / 1e3) / 1e9, 1),
                           "cache_buffers": nbuf_mx},
    }
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
