"""MXFP4 key metadata (the pages' default format, [paper] §3.1 Implementation details)
through the C ABI against the oracle.

Bars as for the fp16 metadata: the MXFP4 records (E2M1 codes, E8M0 exponents, zero
padding) and the key codes are bit-exact; decode outputs over the same packed cache are
within 1e-3 max row relative error of the oracle's float64 attention.
"""
import numpy as np
import pytest

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import synth
from tests.gpu_helpers import (bf16_tensor, cache_to_device, from_dev, make_context, row_errors,
                               sampled_unit_rows, say, to_dev)

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _inputs(cfg, n, seed=0):
    tags = synth.modality_layout(cfg, seed, max(cfg.context, n))
    k = synth.drifting_tensor(cfg, tags, seed, 0, 0, n)
    v = synth.drifting_tensor(cfg, tags, seed, 1, 0, n)
    return tags, k, v


def _dev_kv(cfg, x):
    import torch
    return torch.from_numpy(x).cuda() if cfg.fp32_inputs else bf16_tensor(x)


def _check_keys(cache, k, signs, kbits, d):
    with np.errstate(all="ignore"):
        kc, km, ks = O.quantize_keys(k, signs, kbits, meta="mxfp4")
    gm, gs = from_dev(cache["k_min"], np.uint8), from_dev(cache["k_scale"], np.uint8)
    for name, g, o in (("k_min", gm, km), ("k_scale", gs, ks)):
        if not np.array_equal(g, o):
            bad = np.argwhere(g != o)
            raise AssertionError(f"{name}: {len(bad)} record bytes differ, first at {bad[:4].tolist()}")
    gk = from_dev(cache["k_codes"], np.uint32)
    if not np.array_equal(gk, kc):
        g = O.unpack_windows(gk, "key", d, kbits)
        o = O.unpack_windows(kc, "key", d, kbits)
        bad = np.argwhere(g != o)
        raise AssertionError(f"{len(bad)} key codes differ, first at {bad[:4].tolist()}")


@pytest.mark.parametrize("cid,kbits,n", [
    (1, 2, 256), (1, 4, 256), (2, 2, 10240), (2, 4, 2048), (3, 2, 4096), (3, 4, 4096),
])
def test_mx_quantize_keys_parity(cid, kbits, n):
    import torch
    cfg = synth.CONFIGS[cid]
    say(f"[mx-keys] cfg{cid} K{kbits} n={n}")
    ctx, signs, U, lv = make_context(cfg, kbits, 2, key_meta="mxfp4")
    assert ctx.key_meta_bytes == O.mx_record_bytes(cfg.head_dim)
    tags, k, v = _inputs(cfg, n)
    cache = ctx.alloc_cache(cfg.batch, n)
    ctx.quantize_keys(_dev_kv(cfg, k), 0, cache)
    torch.cuda.synchronize()
    _check_keys(cache, k, signs, kbits, cfg.head_dim)
    ctx.close()


@pytest.mark.parametrize("cid,kbits", [(2, 2), (1, 4)])
def test_mx_quantize_keys_degenerate_windows(cid, kbits):
    """All-zero window (exponent byte 0), identical tokens (zero steps), negative zeros,
    tiny and huge tokens (exponents near both ends of E8M0), one nonzero channel."""
    import torch
    cfg = synth.CONFIGS[cid]
    n = 256
    say(f"[mx-keys-degenerate] cfg{cid} K{kbits}")
    ctx, signs, U, lv = make_context(cfg, kbits, 2, key_meta="mxfp4")
    tags, k, v = _inputs(cfg, n)
    k = k.copy()
    k[:, 0:32] = 0.0
    k[:, 32:64] = k[:, 32:33]
    k[:, 64:96] = np.where(k[:, 64:96] < 0, -0.0, k[:, 64:96])
    k[:, 64:70] = -0.0
    k[:, 96:99] *= 1e-30
    k[:, 128:130] *= 1e30
    k[:, 160:192] = 0.0
    k[:, 160:192, :, 7] = np.linspace(-3.0, 2.0, 32, dtype=np.float32)[None, :, None]
    k[:, 192:224] *= 1e-38                   # window 6: subnormal-range tokens
    if not cfg.fp32_inputs:
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
    cache = ctx.alloc_cache(cfg.batch, n)
    ctx.quantize_keys(_dev_kv(cfg, k), 0, cache)
    torch.cuda.synchronize()
    _check_keys(cache, k, signs, kbits, cfg.head_dim)
    ctx.close()


def _oracle_mx_cache(cfg, signs, U, lv, T, kbits, vbits, seed=0):
    tags, k, v = _inputs(cfg, T, seed)
    kc, km, ks = O.quantize_keys(k, signs, kbits, meta="mxfp4")
    vc, vs = O.quantize_values(v, tags[:, :T], U, lv, vbits)
    return dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags[:, :T].copy(),
                key_bits=kbits, value_bits=vbits, t_cap=T)


@pytest.mark.parametrize("cid,kbits,vbits,T,ragged", [
    (1, 2, 2, 256, False), (1, 2, 2, 256, True), (1, 4, 4, 256, True),
    (2, 2, 2, 10240, True), (2, 4, 4, 4096, True), (2, 2, 4, 2048, False),
])
def test_mx_decode_parity_oracle_cache(cid, kbits, vbits, T, ragged):
    import torch
    cfg = synth.CONFIGS[cid]
    say(f"[mx-decode] cfg{cid} K{kbits}V{vbits} T={T} ragged={ragged}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits, key_meta="mxfp4")
    cache = _oracle_mx_cache(cfg, signs, U, lv, T, kbits, vbits)
    B = cfg.batch
    q = synth.queries(cfg, 3)
    lens = np.full(B, T, np.int32)
    if ragged:
        lens[:] = [T - 17 - 5 * b for b in range(B)]
    out = ctx.decode(to_dev(q), to_dev(lens), T, cache_to_device(cache))
    torch.cuda.synchronize()
    err = row_errors(from_dev(out), O.decode_attention(q, lens, cache, signs, U, lv))
    say(f"    max row error {err.max():.3e}")
    assert err.max() <= TOL
    ctx.close()


def _record_sweep_cache(cfg, T, kbits, vbits, seed):
    """Packed cache with MXFP4 records drawn directly: every element code in every
    window, exponents 2^-9 .. 2^5 (the decoded values stay inside fp16), steps >= 0."""
    r = np.random.default_rng(seed)
    base = synth.random_packed_cache(cfg, seed, key_bits=kbits, value_bits=vbits, length=T)
    B, H, nw = cfg.batch, cfg.kv_heads, T // 32
    d = cfg.head_dim
    mcodes = r.integers(0, 16, (B, H, nw, d)).astype(np.uint8)
    scodes = r.integers(0, 8, (B, H, nw, d)).astype(np.uint8)
    mexp = r.integers(118, 130, (B, H, nw, d // 32)).astype(np.uint8)
    sexp = r.integers(116, 128, (B, H, nw, d // 32)).astype(np.uint8)
    base["k_min"] = O.mx_pack_record(mcodes, mexp)
    base["k_scale"] = O.mx_pack_record(scodes, sexp)
    return base


@pytest.mark.parametrize("cid,kbits,vbits", [(2, 2, 2), (2, 4, 4), (1, 2, 2)])
def test_mx_decode_record_sweep(cid, kbits, vbits):
    import torch
    cfg = synth.CONFIGS[cid]
    T = 2048 if cid == 2 else 256
    say(f"[mx-decode-sweep] cfg{cid} K{kbits}V{vbits} T={T}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits, key_meta="mxfp4")
    cache = _record_sweep_cache(cfg, T, kbits, vbits, 11 + kbits)
    q = synth.queries(cfg, 5) * np.float32(0.05)   # keep the softmax from collapsing onto one token
    lens = np.array([T - 9 * b for b in range(cfg.batch)], np.int32)
    out = ctx.decode(to_dev(q), to_dev(lens), T, cache_to_device(cache))
    torch.cuda.synchronize()
    err = row_errors(from_dev(out), O.decode_attention(q, lens, cache, signs, U, lv))
    say(f"    max row error {err.max():.3e}")
    assert err.max() <= TOL
    ctx.close()


def _drift_range_mx_cache(cfg, T, kbits, vbits, seed):
    """Packed cache whose MXFP4 records encode (with the oracle's encoder) the key minima and
    steps of the fp16-metadata tests' synthetic cache, i.e. the ranges a drifting N(0,1)-like
    cache produces, so that unscaled queries give the same softmax sharpness as there."""
    base = synth.random_packed_cache(cfg, seed, key_bits=kbits, value_bits=vbits, length=T)
    m = O.f16_to_f32(base["k_min"])
    s = O.f16_to_f32(base["k_scale"])
    base["k_min"] = O.mx_pack_record(*O.mxfp4_encode(m))
    base["k_scale"] = O.mx_pack_record(*O.mxfp4_encode(s))
    return base


@pytest.mark.parametrize("cid,kbits,vbits", [(3, 2, 2), (4, 2, 2), (4, 4, 4), (5, 2, 2), (5, 4, 4)])
def test_mx_decode_full_size_sampled(cid, kbits, vbits):
    """The configurations' full sizes, in the launch the benchmark times: records encoding the
    drifting cache's key ranges, unscaled queries, every query head of sampled units against
    the oracle."""
    import torch
    cfg = synth.CONFIGS[cid]
    T = cfg.context
    say(f"[mx-decode-sampled] cfg{cid} K{kbits}V{vbits} B={cfg.batch} T={T}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits, key_meta="mxfp4")
    cache = _drift_range_mx_cache(cfg, T, kbits, vbits, 21)
    lens = synth.seq_lens(cfg, ragged=True, seed=cid)
    lens[0] = T
    q = synth.queries(cfg, 4)
    out = from_dev(ctx.decode(to_dev(q), to_dev(lens), T, cache_to_device(cache)))
    torch.cuda.synchronize()
    rows = sampled_unit_rows(cfg, cid)
    ref = O.decode_attention(q, lens, cache, signs, U, lv, rows=rows)
    bi, hi = [r[0] for r in rows], [r[1] for r in rows]
    err = row_errors(out[bi, hi], ref[bi, hi])
    say(f"    rows {rows} max row error {err.max():.3e}")
    assert err.max() <= TOL and np.all(np.isfinite(out))
    ctx.close()


@pytest.mark.parametrize("cid,lens,cap,kbits,vbits", [
    (1, [200, 257, 129], 256, 4, 4),
    (2, [300, 97, 515, 160], 256, 2, 2),
])
def test_mx_streaming_decode_parity(cid, lens, cap, kbits, vbits):
    """Packed prefix with MXFP4 key records + recent tokens in rings."""
    import torch
    cfg = synth.CONFIGS[cid]
    B = len(lens)
    T = max(32, ((max(lens) + 31) // 32) * 32)
    say(f"[mx-stream-decode] cfg{cid} K{kbits}V{vbits} lens {lens} ring {cap}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits, key_meta="mxfp4")
    tags, k, v = _inputs(cfg, T, 3)
    if not cfg.fp32_inputs:
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
        v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    tags, k, v = tags[:1, :T].repeat(B, 0), np.repeat(k[:1], B, 0), np.repeat(v[:1], B, 0)
    kc, km, ks = O.quantize_keys(k, signs, kbits, meta="mxfp4")
    vc, vs = O.quantize_values(v, tags, U, lv, vbits)
    host = dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags,
                key_bits=kbits, value_bits=vbits)
    dt = torch.float32 if cfg.fp32_inputs else torch.bfloat16
    rings = ctx.alloc_rings(B, cap, dtype=dt)
    rk = np.zeros((B, cap) + k.shape[2:], np.float32)
    rv = np.zeros_like(rk)
    for b, n in enumerate(lens):
        _, vp = O.stream_packed_lengths(n)
        for t in range(max(vp, n - cap), n):
            rk[b, t % cap], rv[b, t % cap] = k[b, t], v[b, t]
    rings["k"].copy_(torch.from_numpy(rk).to(dt).cuda())
    rings["v"].copy_(torch.from_numpy(rv).to(dt).cuda())
    q_np = synth.queries(cfg, 4, B)
    out = from_dev(ctx.decode_streaming(torch.from_numpy(q_np).cuda(), to_dev(np.array(lens, np.int32)), T,
                                        cache_to_device(host), rings))
    ref = O.decode_attention_streaming(q_np, lens, host, k, v, signs, U, lv)
    err = row_errors(out, ref)
    say(f"    max row error {err.max():.3e}")
    assert err.max() <= TOL
    ctx.close()


def test_mx_stream_append_key_flush():
    """Appends through the streaming path write MXFP4 key records bit-exactly (keys flush
    every 128 tokens through the same quantizer, at a byte offset per sequence)."""
    import torch
    cfg = synth.CONFIGS[2]
    B, T, cap = 2, 320, 256
    say(f"[mx-stream-append] cfg2 B={B} {T} tokens")
    ctx, signs, U, lv = make_context(cfg, key_meta="mxfp4")
    tags, k, v = _inputs(cfg, T, 5)
    k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
    tags, k, v = tags[:1, :T].repeat(B, 0), np.repeat(k[:1], B, 0), np.repeat(v[:1], B, 0)
    cache = ctx.alloc_cache(B, T)
    rings = ctx.alloc_rings(B, cap)
    kd, vd = bf16_tensor(k), bf16_tensor(v)
    tg = to_dev(tags)
    lens = np.zeros(B, np.int64)
    for step in range(T):
        ctx.stream_append(kd[:, step].contiguous(), vd[:, step].contiguous(), tg[:, step].contiguous(),
                          to_dev(lens.astype(np.int32)), lens.tolist(), cache, rings)
        lens += 1
    torch.cuda.synchronize()
    kp, _ = O.stream_packed_lengths(T)
    okc, okm, oks = O.quantize_keys(k[:, :kp], signs, cfg.key_bits, meta="mxfp4")
    nw = kp // 32
    assert np.array_equal(from_dev(cache["k_min"], np.uint8)[:, :, :nw], okm)
    assert np.array_equal(from_dev(cache["k_scale"], np.uint8)[:, :, :nw], oks)
    assert np.array_equal(from_dev(cache["k_codes"], np.uint32)[:, :, :nw], okc)
    ctx.close()


def test_mx_decode_split_invariance():
    import torch
    cfg = synth.CONFIGS[2]
    T = 10240
    say("[mx-split-invariance] cfg2")
    ctx, signs, U, lv = make_context(cfg, key_meta="mxfp4")
    cache = cache_to_device(_record_sweep_cache(cfg, T, 2, 2, 31))
    q = to_dev(synth.queries(cfg, 7) * np.float32(0.05))
    lens = to_dev(np.array([T - 3], np.int32))
    outs = [from_dev(ctx.decode(q, lens, T, cache, num_splits=s)) for s in (1, 3, 0, 64, 320)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert row_errors(o, outs[0]).max() < 3e-5
    ctx.close()


def test_mx_decode_graph_replay_matches_eager():
    """The MXFP4 two-launch decode step captured in a HIP graph gives the eager result bit
    for bit on every replay, with eager work between replays."""
    import torch
    cfg = synth.CONFIGS[2]
    T = 4096
    say("[mx-graph-replay] cfg2")
    ctx, signs, U, lv = make_context(cfg, key_meta="mxfp4")
    caches = [cache_to_device(_record_sweep_cache(cfg, T, 2, 2, 40 + i)) for i in range(2)]
    q = to_dev(synth.queries(cfg, 5) * np.float32(0.05))
    lens = to_dev(np.array([T - 9], np.int32))
    ws = torch.empty(ctx.workspace_size(cfg.batch, T), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((cfg.batch, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
            for _ in range(2)]
    eager = []
    for i in range(2):
        ctx.decode_partial(q, lens, T, caches[i], ws)
        ctx.decode_combine(lens, cfg.batch, T, ws, outs[i])
        eager.append(outs[i].clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(2):
            ctx.decode_partial(q, lens, T, caches[i], ws)
            ctx.decode_combine(lens, cfg.batch, T, ws, outs[i])
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], eager[i]), (rep, i)
        ctx.decode(q, lens, T, caches[(rep + 1) % 2])
        torch.cuda.synchronize()
    ctx.close()
