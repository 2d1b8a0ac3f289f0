"""HIP path vs the CPU oracle, element by element, through the C ABI.

Bars (fixed by the target of the build):
  * packed codes, k_min, k_scale, v_scale: bit-exact (the codec's fp32 order is
    part of its definition and both sides follow it);
  * decode outputs: per (sequence, query head) row, max |gpu - oracle| over the
    channels divided by max |oracle| <= 1e-3 (fp32 accumulation on the GPU,
    float64 brute force in the oracle over the same packed cache).
Small sizes are compared in full; the configurations' full sizes are compared
on sampled windows (codec) or sampled rows (decode).
"""
import math

import numpy as np
import pytest

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import binding, synth
from tests.gpu_helpers import (bf16_tensor, cache_to_device, from_dev, make_context, row_errors,
                               sampled_unit_rows, say, to_dev)

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _inputs(cfg, n, seed=0, t0=0):
    tags = synth.modality_layout(cfg, seed, max(cfg.context, t0 + n))
    k = synth.drifting_tensor(cfg, tags, seed, 0, t0, n)
    v = synth.drifting_tensor(cfg, tags, seed, 1, t0, n)
    return tags, k, v


def _dev_kv(cfg, x):
    import torch
    return torch.from_numpy(x).cuda() if cfg.fp32_inputs else bf16_tensor(x)


# ----------------------------------------------------------------------------- codec, full compare
@pytest.mark.parametrize("cid,kbits,vbits,n", [
    (1, 2, 2, 256), (1, 4, 4, 256), (2, 2, 2, 10240), (2, 4, 4, 2048), (3, 2, 2, 4096), (3, 4, 2, 4096),
])
def test_quantize_parity_full(cid, kbits, vbits, n):
    import torch
    cfg = synth.CONFIGS[cid]
    say(f"[codec] cfg{cid} K{kbits}V{vbits} n={n}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits)
    tags, k, v = _inputs(cfg, n)
    t_cap = n
    cache = ctx.alloc_cache(cfg.batch, t_cap)
    cache["modality"].copy_(to_dev(tags[:, :t_cap]))
    ctx.quantize_keys(_dev_kv(cfg, k), 0, cache)
    ctx.quantize_values(_dev_kv(cfg, v), 0, cache)
    torch.cuda.synchronize()
    kc, km, ks = O.quantize_keys(k, signs, kbits)
    vc, vs = O.quantize_values(v, tags[:, :n], U, lv, vbits)
    assert np.array_equal(from_dev(cache["k_min"], np.uint16), km)
    assert np.array_equal(from_dev(cache["k_scale"], np.uint16), ks)
    gk = from_dev(cache["k_codes"], np.uint32)
    assert np.array_equal(gk, kc), f"{np.count_nonzero(gk != kc)} key words differ"
    assert np.array_equal(from_dev(cache["v_scale"], np.uint16), vs)
    gv = from_dev(cache["v_codes"], np.uint32)
    if not np.array_equal(gv, vc):
        gcodes = O.unpack_windows(gv, "value", cfg.head_dim, vbits)
        ocodes = O.unpack_windows(vc, "value", cfg.head_dim, vbits)
        raise AssertionError(f"{np.count_nonzero(gcodes != ocodes)} of {gcodes.size} value codes differ")
    ctx.close()


_SYM16 = (0.1, 0.35, 0.6, 0.9, 1.2, 1.6, 2.0, 2.6)


@pytest.mark.parametrize("vbits,levels", [(2, None), (4, None), (2, (-1.3, -0.35, 0.4, 1.7))])
def test_quantize_values_fp32_inputs(vbits, levels):
    """fp32 values through the matrix-core path (each value as a bf16 hi part and a rounded
    bf16 lo part, the remainder inside the near-threshold tolerance): codes and scales
    bit-exact against the oracle's fp32 definition, d = 128, 4096 tokens of drift data with
    full 24-bit significands, the built-in codebooks and an asymmetric caller codebook."""
    import torch
    cfg = synth.CONFIGS[2]
    n = 4096
    say(f"[codec-fp32] cfg2 V{vbits} n={n} levels={levels}")
    if levels is None:
        ctx, signs, U, lv = make_context(cfg, 2, vbits)
    else:
        lv = O.f16_bits(np.asarray(levels, np.float32))
        signs, U = synth.rademacher_signs(cfg.head_dim, 0), synth.value_rotations(cfg.head_dim, 0)
        ctx = binding.Context(cfg.head_dim, cfg.q_heads, cfg.kv_heads, 2, vbits, signs, U, value_codebook=lv)
    f32 = synth.Config(**{**cfg.__dict__, "fp32_inputs": True})
    tags, k, v = _inputs(f32, n)
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert np.count_nonzero(v.view(np.uint32) & 0xFFFF) > v.size // 2   # not bf16 in disguise
    cache = ctx.alloc_cache(cfg.batch, n)
    cache["modality"].copy_(to_dev(tags[:, :n]))
    ctx.quantize_values(torch.from_numpy(v).cuda(), 0, cache)
    torch.cuda.synchronize()
    vc, vs = O.quantize_values(v, tags[:, :n], U, lv, vbits)
    assert np.array_equal(from_dev(cache["v_scale"], np.uint16), vs)
    gv = from_dev(cache["v_codes"], np.uint32)
    if not np.array_equal(gv, vc):
        gcodes = O.unpack_windows(gv, "value", cfg.head_dim, vbits)
        ocodes = O.unpack_windows(vc, "value", cfg.head_dim, vbits)
        raise AssertionError(f"{np.count_nonzero(gcodes != ocodes)} of {gcodes.size} value codes differ")
    ctx.close()


@pytest.mark.parametrize("levels", [(-1.3, -0.35, 0.4, 1.7), (-2.0, -0.5, 0.5, 2.0),
                                    tuple(np.round(np.linspace(-2.3, 1.9, 16) + 0.07 * np.sin(np.arange(16)), 3)),
                                    tuple(-x for x in reversed(_SYM16)) + _SYM16])
def test_quantize_values_custom_codebook(levels):
    """A caller's value codebook (2 or 4 bits): boundaries symmetric about 0 take the value
    quantizer's sign-and-magnitude classification, any others the general one; both must
    give the oracle's codes with that codebook."""
    import torch
    cfg = synth.CONFIGS[3]
    n = 1024
    bits = 2 if len(levels) == 4 else 4
    say(f"[codec] custom {bits}-bit codebook {levels}")
    d = cfg.head_dim
    signs = synth.rademacher_signs(d, 0)
    U = synth.value_rotations(d, 0, 3)
    lv = O.f16_bits(np.asarray(levels, np.float32))
    ctx = binding.Context(d, cfg.q_heads, cfg.kv_heads, bits, bits, signs, U, value_codebook=lv)
    assert np.array_equal(ctx.value_codebook(), lv)
    tags, k, v = _inputs(cfg, n)
    cache = ctx.alloc_cache(cfg.batch, n)
    cache["modality"].copy_(to_dev(tags[:, :n]))
    ctx.quantize_values(_dev_kv(cfg, v), 0, cache)
    torch.cuda.synchronize()
    vc, vs = O.quantize_values(v, tags[:, :n], U, lv, bits)
    assert np.array_equal(from_dev(cache["v_scale"], np.uint16), vs)
    gv = from_dev(cache["v_codes"], np.uint32)
    if not np.array_equal(gv, vc):
        gcodes = O.unpack_windows(gv, "value", d, bits)
        ocodes = O.unpack_windows(vc, "value", d, bits)
        raise AssertionError(f"{np.count_nonzero(gcodes != ocodes)} of {gcodes.size} value codes differ")
    ctx.close()


def test_quantize_offset_chunk_writes_only_its_windows():
    import torch
    cfg = synth.CONFIGS[2]
    ctx, signs, U, lv = make_context(cfg)
    t0, n, t_cap = 96, 160, 512
    tags, k, v = _inputs(cfg, n, t0=t0)
    cache = ctx.alloc_cache(cfg.batch, t_cap)
    for key in ("k_codes", "v_codes"):
        cache[key].fill_(0x5A5A5A5A)
    for key in ("k_min", "k_scale", "v_scale"):
        cache[key].fill_(0x5A5A)
    cache["modality"].copy_(to_dev(tags[:, :t_cap]))
    ctx.quantize_keys(_dev_kv(cfg, k), t0, cache)
    ctx.quantize_values(_dev_kv(cfg, v), t0, cache)
    torch.cuda.synchronize()
    kc, km, ks = O.quantize_keys(k, signs, 2)
    vc, vs = O.quantize_values(v, tags[:, t0:t0 + n], U, lv, 2)
    w0, w1 = t0 // 32, (t0 + n) // 32
    gkc = from_dev(cache["k_codes"], np.uint32)
    assert np.array_equal(gkc[:, :, w0:w1], kc)
    assert np.all(gkc[:, :, :w0] == 0x5A5A5A5A) and np.all(gkc[:, :, w1:] == 0x5A5A5A5A)
    assert np.array_equal(from_dev(cache["k_min"], np.uint16)[:, :, w0:w1], km)
    assert np.array_equal(from_dev(cache["v_codes"], np.uint32)[:, :, w0:w1], vc)
    gvs = from_dev(cache["v_scale"], np.uint16)
    assert np.array_equal(gvs[:, :, t0:t0 + n], vs)
    assert np.all(gvs[:, :, :t0] == 0x5A5A) and np.all(gvs[:, :, t0 + n:] == 0x5A5A)
    ctx.close()


@pytest.mark.parametrize("vbits", [2, 4])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_values_degenerate_tokens(vbits, dtype):
    """Value codes for tokens at the edges of the matrix-core path (bf16 values, or fp32 values
    as two bf16 parts each): an all-zero window,
    zero tokens, tokens whose squares underflow (sum of squares 0, so sigma = 0 and every
    rotated value lies within the error bound of a threshold: 3 such tokens in a window are
    recomputed one element at a time, 8 force the whole window through the sequential sum),
    and a token whose sum of squares overflows to inf."""
    import torch
    cfg = synth.CONFIGS[2]
    n = 256
    say(f"[codec-degenerate] cfg2 V{vbits} n=256 {dtype}")
    ctx, signs, U, lv = make_context(cfg, 2, vbits)
    tags, k, v = _inputs(cfg, n)
    v = v.copy()
    v[:, 0:32] = 0.0                      # window 0: all zero
    v[:, 32:35] *= 1e-26                  # window 1: three underflowing tokens
    v[:, 64:72] *= 1e-26                  # window 2: eight underflowing tokens
    v[:, 96] = 0.0                        # window 3: a zero token and an overflowing one
    v[:, 101] *= 1e19
    v[:, 130, :, :64] = 0.0               # window 4: a half-zero token
    if dtype == "bf16":
        v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()   # what the bf16 path sees
    cache = ctx.alloc_cache(cfg.batch, n)
    cache["modality"].copy_(to_dev(tags[:, :n]))
    ctx.quantize_values(bf16_tensor(v) if dtype == "bf16" else torch.from_numpy(v).cuda(), 0, cache)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        vc, vs = O.quantize_values(v, tags[:, :n], U, lv, vbits)
    assert np.array_equal(from_dev(cache["v_scale"], np.uint16), vs)
    gv = from_dev(cache["v_codes"], np.uint32)
    if not np.array_equal(gv, vc):
        gcodes = O.unpack_windows(gv, "value", cfg.head_dim, vbits)
        ocodes = O.unpack_windows(vc, "value", cfg.head_dim, vbits)
        bad = np.argwhere(gcodes != ocodes)
        raise AssertionError(f"{len(bad)} value codes differ, first at {bad[:4].tolist()}")
    ctx.close()


@pytest.mark.parametrize("cid,kbits", [(2, 2), (2, 4), (1, 2), (1, 4)])
def test_quantize_keys_degenerate_windows(cid, kbits):
    """Key codes and metadata at the edges of the row-parallel Hadamard transform: an
    all-zero window (m = +0, s = 0), a window of 32 identical tokens (zero range in every
    channel), negative zeros, tokens near the bottom and the top of the fp32 range, and a
    window with a single nonzero channel."""
    import torch
    cfg = synth.CONFIGS[cid]
    n = 256
    say(f"[codec-degenerate-keys] cfg{cid} K{kbits} n=256")
    ctx, signs, U, lv = make_context(cfg, kbits, 2)
    tags, k, v = _inputs(cfg, n)
    k = k.copy()
    k[:, 0:32] = 0.0                         # window 0: all zero
    k[:, 32:64] = k[:, 32:33]                # window 1: identical tokens
    k[:, 64:96] = np.where(k[:, 64:96] < 0, -0.0, k[:, 64:96])   # window 2: negative zeros
    k[:, 64:70] = -0.0
    k[:, 96:99] *= 1e-30                     # window 3: tiny tokens among ordinary ones
    k[:, 128:130] *= 1e30                    # window 4: huge tokens
    k[:, 160:192] = 0.0                      # window 5: one nonzero channel
    k[:, 160:192, :, 7] = np.linspace(-3.0, 2.0, 32, dtype=np.float32)[None, :, None]
    if not cfg.fp32_inputs:                  # what the bf16 path sees
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
    cache = ctx.alloc_cache(cfg.batch, n)
    kd = torch.from_numpy(k).cuda() if cfg.fp32_inputs else bf16_tensor(k)
    ctx.quantize_keys(kd, 0, cache)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        kc, km, ks = O.quantize_keys(k, signs, kbits)
    assert np.array_equal(from_dev(cache["k_min"], np.uint16), km)
    assert np.array_equal(from_dev(cache["k_scale"], np.uint16), ks)
    gk = from_dev(cache["k_codes"], np.uint32)
    if not np.array_equal(gk, kc):
        g = O.unpack_windows(gk, "key", cfg.head_dim, kbits)
        o = O.unpack_windows(kc, "key", cfg.head_dim, kbits)
        bad = np.argwhere(g != o)
        raise AssertionError(f"{len(bad)} key codes differ, first at {bad[:4].tolist()}")
    ctx.close()


# ----------------------------------------------------------------------------- codec at full size, sampled
@pytest.mark.parametrize("cid,kbits,vbits", [(3, 2, 2), (5, 2, 2), (5, 4, 4)])
def test_quantize_parity_prefill_sampled(cid, kbits, vbits):
    import torch
    cfg = synth.CONFIGS[cid]
    n = cfg.prefill
    say(f"[codec-sampled] cfg{cid} K{kbits}V{vbits} prefill {n} tokens x batch {cfg.batch}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits)
    tags, k, v = _inputs(cfg, n)
    cache = ctx.alloc_cache(cfg.batch, n)
    cache["modality"].copy_(to_dev(tags[:, :n]))
    ctx.quantize_keys(_dev_kv(cfg, k), 0, cache)
    ctx.quantize_values(_dev_kv(cfg, v), 0, cache)
    torch.cuda.synchronize()
    gk = from_dev(cache["k_codes"], np.uint32)
    gkm = from_dev(cache["k_min"], np.uint16)
    gks = from_dev(cache["k_scale"], np.uint16)
    gv = from_dev(cache["v_codes"], np.uint32)
    gvs = from_dev(cache["v_scale"], np.uint16)
    rng = np.random.default_rng(cid)
    picks = [(int(rng.integers(cfg.batch)), int(rng.integers(cfg.kv_heads)), int(rng.integers(n // 32)))
             for _ in range(48)]
    picks += [(cfg.batch - 1, cfg.kv_heads - 1, n // 32 - 1), (0, 0, 0)]
    for b, h, w in picks:
        ks_ = slice(32 * w, 32 * w + 32)
        kc, km, ksc = O.quantize_keys(k[b:b + 1, ks_, h:h + 1], signs, kbits)
        assert np.array_equal(gk[b, h, w], kc[0, 0, 0]), (b, h, w)
        assert np.array_equal(gkm[b, h, w], km[0, 0, 0]) and np.array_equal(gks[b, h, w], ksc[0, 0, 0])
        vc, vs = O.quantize_values(v[b:b + 1, ks_, h:h + 1], tags[b:b + 1, ks_], U, lv, vbits)
        assert np.array_equal(gv[b, h, w], vc[0, 0, 0]), (b, h, w)
        assert np.array_equal(gvs[b, h, ks_], vs[0, 0])
    ctx.close()


# ----------------------------------------------------------------------------- decode, full compare
def _oracle_cache(cfg, ctx, signs, U, lv, T, kbits, vbits, seed=0):
    tags, k, v = _inputs(cfg, T, seed)
    kc, km, ks = O.quantize_keys(k, signs, kbits)
    vc, vs = O.quantize_values(v, tags[:, :T], U, lv, vbits)
    return dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags[:, :T].copy(),
                key_bits=kbits, value_bits=vbits, t_cap=T)


@pytest.mark.parametrize("cid,kbits,vbits,T,ragged", [
    (1, 2, 2, 256, False), (1, 2, 2, 256, True), (1, 4, 4, 256, False),
    (2, 2, 2, 10240, False), (2, 2, 2, 10240, True), (2, 4, 4, 4096, True), (2, 2, 4, 2048, False),
])
def test_decode_parity_oracle_cache(cid, kbits, vbits, T, ragged):
    import torch
    cfg = synth.CONFIGS[cid]
    say(f"[decode] cfg{cid} K{kbits}V{vbits} T={T} ragged={ragged}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits)
    cache = _oracle_cache(cfg, ctx, signs, U, lv, T, kbits, vbits)
    B = cfg.batch
    q = synth.queries(cfg, 3)
    lens = np.full(B, T, np.int32)
    if ragged:
        lens[:] = [T - 17 - 5 * b for b in range(B)]
    dcache = cache_to_device(cache)
    out = ctx.decode(to_dev(q), to_dev(lens), T, dcache)
    torch.cuda.synchronize()
    got = from_dev(out)
    ref = O.decode_attention(q, lens, cache, signs, U, lv)
    err = row_errors(got, ref)
    say(f"    max row error {err.max():.3e}")
    assert err.max() <= TOL
    ctx.close()


def test_decode_edge_lengths():
    import torch
    cfg = synth.CONFIGS[2]
    T = 256
    ctx, signs, U, lv = make_context(cfg)
    cache = _oracle_cache(cfg, ctx, signs, U, lv, T, 2, 2)
    # batch of four sequences sharing the same cache rows: lengths 0, 1, 33, 256
    B = 4
    big = {k: (np.repeat(v, B, axis=0) if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
    q = np.random.default_rng(5).standard_normal((B, cfg.q_heads, cfg.head_dim)).astype(np.float32)
    lens = np.array([0, 1, 33, 256], np.int32)
    out = from_dev(ctx.decode(to_dev(q), to_dev(lens), T, cache_to_device(big)))
    torch.cuda.synchronize()
    ref = O.decode_attention(q, lens, big, signs, U, lv)
    assert np.all(out[0] == 0.0)
    err = row_errors(out[1:], ref[1:])
    say(f"    max row error {err.max():.3e}")
    assert err.max() <= TOL
    ctx.close()


def test_decode_split_invariance():
    import torch
    cfg = synth.CONFIGS[2]
    T = 10240
    ctx, signs, U, lv = make_context(cfg)
    cache = cache_to_device(synth.random_packed_cache(cfg, 1, length=T))
    q = to_dev(synth.queries(cfg, 7))
    lens = to_dev(np.array([T - 3], np.int32))
    # (5000 asks for more splits than the 320 windows: one window per split, as for 320)
    outs = [from_dev(ctx.decode(q, lens, T, cache, num_splits=s)) for s in (1, 3, 0, 64, 320, 5000)]
    torch.cuda.synchronize()
    # Splits change each partial's reference max, hence the fp16 hi/lo rounding
    # of the probability operand (~2^-22 relative, 2^-25 absolute when the low
    # part is subnormal) and the order of the fp32 sums; the spread stays far
    # below the 1e-3 bar against the oracle.
    for o in outs[1:]:
        assert row_errors(o, outs[0]).max() < 3e-5
    ctx.close()


def test_decode_max_splits():
    """1024 splits per (sequence, KV head), the most the plan makes, and a request beyond it:
    a 32,768-token context (1024 windows, one per split) against the default plan, and
    against the oracle on sampled rows."""
    import torch
    cfg = synth.CONFIGS[2]
    T = 32768
    say(f"[max-splits] cfg2 T={T}")
    ctx, signs, U, lv = make_context(cfg)
    host = synth.random_packed_cache(cfg, 21, length=T)
    cache = cache_to_device(host)
    q_np = synth.queries(cfg, 21)
    q = to_dev(q_np)
    lens_np = np.array([T - 17], np.int32)
    lens = to_dev(lens_np)
    outs = [from_dev(ctx.decode(q, lens, T, cache, num_splits=s)) for s in (0, 1024, 100000)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert row_errors(o, outs[0]).max() < 3e-5
    ref = O.decode_attention(q_np, lens_np, host, signs, U, lv)
    err = row_errors(outs[1], ref)
    say(f"    max row error {err.max():.3e}")
    assert err.max() <= TOL
    ctx.close()


def test_decode_graph_replay_matches_eager():
    """The two-launch decode step (omnikv_decode_partial + omnikv_decode_combine) captured in
    a HIP graph gives the eager result bit for bit on every replay, with eager work between
    replays."""
    import torch
    cfg = synth.CONFIGS[2]
    T = 4096
    ctx, signs, U, lv = make_context(cfg)
    caches = [cache_to_device(synth.random_packed_cache(cfg, 20 + i, length=T)) for i in range(2)]
    q = to_dev(synth.queries(cfg, 5))
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
        # eager work between replays, on other buffers
        ctx.decode(q, lens, T, caches[(rep + 1) % 2])
        torch.cuda.synchronize()
    ctx.close()


# ----------------------------------------------------------------------------- decode at full size, sampled rows
@pytest.mark.parametrize("cid,kbits,vbits", [(3, 2, 2), (4, 2, 2), (5, 2, 2), (4, 4, 4), (5, 4, 4)])
def test_decode_parity_full_size_sampled(cid, kbits, vbits):
    import torch
    cfg = synth.CONFIGS[cid]
    T = cfg.context
    say(f"[decode-sampled] cfg{cid} K{kbits}V{vbits} B={cfg.batch} T={T}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits)
    cache = synth.random_packed_cache(cfg, 2, key_bits=kbits, value_bits=vbits)
    lens = synth.seq_lens(cfg, ragged=True, seed=cid)
    lens[0] = T
    q = synth.queries(cfg, 4)
    out = from_dev(ctx.decode(to_dev(q), to_dev(lens), T, cache_to_device(cache)))
    torch.cuda.synchronize()
    rows = sampled_unit_rows(cfg, cid)
    ref = O.decode_attention(q, lens, cache, signs, U, lv, rows=rows)
    bi = [r[0] for r in rows]
    hi = [r[1] for r in rows]
    err = row_errors(out[bi, hi], ref[bi, hi])
    say(f"    rows {rows} max row error {err.max():.3e}")
    assert err.max() <= TOL
    assert np.all(np.isfinite(out))
    ctx.close()


# ----------------------------------------------------------------------------- the whole step
def test_decode_workspace_reused_across_plans():
    """One workspace, NaN-patterned on entry, serves decode steps of different batch sizes,
    lengths and split counts: every result equals the one computed on a fresh workspace, bit
    for bit (no state is carried from one call to the next)."""
    import torch
    cfg = synth.CONFIGS[2]
    T = 10240
    say("[workspace-reuse] cfg2")
    ctx, signs, U, lv = make_context(cfg)
    big = synth.Config(**{**cfg.__dict__, "batch": 4})
    cache = cache_to_device(synth.random_packed_cache(big, 13, length=T))
    q = to_dev(synth.queries(big, 13))
    need = max(ctx.workspace_size(B, n, s) for B in (1, 4) for n in (T, 2048) for s in (0, 7, 200))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for B, n, s in ((4, T, 0), (1, 2048, 7), (4, 2048, 200), (1, T, 0), (4, T, 3)):
            sub = {k: (v[:B] if k != "t_cap" else v) for k, v in cache.items()}
            lens = to_dev(np.array([n - 3 * b for b in range(B)], np.int32))
            got = ctx.decode(q[:B].contiguous(), lens, n, sub, workspace=ws, num_splits=s)
            ref = ctx.decode(q[:B].contiguous(), lens, n, sub, num_splits=s)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (rep, B, n, s)
    ctx.close()


def test_decode_step_graph_replay_matches_eager():
    """omnikv_decode_attention captured in a HIP graph gives the eager result bit for bit on
    every replay, with eager work on the same workspace between replays."""
    import torch
    cfg = synth.CONFIGS[3]
    T = 4096
    one = synth.Config(**{**cfg.__dict__, "context": T})
    say("[step-graph-replay] cfg3")
    ctx, signs, U, lv = make_context(cfg)
    caches = [cache_to_device(synth.random_packed_cache(one, 30 + i, length=T)) for i in range(2)]
    q = to_dev(synth.queries(cfg, 5))
    lens = to_dev(np.full(cfg.batch, T - 9, np.int32))
    ws = torch.empty(ctx.workspace_size(cfg.batch, T), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((cfg.batch, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
            for _ in range(2)]
    eager = []
    for i in range(2):
        ctx.decode(q, lens, T, caches[i], out=outs[i], workspace=ws)
        eager.append(outs[i].clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(2):
            ctx.decode(q, lens, T, caches[i], out=outs[i], workspace=ws)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], eager[i]), (rep, i)
        ctx.decode(q, lens, T, caches[(rep + 1) % 2], workspace=ws)
        torch.cuda.synchronize()
    ctx.close()
