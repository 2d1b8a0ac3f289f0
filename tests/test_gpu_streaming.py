"""Streaming generation through the C ABI against the oracle.

The schedule ([paper] §3.1 Implementation details, captioning): keys are quantized
every 128 tokens in groups of 32, values keep a 128-token sliding window; recent
tokens live in rings and enter the attention as stored.

Bars: packed codes, k_min, k_scale, v_scale written by the append path are
bit-exact against the oracle's quantization of the same tokens; decode outputs
are within 1e-3 max row relative error of the oracle's float64 attention over the
same packed cache and the same stored recent tokens.
"""
import numpy as np
import pytest

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import synth
from tests.gpu_helpers import (bf16_tensor, cache_to_device, from_dev, make_context, row_errors, say, to_dev)

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _tokens(cfg, T, seed):
    tags = synth.modality_layout(cfg, seed, T)
    k = synth.drifting_tensor(cfg, tags, seed, 0, 0, T)
    v = synth.drifting_tensor(cfg, tags, seed, 1, 0, T)
    if not cfg.fp32_inputs:  # what a bf16 ring stores
        import torch
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
        v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    return tags, k, v


def _rings(ctx, cfg, k, v, lens, cap):
    """Rings holding every sequence's recent tokens (row t % cap) as the append path would."""
    import torch
    dt = torch.float32 if cfg.fp32_inputs else torch.bfloat16
    rings = ctx.alloc_rings(k.shape[0], cap, dtype=dt)
    rk = np.zeros((k.shape[0], cap) + k.shape[2:], np.float32)
    rv = np.zeros_like(rk)
    for b, n in enumerate(lens):
        _, vp = O.stream_packed_lengths(n)
        for t in range(max(vp, n - cap), n):
            rk[b, t % cap] = k[b, t]
            rv[b, t % cap] = v[b, t]
    rings["k"].copy_(torch.from_numpy(rk).to(dt).cuda())
    rings["v"].copy_(torch.from_numpy(rv).to(dt).cuda())
    return rings


@pytest.mark.parametrize("cid,lens,cap,kbits,vbits", [
    (1, [0, 1, 127, 128], 256, 2, 2),
    (1, [200, 257, 129], 256, 4, 4),
    (2, [300, 97, 515, 160], 256, 2, 2),
    (2, [640, 383, 129], 512, 2, 2),
    (2, [400, 260], 256, 4, 2),
])
def test_streaming_decode_parity(cid, lens, cap, kbits, vbits):
    """Packed prefix + recent tokens, cache quantized by the oracle (the same packed
    cache on both sides), recent tokens in rings that have wrapped."""
    import torch
    cfg = synth.CONFIGS[cid]
    B = len(lens)
    T = max(32, ((max(lens) + 31) // 32) * 32)
    say(f"[stream-decode] cfg{cid} K{kbits}V{vbits} lens {lens} ring {cap}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits)
    tags, k, v = _tokens(cfg, T, 3)
    tags, k, v = tags[:1].repeat(B, 0), np.repeat(k[:1], B, 0), np.repeat(v[:1], B, 0)
    kc, km, ks = O.quantize_keys(k, signs, kbits)
    vc, vs = O.quantize_values(v, tags, U, lv, vbits)
    host = dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags,
                key_bits=kbits, value_bits=vbits)
    cache = cache_to_device(host)
    rings = _rings(ctx, cfg, k, v, lens, cap)
    q_np = synth.queries(cfg, 4, B)
    q = torch.from_numpy(q_np).cuda()
    out = from_dev(ctx.decode_streaming(q, to_dev(np.array(lens, np.int32)), T, cache, rings))
    ref = O.decode_attention_streaming(q_np, lens, host, k, v, signs, U, lv)
    err = row_errors(out, ref)
    say(f"    max row error {err.max():.3e}")
    assert err.max() <= TOL
    assert np.all(out[[i for i, n in enumerate(lens) if n == 0]] == 0.0)
    ctx.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_stream_append_writes_what_the_schedule_quantizes(dtype):
    """Token-by-token appends: the packed cache equals the oracle's quantization of the
    same tokens over the packed ranges, the rings hold the recent tokens, and decoding
    the stream matches the oracle, at several points of the stream.  bf16 and fp32 rings
    (fp32 tokens with full significands: the flushes take the quantizers' fp32 forms)."""
    import torch
    cfg = synth.CONFIGS[2]
    if dtype == "fp32":
        cfg = synth.Config(**{**cfg.__dict__, "fp32_inputs": True})
    B, T, cap = 2, 576, 256
    say(f"[stream-append] cfg2 B={B} {T} tokens ring {cap} {dtype}")
    ctx, signs, U, lv = make_context(cfg)
    tags, k, v = _tokens(cfg, T, 5)
    tags, k, v = tags[:1].repeat(B, 0), np.repeat(k[:1], B, 0), np.repeat(v[:1], B, 0)
    cache = ctx.alloc_cache(B, T)
    if dtype == "fp32":
        rings = ctx.alloc_rings(B, cap, dtype=torch.float32)
        kd, vd = torch.from_numpy(np.ascontiguousarray(k)).cuda(), torch.from_numpy(np.ascontiguousarray(v)).cuda()
    else:
        rings = ctx.alloc_rings(B, cap)
        kd, vd = bf16_tensor(k), bf16_tensor(v)
    tg = to_dev(tags)
    q_np = synth.queries(cfg, 6, B)
    q = torch.from_numpy(q_np).cuda()
    # sequence 1 runs 37 tokens ahead: its first tokens go in alone, through views of
    # its rows of the cache and the rings
    lead = 37
    c1 = {key: (val[1:2] if key != "t_cap" else val) for key, val in cache.items()}
    r1 = {key: (val[1:2] if key != "cap" else val) for key, val in rings.items()}
    for t in range(lead):
        ctx.stream_append(kd[1:2, t].contiguous(), vd[1:2, t].contiguous(), tg[1:2, t].contiguous(),
                          to_dev(np.array([t], np.int32)), [t], c1, r1)
    lens = np.array([0, lead], np.int64)
    checks = {1, 140, 288, 385, T - lead}
    for step in range(1, T - lead + 1):
        k_new = torch.stack([kd[b, int(lens[b])] for b in range(B)]).contiguous()
        v_new = torch.stack([vd[b, int(lens[b])] for b in range(B)]).contiguous()
        t_new = torch.stack([tg[b, int(lens[b])] for b in range(B)]).contiguous()
        ctx.stream_append(k_new, v_new, t_new, to_dev(lens.astype(np.int32)), lens.tolist(), cache, rings)
        lens += 1
        if step not in checks:
            continue
        n = lens.tolist()
        out = from_dev(ctx.decode_streaming(q, to_dev(lens.astype(np.int32)), T, cache, rings))
        host = dict(k_codes=from_dev(cache["k_codes"], np.uint32), k_min=from_dev(cache["k_min"], np.uint16),
                    k_scale=from_dev(cache["k_scale"], np.uint16), v_codes=from_dev(cache["v_codes"], np.uint32),
                    v_scale=from_dev(cache["v_scale"], np.uint16), modality=from_dev(cache["modality"]),
                    key_bits=cfg.key_bits, value_bits=cfg.value_bits)
        for b in range(B):
            kp, vp = O.stream_packed_lengths(n[b])
            if kp:
                okc, okm, oks = O.quantize_keys(k[b:b + 1, :kp], signs, cfg.key_bits)
                assert np.array_equal(host["k_codes"][b, :, :kp // 32], okc[0]), (step, b)
                assert np.array_equal(host["k_min"][b, :, :kp // 32], okm[0])
                assert np.array_equal(host["k_scale"][b, :, :kp // 32], oks[0])
            if vp:
                ovc, ovs = O.quantize_values(v[b:b + 1, :vp], tags[b:b + 1, :vp], U, lv, cfg.value_bits)
                assert np.array_equal(host["v_codes"][b, :, :vp // 32], ovc[0]), (step, b)
                assert np.array_equal(host["v_scale"][b, :, :vp], ovs[0])
            assert np.array_equal(host["modality"][b, :n[b]], tags[b, :n[b]])
        ref = O.decode_attention_streaming(q_np, n, host, k, v, signs, U, lv)
        err = row_errors(out, ref)
        say(f"    step {step} lens {n} max row error {err.max():.3e}")
        assert err.max() <= TOL
    ctx.close()
