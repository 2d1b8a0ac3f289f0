"""Edges of the input space through the C ABI against the CPU oracle.

  * the library's built-in value codebook equals the oracle's (Lloyd-Max levels of N(0,1)
    rounded to fp16, pinned to the textbook values in tests/golden/);
  * contexts with one or two modalities (one U_m per modality m in {V, A, L}, [paper] §2.3;
    the unused rotation slots of the decode stay unread by the result);
  * a cache whose capacity exceeds the context, with NaN metadata, NaN scales and
    out-of-range tags everywhere past each sequence's length;
  * value scales far from 1: values scaled by 1e-4, 1e3 and per-token powers of two
    2^-20 .. 2^12 sent through the write path, and scales drawn directly over 2^-20 .. 2^15,
    decoded.

Bars as everywhere: packed codes and metadata bit-exact, decode rows within 1e-3.
"""
import numpy as np
import pytest

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import binding, synth
from tests.gpu_helpers import (bf16_tensor, cache_to_device, from_dev, make_context, oracle_codebook,
                               row_errors, say, to_dev)

pytestmark = pytest.mark.gpu
TOL = 1e-3
F16_NAN = 0x7E00


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 4), (64, 2), (64, 4)])
def test_library_codebook_equals_oracle_codebook(d, bits):
    """omnikv_create's built-in table (NULL codebook) against the oracle's Lloyd-Max table."""
    from decode_attention_fwht_amd import binding
    say(f"[codebook] d={d} bits={bits}")
    ctx = binding.Context(d, 8, 1, 2, bits, synth.rademacher_signs(d, 0), synth.value_rotations(d, 0))
    got = ctx.value_codebook()
    ref = O.value_codebook_f16(bits)
    say(f"    library {got.view(np.float16).tolist()} oracle {ref.view(np.float16).tolist()}")
    assert np.array_equal(got, ref)
    ctx.close()


def _codec_and_decode(cfg, ctx, signs, U, lv, tags, k, v, kbits, vbits, lens, q):
    """GPU write path vs oracle quantization (bit-exact), then GPU decode over the oracle's
    cache vs the oracle's attention.  Returns the max row error."""
    import torch
    B, n = k.shape[0], k.shape[1]
    cache = ctx.alloc_cache(B, n)
    cache["modality"].copy_(to_dev(tags))
    dev = (lambda x: torch.from_numpy(x).cuda()) if cfg.fp32_inputs else bf16_tensor
    ctx.quantize_keys(dev(k), 0, cache)
    ctx.quantize_values(dev(v), 0, cache)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        kc, km, ks = O.quantize_keys(k, signs, kbits)
        vc, vs = O.quantize_values(v, tags, U, lv, vbits)
    assert np.array_equal(from_dev(cache["k_min"], np.uint16), km)
    assert np.array_equal(from_dev(cache["k_scale"], np.uint16), ks)
    assert np.array_equal(from_dev(cache["k_codes"], np.uint32), kc)
    assert np.array_equal(from_dev(cache["v_scale"], np.uint16), vs)
    gv = from_dev(cache["v_codes"], np.uint32)
    if not np.array_equal(gv, vc):
        g = O.unpack_windows(gv, "value", cfg.head_dim, vbits)
        o = O.unpack_windows(vc, "value", cfg.head_dim, vbits)
        raise AssertionError(f"{np.count_nonzero(g != o)} of {g.size} value codes differ")
    host = dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags, key_bits=kbits,
                value_bits=vbits, t_cap=n)
    out = from_dev(ctx.decode(to_dev(q), to_dev(lens), n, cache_to_device(host)))
    torch.cuda.synchronize()
    ref = O.decode_attention(q, lens, host, signs, U, lv)
    assert np.all(np.isfinite(out))
    return row_errors(out, ref).max()


@pytest.mark.parametrize("cid,M,kbits,vbits", [(2, 1, 2, 2), (2, 2, 2, 2), (2, 2, 4, 4), (1, 1, 2, 2), (1, 2, 4, 4)])
def test_fewer_modalities(cid, M, kbits, vbits):
    """num_modalities 1 and 2: tags restricted to 0 .. M-1, the context holds M rotations."""
    cfg = synth.CONFIGS[cid]
    n = 2048 if cid == 2 else 256
    say(f"[modalities] cfg{cid} M={M} K{kbits}V{vbits} n={n}")
    ctx, signs, U, lv = make_context(cfg, kbits, vbits, modalities=M)
    assert ctx.num_modalities == M and U.shape[0] == M
    tags = np.minimum(synth.modality_layout(cfg, 0, n), M - 1).astype(np.uint8)
    k = synth.drifting_tensor(cfg, tags, 0, 0, 0, n)
    v = synth.drifting_tensor(cfg, tags, 0, 1, 0, n)
    lens = np.array([n - 11 * b for b in range(cfg.batch)], np.int32)
    err = _codec_and_decode(cfg, ctx, signs, U, lv, tags, k, v, kbits, vbits, lens, synth.queries(cfg, 2))
    say(f"    max row error {err:.3e}")
    assert err <= TOL
    ctx.close()


@pytest.mark.parametrize("key_meta", ["fp16", "mxfp4"])
def test_decode_spare_capacity_nan_padding(key_meta):
    """t_cap = 2 max_len.  Every token past a sequence's length holds a NaN value scale and
    an out-of-range tag, every window past it NaN metadata (fp16 NaN, or MXFP4 records of
    all-ones bytes) and random codes, up to t_cap; the decode must read none of it."""
    import torch
    cfg = synth.CONFIGS[2]
    B, max_len = 3, 2048
    t_cap = 2 * max_len
    say(f"[spare-capacity] cfg2 B={B} max_len={max_len} t_cap={t_cap} {key_meta}")
    ctx, signs, U, lv = make_context(cfg, key_meta=key_meta)
    one = synth.Config(**{**cfg.__dict__, "batch": B})
    tags = synth.modality_layout(one, 0, t_cap)
    k = synth.drifting_tensor(one, tags, 1, 0, 0, t_cap)
    v = synth.drifting_tensor(one, tags, 1, 1, 0, t_cap)
    kc, km, ks = O.quantize_keys(k, signs, 2, meta=key_meta)
    vc, vs = O.quantize_values(v, tags, U, lv, 2)
    lens = np.array([max_len - 40, max_len // 2 + 7, max_len], np.int32)
    rng = np.random.default_rng(3)
    tags = tags.copy()
    for b, n in enumerate(lens):
        w0 = (n + 31) // 32           # first window wholly past the length
        vs[b, :, n:] = F16_NAN
        tags[b, n:] = rng.integers(3, 256, t_cap - n)
        km[b, :, w0:] = 0xFF if key_meta == "mxfp4" else F16_NAN
        ks[b, :, w0:] = 0xFF if key_meta == "mxfp4" else F16_NAN
        kc[b, :, w0:] = rng.integers(0, 2**32, kc[b, :, w0:].shape, dtype=np.uint64).astype(np.uint32)
        vc[b, :, w0:] = rng.integers(0, 2**32, vc[b, :, w0:].shape, dtype=np.uint64).astype(np.uint32)
    host = dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags, key_bits=2,
                value_bits=2, t_cap=t_cap)
    q = synth.queries(one, 6)
    out = from_dev(ctx.decode(to_dev(q), to_dev(lens), max_len, cache_to_device(host)))
    torch.cuda.synchronize()
    ref = O.decode_attention(q, lens, host, signs, U, lv)
    err = row_errors(out, ref)
    say(f"    max row error {err.max():.3e}")
    assert np.all(np.isfinite(out)) and err.max() <= TOL
    ctx.close()


def test_value_scale_range():
    """Value scales far from 1 through the write path and the decode: one sequence with its
    values scaled by 1e-4, one by 1e3, one with every token scaled by its own power of two
    2^u, u uniform in -20 .. 12 (the tokens' RMS reach ~2^14, scales span ~34 binades within a
    window; 2^13 would take some RMS past fp16's largest finite value, where the stored scale
    is infinite on both sides).  Codes and scales bit-exact, decode rows within 1e-3."""
    cfg = synth.CONFIGS[2]
    B, n = 3, 2048
    say(f"[value-scale-range] cfg2 B={B} n={n}")
    ctx, signs, U, lv = make_context(cfg)
    one = synth.Config(**{**cfg.__dict__, "batch": B})
    tags = synth.modality_layout(one, 0, n)
    k = synth.drifting_tensor(one, tags, 4, 0, 0, n)
    v = synth.drifting_tensor(one, tags, 4, 1, 0, n).copy()
    v[0] *= np.float32(1e-4)
    v[1] *= np.float32(1e3)
    u = np.random.default_rng(8).integers(-20, 13, (n, 1, 1))
    v[2] *= np.exp2(u).astype(np.float32)
    v = synth.to_bf16(v)
    assert np.isfinite(O.f16_to_f32(O.f16_bits(O.value_scale_f32(v)))).all()
    lens = np.array([n, n - 5, n - 33], np.int32)
    err = _codec_and_decode(one, ctx, signs, U, lv, tags, k, v, 2, 2, lens, synth.queries(one, 9))
    say(f"    max row error {err:.3e}")
    assert err <= TOL
    ctx.close()


def test_value_scale_range_sampled_scales():
    """Value scales drawn directly as fp16 bit patterns log-uniform over 2^-20 .. 2^15 per
    token (no write path), on a packed cache of random codes."""
    import torch
    cfg = synth.CONFIGS[2]
    T = 4096
    say(f"[value-scale-bits] cfg2 T={T}")
    ctx, signs, U, lv = make_context(cfg)
    cache = synth.random_packed_cache(cfg, 12, length=T)
    r = np.random.default_rng(12)
    cache["v_scale"] = np.exp2(r.uniform(-20, 15, cache["v_scale"].shape)).astype(np.float16).view(np.uint16)
    q = synth.queries(cfg, 12)
    lens = np.array([T - 7], np.int32)
    out = from_dev(ctx.decode(to_dev(q), to_dev(lens), T, cache_to_device(cache)))
    torch.cuda.synchronize()
    ref = O.decode_attention(q, lens, cache, signs, U, lv)
    err = row_errors(out, ref)
    say(f"    max row error {err.max():.3e}")
    assert np.all(np.isfinite(out)) and err.max() <= TOL
    ctx.close()


@pytest.mark.parametrize("bits", [2, 4])
def test_error_metrics_of_the_gpu_codec(bits):
    """The pages' three error metrics ([paper] §3.3 Error comparison: key reconstruction MSE,
    attention KL, attention-output MSE) on the GPU write path's output for drift data: equal to
    those of the oracle's own quantization (the codes are the same), and the values are
    reported.  Both KV heads of a config-2 sequence, 4096 tokens, all 8 query heads each."""
    import math
    import torch
    cfg = synth.CONFIGS[2]
    n = 4096
    say(f"[metrics] cfg2 K{bits}V{bits} n={n}")
    ctx, signs, U, lv = make_context(cfg, bits, bits)
    tags = synth.modality_layout(cfg, 3, n)
    k = synth.drifting_tensor(cfg, tags, 3, 0, 0, n)
    v = synth.drifting_tensor(cfg, tags, 3, 1, 0, n)
    cache = ctx.alloc_cache(cfg.batch, n)
    cache["modality"].copy_(to_dev(tags))
    ctx.quantize_keys(bf16_tensor(k), 0, cache)
    ctx.quantize_values(bf16_tensor(v), 0, cache)
    torch.cuda.synchronize()
    g = {key: from_dev(cache[key], dt) for key, dt in (("k_codes", np.uint32), ("k_min", np.uint16),
                                                      ("k_scale", np.uint16), ("v_codes", np.uint32),
                                                      ("v_scale", np.uint16))}
    kc, km, ks = O.quantize_keys(k, signs, bits)
    vc, vs = O.quantize_values(v, tags, U, lv, bits)
    q = synth.queries(cfg, 3)[0]
    scale = 1.0 / math.sqrt(cfg.head_dim)

    def metrics(kc_, km_, ks_, vc_, vs_):
        kh = O.dequantize_keys(kc_, km_, ks_, signs, bits)[0]
        vh = O.dequantize_values(vc_, vs_, tags, U, lv, bits)[0]
        out = []
        for h in range(cfg.kv_heads):
            kk, vv = k[0, :, h].astype(np.float64), v[0, :, h].astype(np.float64)
            qq = q[h * cfg.group:(h + 1) * cfg.group]
            out.append((O.key_reconstruction_mse(kk, kh[h]), O.attention_kl(qq, kk, kh[h], scale),
                        O.attention_output_mse(qq, kk, vv, kh[h], vh[h], scale)))
        return np.array(out)

    got = metrics(g["k_codes"], g["k_min"], g["k_scale"], g["v_codes"], g["v_scale"])
    ref = metrics(kc, km, ks, vc, vs)
    for h in range(cfg.kv_heads):
        say(f"    KV head {h}: key MSE {got[h, 0]:.4f}  attention KL {got[h, 1]:.4f}  output MSE {got[h, 2]:.5f}")
    assert np.array_equal(got, ref)
    assert np.all(np.isfinite(got)) and np.all(got > 0)
    ctx.close()


def test_quantize_rejects_more_than_2_32_windows_per_call():
    """A chunk of more than 2^32 - 1 windows (batch x KV heads x n / 32) is refused on the
    host before anything is launched (the kernels index windows in 32 bits); the buffers
    are never touched."""
    import ctypes
    import torch
    cfg = synth.CONFIGS[2]
    ctx, signs, U, lv = make_context(cfg)
    L = binding.load()
    buf = torch.zeros(1 << 12, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    batch, n = (1 << 31) - 1, 128            # x 2 KV heads x 4 windows: 2^34 windows
    for fn in ("keys", "values"):
        if fn == "keys":
            st = L.omnikv_quantize_keys(ctx._h, p, binding.BF16, batch, 0, n, n, p, p, p, None)
        else:
            st = L.omnikv_quantize_values(ctx._h, p, binding.BF16, p, batch, 0, n, n, p, p, None)
        assert st == binding.EINVAL, fn
        assert "2^32" in L.omnikv_last_error().decode()
    torch.cuda.synchronize()
    ctx.close()
