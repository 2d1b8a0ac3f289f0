"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: a closed
form, a textbook table, an invariant, a worked example or brute force.
"""
import math
import os

import numpy as np
import pytest

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- fp16
def test_fp16_rounding_matches_binary16_definition():
    for line in open(os.path.join(GOLDEN, "fp16_rne.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v, bits = line.split()
        with np.errstate(over="ignore"):
            got = int(O.f16_bits(np.float32(float(v))))
        assert got == int(bits, 16), (v, hex(got), bits)


# ----------------------------------------------------------------------------- rotation (T1)
@pytest.mark.parametrize("d", [64, 128])
def test_rotation_equals_sylvester_closed_form(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d)).astype(np.float32)
    signs = synth.rademacher_signs(d, 3)
    y = O.rotate_keys_f32(x, signs).astype(np.float64)
    # closed form: H_ij = (-1)^popcount(i&j), written out element by element here
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(d)] for i in range(d)], dtype=np.float64)
    ref = (x.astype(np.float64) * signs) @ H.T / math.sqrt(d)
    assert np.max(np.abs(y - ref)) < 1e-5 * np.max(np.abs(ref))


def test_rotation_is_an_involution_on_small_integers_d64():
    # d = 64: c_d = 1/8 exactly, H H = 64 I, so (c H)(c H) x = x with no rounding at all
    rng = np.random.default_rng(1)
    x = rng.integers(-7, 8, (9, 64)).astype(np.float32)
    ones = np.ones(64, np.int8)
    y = O.rotate_keys_f32(O.rotate_keys_f32(x, ones), ones)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_orthogonal_and_inverse_recovers_input(d):
    signs = synth.rademacher_signs(d, 5)
    eye = np.eye(d, dtype=np.float32)
    R = O.rotate_keys_f32(eye, signs).astype(np.float64).T        # columns = R e_i
    assert np.max(np.abs(R @ R.T - np.eye(d))) < 1e-6
    x = np.random.default_rng(2).standard_normal((4, d)).astype(np.float32)
    back = O.inverse_key_rotation_f64(O.rotate_keys_f32(x, signs), signs)
    assert np.max(np.abs(back - x)) < 1e-5


def test_rotation_stage_order_scalar_reference():
    # A scalar loop that follows the documented stage order one butterfly at a
    # time (h = 1, 2, ..., d/2; (a, b) -> (a + b, a - b)), in fp32, must match
    # the vectorised oracle bit for bit.
    d = 16
    rng = np.random.default_rng(4)
    x = rng.standard_normal(d).astype(np.float32)
    signs = synth.rademacher_signs(d, 1)
    z = [np.float32(x[i]) * np.float32(signs[i]) for i in range(d)]
    h = 1
    while h < d:
        for i in range(d):
            if i & h == 0:
                a, b = z[i], z[i + h]
                z[i], z[i + h] = np.float32(a + b), np.float32(a - b)
        h *= 2
    c = np.float32(1.0 / math.sqrt(d))
    ref = np.array([np.float32(v * c) for v in z], np.float32)
    assert np.array_equal(O.rotate_keys_f32(x, signs), ref)


# ----------------------------------------------------------------------------- layouts (T3)
@pytest.mark.parametrize("kind", ["key", "value"])
@pytest.mark.parametrize("d,bits", [(64, 2), (64, 4), (128, 2), (128, 4)])
def test_layout_is_a_bijection(kind, d, bits):
    word, bit = O.position_table(kind, d, bits)
    flat = word * 32 + bit
    assert flat.min() >= 0 and flat.max() < d * bits * 32
    assert len(np.unique(flat)) == 32 * d
    assert np.all(bit % bits == 0)
    # every code stays inside one 16-bit half
    assert np.all((bit % 16) + bits <= 16)


@pytest.mark.parametrize("kind", ["key", "value"])
@pytest.mark.parametrize("d,bits", [(64, 2), (64, 4), (128, 2), (128, 4)])
def test_pack_unpack_round_trip(kind, d, bits):
    rng = np.random.default_rng(d * bits)
    codes = rng.integers(0, 2**bits, (3, 32, d)).astype(np.uint8)
    words = O.pack_windows(codes, kind, bits)
    assert words.shape == (3, d * bits) and words.dtype == np.uint32
    assert np.array_equal(O.unpack_windows(words, kind, d, bits), codes)


def test_layout_worked_examples_keys_d128_2bit():
    # Hand-derived from the documented key layout (d = 128, 2 bits, 4 words per lane):
    # lane = 16*(c // 32) + t % 16; word = 4*lane + (c % 8) // 2;
    # bit = 16*(c % 2) + 2*(4*(t // 16) + (c % 32) // 8).
    P = lambda t, c: O.key_code_position(128, 2, t, c)
    assert P(0, 0) == (0, 0)
    assert P(0, 1) == (0, 16)
    assert P(0, 2) == (1, 0)
    assert P(0, 8) == (0, 2)
    assert P(16, 0) == (0, 8)
    assert P(1, 0) == (4, 0)
    assert P(0, 32) == (64, 0)
    assert P(31, 127) == (4 * (16 * 3 + 15) + 3, 16 + 2 * (4 + 3))
    codes = np.zeros((32, 128), np.uint8)
    codes[0, 0], codes[16, 0], codes[0, 1], codes[0, 8] = 1, 2, 3, 1
    w = O.pack_windows(codes[None], "key", 2)[0]
    assert w[0] == 0x1 | (2 << 8) | (3 << 16) | (1 << 2)
    assert np.count_nonzero(w) == 1


def test_layout_worked_examples_values_d128_2bit():
    # value layout (d = 128, 2 bits): lane = 16*g + c % 16 with token t -> (g, j):
    # t < 16: g = t // 4, j = t % 4; else g = (t - 16) // 4, j = 4 + t % 4;
    # pair p = 4*(c // 16) + j // 2; word = 4*lane + p // 8; bit = 4*(p % 8) + 2*(j % 2).
    P = lambda t, c: O.value_code_position(128, 2, t, c)
    assert P(0, 0) == (0, 0)
    assert P(1, 0) == (0, 2)
    assert P(2, 0) == (0, 4)
    assert P(16, 0) == (0, 8)
    assert P(4, 0) == (16 * 4, 0)
    assert P(0, 16) == (0, 16)
    assert P(0, 5) == (4 * 5, 0)
    assert P(0, 32) == (1, 0)
    assert P(31, 127) == (4 * 63 + 3, 30)
    codes = np.zeros((32, 128), np.uint8)
    codes[0, 0], codes[1, 0], codes[16, 0], codes[0, 16] = 3, 1, 2, 1
    w = O.pack_windows(codes[None], "value", 2)[0]
    assert w[0] == 3 | (1 << 2) | (2 << 8) | (1 << 16) and np.count_nonzero(w) == 1


def test_layout_worked_examples_values_d128_4bit():
    # 4 bits: a pair is one byte, four pairs per word: word = 8*lane + p // 4, bit = 8*(p % 4) + 4*(j % 2)
    P = lambda t, c: O.value_code_position(128, 4, t, c)
    assert P(0, 0) == (0, 0)
    assert P(1, 0) == (0, 4)
    assert P(16, 0) == (0, 16)
    assert P(0, 16) == (1, 0)
    assert P(31, 127) == (8 * 63 + 7, 28)


# ----------------------------------------------------------------------------- key codec (T4)
def test_key_window_worked_example():
    # one channel whose 32 rotated values are 0, 1, ..., 31 (2 bits, L = 3):
    # mn = 0, mx = 31, s = fp16(31/3) = 10.3359375, m = 0;
    # thresholds 5.16796875, 15.50390625, 25.83984375 -> codes by hand.
    y = np.zeros((32, 1), np.float32)
    y[:, 0] = np.arange(32)
    codes, m16, s16 = O.key_window_quantize(y, 2)
    assert O.f16_to_f32(m16)[0] == 0.0
    assert O.f16_to_f32(s16)[0] == np.float32(np.float16(31.0 / 3.0))
    expect = np.array([0] * 6 + [1] * 10 + [2] * 10 + [3] * 6)
    assert np.array_equal(codes[:, 0], expect)


@pytest.mark.parametrize("bits", [2, 4])
def test_key_window_bounds(bits):
    L = 2**bits - 1
    rng = np.random.default_rng(bits)
    y = (rng.standard_normal((50, 32, 16)) * rng.uniform(0.1, 3, (50, 1, 16))
         + rng.uniform(-2, 2, (50, 1, 16))).astype(np.float32)
    codes, m16, s16 = O.key_window_quantize(y, bits)
    m, s = O.f16_to_f64(m16), O.f16_to_f64(s16)
    yhat = m[:, None, :] + s[:, None, :] * codes
    # min token -> 0, max token -> L
    amin, amax = y.argmin(1), y.argmax(1)
    assert np.all(np.take_along_axis(codes, amin[:, None, :], 1) == 0)
    assert np.all(np.take_along_axis(codes, amax[:, None, :], 1) == L)
    # reconstruction bound: half a step plus the fp16 rounding of m and s
    mn, mx = y.min(1).astype(np.float64), y.max(1).astype(np.float64)
    slack = np.abs(m - mn) + L * np.abs(s - (mx - mn) / L) + 1e-6
    err = np.abs(yhat - y)
    assert np.all(err <= (s / 2 + slack)[:, None, :])
    assert np.all(yhat >= m[:, None, :]) and np.all(yhat <= (m + L * s)[:, None, :] + 1e-9)


# ----------------------------------------------------------------------------- MXFP4 key metadata
def test_e2m1_values_from_bit_definition():
    # E2M1: sign bit 3, exponent bits 2-1 with bias 1 (exponent 0: subnormal, value m/2),
    # mantissa bit 0.  Decoding a block with exponent byte 127 (scale 1) gives the
    # element values themselves.
    codes = np.array([c % 16 for c in range(32)], np.uint8)
    got = O.mxfp4_decode(codes, np.array([127], np.uint8))
    for c in range(32):
        sg, ex, m = (c % 16) >> 3, ((c % 16) >> 1) & 3, c & 1
        mag = m * 0.5 if ex == 0 else 2.0 ** (ex - 1) * (1 + m / 2)
        assert got[c] == (-mag if sg else mag), c


def _rne_e2m1(v):
    # round to nearest even significand, binade by binade (numpy's round is half-to-even):
    # step 0.5 below 2, step 1 in [2, 4), step 2 from 4, largest value 6
    v = np.abs(np.asarray(v, np.float64))
    r = np.where(v < 2, 0.5 * np.round(v / 0.5), np.where(v < 4, np.round(v), 2 * np.round(v / 2)))
    return np.minimum(r, 6.0)


def test_mxfp4_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(5)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.125, 6.0, 7.0, 7.99], np.float64)
    for trial in range(200):
        blk = rng.uniform(-8, 8, 32)
        blk[:len(ties)] = ties * rng.choice([-1, 1], len(ties))
        blk[len(ties)] = 7.5  # the block maximum lies in [4, 8): shared exponent 0
        blk = np.clip(blk, -7.99, 7.99)
        k = int(rng.integers(-20, 21))   # the same block scaled by 2^k: exponent moves by k
        x = (blk * 2.0 ** k).astype(np.float32)
        codes, e = O.mxfp4_encode(x)
        assert int(e[0]) == 127 + k
        got = O.mxfp4_decode(codes, e)
        want = np.sign(blk) * _rne_e2m1(blk) * 2.0 ** k
        assert np.array_equal(np.abs(got), np.abs(want)), trial
        assert np.array_equal(np.signbit(got) | (got == 0), np.signbit(x.astype(np.float64)) | (want == 0))


def test_mxfp4_shared_exponent_examples():
    def exp_of(amax):
        x = np.zeros(32, np.float32)
        x[7] = amax
        return int(O.mxfp4_encode(x)[1][0])
    # e = floor(log2 amax) - 2, stored + 127
    assert exp_of(6.0) == 127
    assert exp_of(4.0) == 127
    assert exp_of(3.99) == 126
    assert exp_of(1.0) == 125
    assert exp_of(0.75) == 124
    assert exp_of(-12.0) == 128
    assert exp_of(3e38) == 127 + 127 - 2
    assert exp_of(np.float32(2.0 ** -130)) == 0      # clamped at -127
    codes, e = O.mxfp4_encode(np.zeros(64, np.float32))  # all-zero blocks
    assert np.all(codes == 0) and np.all(e == 0)
    # the block maximum keeps at least 3/4 of its magnitude (x / 2^e in [4, 8) -> 4 or 6)
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((100, 32)) * np.exp(rng.uniform(-10, 10, (100, 1)))).astype(np.float32)
    dec = O.mxfp4_decode(*O.mxfp4_encode(x))
    i = np.argmax(np.abs(x), axis=1)
    a = np.abs(x[np.arange(100), i]).astype(np.float64)
    b = np.abs(dec[np.arange(100), i])
    assert np.all(b >= 0.75 * a * (1 - 1e-12)) and np.all(b <= a * 1.5)


@pytest.mark.parametrize("d", [64, 128])
def test_mx_record_layout(d):
    assert O.mx_record_bytes(d) == {64: 48, 128: 80}[d]
    rng = np.random.default_rng(d)
    codes = rng.integers(0, 16, (3, d)).astype(np.uint8)
    exps = rng.integers(0, 255, (3, d // 32)).astype(np.uint8)
    rec = O.mx_pack_record(codes, exps)
    # channel 2i in the low nibble of byte i, channel 2i + 1 in the high nibble
    assert rec[0, 0] == codes[0, 0] | (codes[0, 1] << 4)
    assert rec[1, d // 2 - 1] == codes[1, d - 2] | (codes[1, d - 1] << 4)
    assert np.array_equal(rec[:, d // 2:d // 2 + d // 32], exps)
    assert np.all(rec[:, d // 2 + d // 32:] == 0)
    c2, e2 = O.mx_unpack_record(rec, d)
    assert np.array_equal(c2, codes) and np.array_equal(e2, exps)


@pytest.mark.parametrize("bits", [2, 4])
def test_key_window_mx_codes_are_nearest_levels(bits):
    # with MXFP4 metadata every code is still the nearest level m + s c of the decoded
    # m and s (ties up), clamped to 0 .. L outside the levels
    L = 2**bits - 1
    rng = np.random.default_rng(10 + bits)
    y = (rng.standard_normal((40, 32, 64)) * rng.uniform(0.1, 3, (40, 1, 64))
         + rng.uniform(-2, 2, (40, 1, 64))).astype(np.float32)
    codes, mrec, srec = O.key_window_quantize_mx(y, bits)
    m, s = O.mx_record_values(mrec, 64), O.mx_record_values(srec, 64)
    yy = y.astype(np.float64)
    lev = m[:, None, :, None] + s[:, None, :, None] * np.arange(L + 1)     # [40][1][64][L+1]
    dist = np.abs(yy[..., None] - lev)
    best = dist.min(-1)
    d_code = np.take_along_axis(dist, codes[..., None].astype(np.int64), -1)[..., 0]
    # a code may differ from the exact nearest only by the fp32 rounding of a threshold
    assert np.all(d_code <= best + 1e-5 * (np.abs(yy) + 1))
    assert codes.max() <= L
    # the MX block scale of m bounds how far m can sit from the window minimum
    mn = yy.min(1)
    # (grid spacing at most 2 * 2^e, and saturation from below 8 * 2^e to 6 * 2^e)
    amax_m = np.abs(mn.reshape(40, 2, 32)).max(-1)
    unit = np.repeat(2.0 ** (np.floor(np.log2(amax_m)) - 2), 32, axis=1)
    assert np.all(np.abs(m - mn) <= 2 * unit)


def test_mx_cache_dequantizes_to_its_levels():
    cfg = synth.CONFIGS[1]
    T, d = 128, 64
    tags = synth.modality_layout(cfg, 0, T)
    k = synth.drifting_tensor(cfg, tags, 0, 0, 0, T)
    signs = synth.rademacher_signs(d, 0)
    kc, mrec, srec = O.quantize_keys(k, signs, 2, meta="mxfp4")
    assert mrec.dtype == np.uint8 and mrec.shape == (1, 1, T // 32, 48)
    x = O.dequantize_keys(kc, mrec, srec, signs, 2)[0, 0]
    # rotate back and compare with m + s * code from the records, window by window
    y = O.rotate_keys_f32(x.astype(np.float32), signs).astype(np.float64)
    codes = O.unpack_windows(kc, "key", d, 2)[0, 0]
    m, s = O.mx_record_values(mrec, d)[0, 0], O.mx_record_values(srec, d)[0, 0]
    want = (m[:, None, :] + s[:, None, :] * codes).reshape(T, d)
    assert np.max(np.abs(y - want)) < 1e-5 * (np.max(np.abs(want)) + 1)


# ----------------------------------------------------------------------------- value codec
def test_lloyd_max_matches_textbook_table():
    for line in open(os.path.join(GOLDEN, "lloyd_max_gaussian.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, mse = line.split("|")
        parts = left.split()
        n = int(parts[0])
        pos = np.array([float(v) for v in parts[1:]])
        lv = O.lloyd_max_gaussian(n)
        assert np.allclose(lv[n // 2:], pos, atol=6e-4), (n, lv)
        assert np.allclose(lv[: n // 2], -pos[::-1], atol=6e-4)
        # MSE by numeric integration over the Gaussian density
        x = np.linspace(-12, 12, 400001)
        p = np.exp(-x * x / 2) / math.sqrt(2 * math.pi)
        th = (lv[:-1] + lv[1:]) / 2
        got = ((x - lv[np.searchsorted(th, x)]) ** 2 * p).sum() * (x[1] - x[0])
        assert abs(got - float(mse)) < 2e-4 * max(1.0, float(mse) * 100)


def test_value_scale_closed_forms():
    d = 128
    v = np.full((1, d), -3.0, np.float32)
    assert O.value_scale_f32(v)[0] == np.float32(3.0)
    e = np.zeros((1, d), np.float32)
    e[0, 77] = 8.0
    assert O.value_scale_f32(e)[0] == np.float32(8.0 / math.sqrt(d))
    x = np.random.default_rng(0).standard_normal((100, d)).astype(np.float32)
    ref = np.sqrt((x.astype(np.float64) ** 2).mean(1))
    assert np.max(np.abs(O.value_scale_f32(x) - ref) / ref) < 1e-6


def test_value_scale_tree_order():
    # the stride-halving tree: pairs (i, i+d/2) first.  With d = 4 and values
    # whose squares are 2^24, 1, -.. the tree ((a+c)+(b+d)) differs from a
    # left-to-right sum; check the oracle follows the tree.
    v = np.array([[4096.0, 1.0, 1.0, 1.0]], np.float32)   # squares 2^24, 1, 1, 1
    S_tree = np.float32(np.float32(2**24 + 1.0) + np.float32(2.0))  # (a^2+c^2) + (b^2+d^2)
    assert O.value_scale_f32(v)[0] == np.sqrt(S_tree / np.float32(4))


def test_value_rotation_is_U_transpose_v():
    d = 32
    rng = np.random.default_rng(9)
    U = rng.standard_normal((d, d)).astype(np.float32)   # deliberately not symmetric
    v = rng.standard_normal((6, d)).astype(np.float32)
    got = O.rotate_values_f32(v, U).astype(np.float64)
    ref = v.astype(np.float64) @ U.astype(np.float64)     # (U^T v)_i = sum_k U[k][i] v_k
    assert np.max(np.abs(got - ref)) < 1e-4
    assert np.max(np.abs(got - v.astype(np.float64) @ U.T.astype(np.float64))) > 1e-2


def test_value_worked_example_identity_rotation():
    # U = I, one token with v = sigma * (0.1, -0.1, 1.2, -1.2, 0, ...) scaled so
    # that sigma is exactly representable; 2-bit levels +-0.45288, +-1.5107,
    # boundaries -0.98181, 0, 0.98181 -> codes 2, 1, 3, 0, 2 (0 >= 0 counts).
    d = 64
    v = np.zeros((1, 1, 1, d), np.float32)
    v[..., :4] = [0.1, -0.1, 1.2, -1.2]
    U = np.eye(d, dtype=np.float32)[None]
    lv = O.value_codebook_f16(2)
    words, sig16 = O.quantize_values(np.repeat(np.repeat(v, 32, 1), 1, 2), np.zeros((1, 32), np.uint8), U, lv, 2)
    codes = O.unpack_windows(words, "value", d, 2)[0, 0, 0]
    sig = O.f16_to_f32(sig16)[0, 0, 0]
    assert sig == np.float32(np.float16(math.sqrt((0.01 + 0.01 + 1.44 + 1.44) / d)))
    beta = O.value_boundaries_f32(lv)
    assert np.array_equal(codes[0, :5], np.array(
        [sum(x >= sig * b for b in beta) for x in [0.1, -0.1, 1.2, -1.2, 0.0]]))
    # sigma * beta = (-0.2090, 0, 0.2090): 0.1 -> 2, -0.1 -> 1, 1.2 -> 3, -1.2 -> 0, 0 -> 2
    assert list(codes[0, :5]) == [2, 1, 3, 0, 2]


# ----------------------------------------------------------------------------- codec error (T5)
def _codec_mse(cfg_id, kbits, vbits, seed=0):
    cfg = synth.CONFIGS[cfg_id]
    T = 256
    tags = synth.modality_layout(cfg, seed, T)
    k = synth.drifting_tensor(cfg, tags, seed, 0, 0, T)
    v = synth.drifting_tensor(cfg, tags, seed, 1, 0, T)
    d = cfg.head_dim
    signs = synth.rademacher_signs(d, seed)
    U = synth.value_rotations(d, seed)
    kc, km, ks = O.quantize_keys(k, signs, kbits)
    lv = O.value_codebook_f16(vbits)
    vc, vs = O.quantize_values(v, tags, U, lv, vbits)
    khat = O.dequantize_keys(kc, km, ks, signs, kbits)                   # [B][H][T][d]
    vhat = O.dequantize_values(vc, vs, tags, U, lv, vbits)
    kref = k.transpose(0, 2, 1, 3).astype(np.float64)
    vref = v.transpose(0, 2, 1, 3).astype(np.float64)
    rel = lambda a, b: np.mean((a - b) ** 2) / np.mean(b ** 2)
    return rel(khat, kref), rel(vhat, vref)


@pytest.mark.parametrize("cfg_id", [1, 2])
def test_four_bits_beat_two_bits(cfg_id):
    k2, v2 = _codec_mse(cfg_id, 2, 2)
    k4, v4 = _codec_mse(cfg_id, 4, 4)
    assert k4 < 0.25 * k2 and v4 < 0.25 * v2
    # values: per-token RMS scale + Lloyd-Max -> distortion near the textbook MSE
    assert 0.08 < v2 < 0.16 and 0.005 < v4 < 0.02
    # keys: window min-max at 2 bits keeps the error well below a global range
    assert k2 < 0.2


def test_value_codec_reaches_lloyd_max_distortion_on_gaussian():
    d = 128
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 4096, 1, d)).astype(np.float32)
    tags = np.zeros((1, 4096), np.uint8)
    U = np.eye(d, dtype=np.float32)[None]
    for bits, target in [(2, 0.1175), (4, 0.009497)]:
        lv = O.value_codebook_f16(bits)
        vc, vs = O.quantize_values(v, tags, U, lv, bits)
        vhat = O.dequantize_values(vc, vs, tags, U, lv, bits)[0, 0]
        mse = np.mean((vhat - v[0, :, 0].astype(np.float64)) ** 2)
        assert abs(mse - target) < 0.06 * target, (bits, mse)


# ----------------------------------------------------------------------------- attention (T7, T8)
def _tiny_cache(seed=0, T=256, d=64, G=2):
    cfg = synth.CONFIGS[1]
    tags = synth.modality_layout(cfg, seed, T)
    k = synth.drifting_tensor(cfg, tags, seed, 0, 0, T)
    v = synth.drifting_tensor(cfg, tags, seed, 1, 0, T)
    signs = synth.rademacher_signs(d, seed)
    U = synth.value_rotations(d, seed)
    lv = O.value_codebook_f16(2)
    kc, km, ks = O.quantize_keys(k, signs, 2)
    vc, vs = O.quantize_values(v, tags, U, lv, 2)
    cache = dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags,
                 key_bits=2, value_bits=2)
    return cache, signs, U, lv


def test_attention_brute_force_equals_rotated_domain_formula():
    # The fused kernel's restructuring: q . R^{-1} y_hat = (R^{-T} q) . y_hat and
    # sum_t p_t U_m(t) v'_t = sum_m U_m (sum_{t in m} p_t v'_t).  Both sides in fp64.
    cache, signs, U, lv = _tiny_cache()
    q = synth.queries(synth.CONFIGS[1], 0)
    out = O.decode_attention(q, [256], cache, signs, U, lv)
    d, T = 64, 256
    codes_k = O.unpack_windows(cache["k_codes"], "key", d, 2).reshape(1, 1, T, d)[0, 0]
    yhat = (O.f16_to_f64(cache["k_min"])[0, 0].repeat(32, 0)
            + O.f16_to_f64(cache["k_scale"])[0, 0].repeat(32, 0) * codes_k)
    codes_v = O.unpack_windows(cache["v_codes"], "value", d, 2).reshape(T, d)
    vprime = O.f16_to_f64(cache["v_scale"])[0, 0][:, None] * O.f16_to_f64(lv)[codes_v]
    c = float(O.rotation_constant(d))
    H = O.sylvester(d)
    for h in range(2):
        qr = (H @ (signs * q[0, h].astype(np.float64))) / (c * d)          # R^{-T} q
        s = (yhat @ qr) / math.sqrt(d)
        p = np.exp(s - s.max())
        acc = np.zeros((3, d))
        for m in range(3):
            sel = cache["modality"][0] == m
            acc[m] = p[sel] @ vprime[sel]
        fused = sum(U[m].astype(np.float64) @ acc[m] for m in range(3)) / p.sum()
        assert np.max(np.abs(fused - out[0, h])) < 1e-12 * max(1.0, np.max(np.abs(out[0, h])))


def test_attention_special_cases():
    cache, signs, U, lv = _tiny_cache()
    d = 64
    vals = O.dequantize_values(cache["v_codes"], cache["v_scale"], cache["modality"], U, lv, 2)[0, 0]
    q = synth.queries(synth.CONFIGS[1], 1)
    # one token: the output is that token's value
    out1 = O.decode_attention(q, [1], cache, signs, U, lv)
    assert np.allclose(out1[0, 0], vals[0], atol=1e-12)
    # zero query: uniform attention -> mean of the values over the prefix
    out0 = O.decode_attention(np.zeros_like(q), [100], cache, signs, U, lv)
    assert np.allclose(out0[0, 1], vals[:100].mean(0), atol=1e-12)
    # empty prefix -> zeros
    oute = O.decode_attention(q, [0], cache, signs, U, lv)
    assert np.all(oute == 0)


def test_attention_identity_rotation_single_modality_is_plain_attention():
    cache, signs, U, lv = _tiny_cache()
    d, T = 64, 256
    I3 = np.stack([np.eye(d, dtype=np.float32)] * 3)
    q = synth.queries(synth.CONFIGS[1], 2)
    out = O.decode_attention(q, [T], cache, signs, I3, lv)
    keys = O.dequantize_keys(cache["k_codes"], cache["k_min"], cache["k_scale"], signs, 2)[0, 0]
    codes_v = O.unpack_windows(cache["v_codes"], "value", d, 2).reshape(T, d)
    vals = O.f16_to_f64(cache["v_scale"])[0, 0][:, None] * O.f16_to_f64(lv)[codes_v]
    for h in range(2):
        s = keys @ q[0, h].astype(np.float64) / 8.0
        p = np.exp(s - s.max())
        assert np.allclose(out[0, h], p @ vals / p.sum(), atol=1e-12)


def test_gqa_head_mapping():
    cfg = synth.CONFIGS[2]
    cache = synth.random_packed_cache(cfg, 0, length=64)
    d = cfg.head_dim
    signs = synth.rademacher_signs(d, 0)
    U = synth.value_rotations(d, 0)
    lv = O.value_codebook_f16(2)
    q = np.zeros((1, 16, d), np.float32)
    out = O.decode_attention(q, [64], cache, signs, U, lv)
    vals = O.dequantize_values(cache["v_codes"], cache["v_scale"], cache["modality"], U, lv, 2)
    for h in range(16):
        assert np.allclose(out[0, h], vals[0, h // 8].mean(0), atol=1e-12)
    assert not np.allclose(out[0, 0], out[0, 8])


# ----------------------------------------------------------------------------- streaming
def test_stream_schedule_follows_the_pages():
    """[paper] §3.1 Implementation details: keys are quantized every 128 tokens in
    groups of 32; values keep a 128-token sliding FP16 window.  Checked on every
    length up to 1000: key_packed is the largest multiple of 128 <= n; every value
    among the 128 most recent stays FP16 and at most 31 older ones wait for their
    32-token window to complete."""
    for n in range(1001):
        kp, vp = O.stream_packed_lengths(n)
        assert kp % 128 == 0 and kp <= n < kp + 128
        assert vp % 32 == 0 and vp <= max(0, n - 128)
        assert n - vp < 128 + 32 or n < 128
        assert vp <= kp  # a token with a quantized value also has a quantized key
    assert [O.stream_packed_lengths(n) for n in (0, 127, 128, 159, 160, 255, 256, 300, 384)] == [
        (0, 0), (0, 0), (128, 0), (128, 0), (128, 32), (128, 96), (256, 128), (256, 160), (384, 256)]


def test_key_groups_do_not_depend_on_flush_granularity():
    """Quantizing 128 tokens at once or as four 32-token groups gives the same codes
    and metadata: the range belongs to the group alone ([paper] §3.1, g = 32)."""
    cfg = synth.CONFIGS[1]
    rng = np.random.default_rng(11)
    k = rng.standard_normal((1, 128, 1, cfg.head_dim)).astype(np.float32)
    signs = synth.rademacher_signs(cfg.head_dim, 0)
    whole = O.quantize_keys(k, signs, 2)
    parts = [O.quantize_keys(k[:, 32 * i:32 * i + 32], signs, 2) for i in range(4)]
    for j in range(3):
        assert np.array_equal(whole[j], np.concatenate([p[j] for p in parts], axis=2))


def test_streaming_attention_special_cases():
    """No packed token: plain attention over the stored keys and values (brute force
    over a tiny input).  Every token packed: the non-streaming decode."""
    cfg = synth.CONFIGS[1]
    d, G = cfg.head_dim, cfg.q_heads // cfg.kv_heads
    rng = np.random.default_rng(5)
    T = 96
    k = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    q = rng.standard_normal((1, cfg.q_heads, d)).astype(np.float32)
    signs = synth.rademacher_signs(d, 0)
    U = synth.value_rotations(d, 0)
    lv = O.value_codebook_f16(2)
    tags = np.zeros((1, T), np.uint8)
    kc, km, ks = O.quantize_keys(k, signs, 2)
    vc, vs = O.quantize_values(v, tags, U, lv, 2)
    cache = dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags, key_bits=2, value_bits=2)
    out = O.decode_attention_streaming(q, [T], cache, k, v, signs, U, lv)   # T < 128: nothing packed
    for h in range(cfg.q_heads):
        logits = [sum(float(q[0, h, c]) * float(k[0, t, 0, c]) for c in range(d)) / math.sqrt(d) for t in range(T)]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        ref = [sum(w[t] * float(v[0, t, 0, c]) for t in range(T)) / sum(w) for c in range(d)]
        assert np.allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)
    # a 300-token stream: keys of tokens 256.. and values of tokens 160.. unquantized;
    # against attention over explicitly assembled keys and values
    T, n = 320, 300
    k = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    tags = np.zeros((1, T), np.uint8)
    kc, km, ks = O.quantize_keys(k, signs, 2)
    vc, vs = O.quantize_values(v, tags, U, lv, 2)
    cache = dict(k_codes=kc, k_min=km, k_scale=ks, v_codes=vc, v_scale=vs, modality=tags, key_bits=2, value_bits=2)
    out = O.decode_attention_streaming(q, [n], cache, k, v, signs, U, lv)
    kq = O.dequantize_keys(kc, km, ks, signs, 2)[0, 0]
    vq = O.dequantize_values(vc, vs, tags, U, lv, 2)[0, 0]
    keys = np.concatenate([kq[:256], k[0, 256:n, 0].astype(np.float64)])
    vals = np.concatenate([vq[:160], v[0, 160:n, 0].astype(np.float64)])
    for h in range(cfg.q_heads):
        assert np.allclose(out[0, h], O.attention_f64(q[0, h], keys, vals, 1.0 / math.sqrt(d)), rtol=1e-12, atol=1e-14)
    full = O.decode_attention(q, [n], cache, signs, U, lv)
    assert not np.allclose(out, full)  # the unquantized tokens matter


# ----------------------------------------------------------------------------- value-rotation calibration
def test_calibration_closed_form_diagonal_moment():
    """A diagonal second moment with distinct entries: its eigenvectors are the unit
    vectors in descending order, so U = P H / sqrt(d) with P that permutation."""
    d = 64
    c = np.random.default_rng(2).permutation(np.arange(1, d + 1, dtype=np.float64))
    v = np.diag(np.sqrt(c * d))                      # one token per channel
    U = O.calibrate_value_rotation(v)
    P = np.zeros((d, d))
    P[np.argsort(-c), np.arange(d)] = 1.0
    assert np.allclose(U, P @ O.sylvester(d) / 8.0, atol=1e-12)
    assert np.allclose(U.T @ U, np.eye(d), atol=1e-12)


def test_calibration_weights_count_like_repeated_tokens():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((400, 64)) * np.linspace(3, 0.1, 64)   # full rank, distinct eigenvalues
    w = rng.integers(1, 4, 400)
    assert np.allclose(O.calibrate_value_rotation(v, w.astype(float)),
                       O.calibrate_value_rotation(np.repeat(v, w, axis=0)), atol=1e-10)


@pytest.mark.parametrize("d,heavy", [(64, False), (64, True), (128, False), (128, True)])
def test_matched_rotation_beats_shared_and_transferred(d, heavy):
    """On per-modality clusters, each modality's calibrated rotation quantizes its
    held-out values with lower error than one randomized Hadamard shared by all
    modalities and than the other modalities' rotations ([paper] §1 and §2.3:
    heterogeneous value geometry)."""
    cal, held = synth.modality_clusters(d, 0, n=2048, heavy_tail=heavy)
    held = [h[:1024] for h in held]
    Us = [O.calibrate_value_rotation(c) for c in cal]
    signs = synth.rademacher_signs(d, 0).astype(np.float64)
    shared = (O.sylvester(d) * signs[None, :]).T / math.sqrt(d)   # U with U^T v = H D v / sqrt(d)
    for m in range(3):
        matched = O.value_codec_mse(held[m], Us[m])
        assert matched < O.value_codec_mse(held[m], shared), (d, heavy, m)
        for o in range(3):
            if o != m:
                assert matched < O.value_codec_mse(held[m], Us[o]), (d, heavy, m, o)
