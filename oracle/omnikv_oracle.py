"""Plain CPU oracle for the OmniKVQuant hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the benchmark's CPU-baseline leg may import, call or execute this
module.  The library (HIP kernels + C ABI + Python binding) never does, and
this module shares no code, table or constant with it.

What it computes, and from which passage
----------------------------------------
Source pages (cited by title and section):
  [paper]  "OmniKVQuant: KV Cache Quantization for Omni-LLMs" (paper text)
  [digest] "OmniKVQuant：面向 Omni-LLM 的 KV 缓存量化" (Chinese digest of the paper)

* Keys: a randomized Hadamard rotation shared by every modality, inherited
  from TurboQuant ([paper] §1 Introduction; [digest] "这篇论文解决什么问题",
  "关联工作"), then a min-max range per 32-token window of the stream mapped
  onto a fixed codebook ([paper] §1 and §3.1 Implementation details, g = 32;
  [digest] "方法概览"), with a minimum m_gc and a scale s_gc per group g and
  channel c stored in FP16 ([paper] §3.3 Error comparison).
* Values: a separate basis U_m per modality m in {V, A, L} ([paper] §2.3),
  then a fixed codebook.  The per-token scale and the codebook's values are
  not printed; the reading used here is TurboQuant's fixed Lloyd-Max codebook
  for N(0,1), applied to v'/sigma with sigma the token's RMS.
* Decode: attention over the dequantized cache.  The pages' fused kernel
  reorders this computation ([paper] §1, Fig. 1(d)); the oracle computes the
  plain definition, softmax(scale * q . k_hat) . v_hat, in float64.
* Value-rotation calibration ([paper] §2.3: a basis U_m calibrated for each
  modality; [digest] 方法概览: an attention-contribution-weighted covariance,
  eigendecomposed).  Reading: the weighted second moment, its eigenvectors in
  descending order composed with the normalized Hadamard ("modality-aware
  correction of the Hadamard rotation", [paper] §2.3).
* Error metrics ([paper] §3.3 Error comparison, Table 3): key reconstruction MSE,
  KL divergence of the attention distributions, attention-output MSE, each by its
  plain definition.
* Streaming generation ([paper] §3.1 Implementation details, captioning):
  keys are quantized every 128 tokens in groups of 32; values stay in a
  128-token sliding FP16 window before quantization.  Recent tokens enter the
  attention as stored (no quantization).

Fixed arithmetic of the codec (fp32, in this exact order, so that the GPU
codes and metadata can be compared bit for bit):
  rotation   y = c_d * FWHT(D x): z = D x; butterfly stages h = 1, 2, ..., d/2,
             each mapping (z_i, z_{i+h}) -> (z_i + z_{i+h}, z_i - z_{i+h})
             for i with bit h clear; then one multiply by c_d = fp32(1/sqrt(d)).
  key range  mn, mx over the 32 tokens of a window, each + 0 (so that a zero
             extreme is +0); m = fp16(mn);
             s = fp16((mx - mn) / L) with L = 2^bits - 1 (IEEE fp32 division,
             fp16 round-to-nearest-even).
  key code   theta_j = m + s * (j + 1/2) (product and sum each rounded to fp32),
             code = #{ j < L : y >= theta_j }.
  MXFP4 key metadata (the pages' default format, [paper] §3.1 Implementation
             details): the window's vectors mn and (mx - mn) / L are each cut into
             blocks of 32 consecutive channels; a block stores one E8M0 exponent
             e = floor(log2 max|x|) - 2 (clamped to [-127, 127]; -127 for an
             all-zero block) and 32 E2M1 elements, x * 2^-e rounded to the nearest
             of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, sign kept.
             The codes use the decoded m and s in the key-code rule above.
  value scale  S = sum of v_i^2 by the stride-halving tree (pairs (i, i + d/2),
             then (i, i + d/4), ..., each square and sum rounded to fp32);
             sigma = sqrt(S / d) (correctly rounded); stored fp16.
  value rot  v'_i = sum_k U[k][i] v_k accumulated for k = 0, 1, ..., d-1 with
             every product and every partial sum rounded to fp32 (no fma).
  value code theta_j = fp32(sigma_fp16) * beta_j with beta_j the fp32 midpoint of
             adjacent fp16 codebook levels; code = #{ j : v' >= theta_j }.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

F32 = np.float32
WINDOW = 32


# ----------------------------------------------------------------------------- fp16 helpers
def f16_bits(x) -> np.ndarray:
    """fp32 -> IEEE binary16 bit patterns, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------- key rotation
def rotation_constant(d: int) -> np.float32:
    """c_d: the fp32 number nearest to 1/sqrt(d)."""
    return F32(1.0 / math.sqrt(d))


def rotate_keys_f32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = c_d * H_d (D x) in fp32, butterfly stages h = 1, 2, ..., d/2 in order.

    Randomized Hadamard rotation of TurboQuant ([paper] §1 Introduction;
    [digest] "关联工作").  x: fp32 [..., d]; signs: +-1 [d] (the diagonal D).
    """
    x = np.asarray(x, dtype=F32)
    d = x.shape[-1]
    lead = x.shape[:-1]
    z = (x * np.asarray(signs, dtype=F32)).reshape(-1, d)
    h = 1
    while h < d:
        z = z.reshape(-1, d // (2 * h), 2, h)
        a = z[:, :, 0, :]
        b = z[:, :, 1, :]
        z = np.stack([a + b, a - b], axis=2).reshape(-1, d)
        h *= 2
    return (z * rotation_constant(d)).reshape(*lead, d)


def sylvester(d: int) -> np.ndarray:
    """H_d with H_ij = (-1)^popcount(i & j), float64."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pc = np.zeros_like(bits)
    while bits.any():
        pc += bits & 1
        bits >>= 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def inverse_key_rotation_f64(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x = R^{-1} y for R = c_d H D, in float64: x = D H y / (c_d d)."""
    d = y.shape[-1]
    H = sylvester(d)
    c = float(rotation_constant(d))
    return (np.asarray(y, dtype=np.float64) @ H) * (np.asarray(signs, np.float64) / (c * d))


# ----------------------------------------------------------------------------- packed layouts
def key_code_position(d: int, bits: int, t: int, c: int):
    """(word, bit) of key code (window token t, rotated channel c) in a window block.

    A window block holds the 32 x d codes of one (sequence, KV head, window) in
    d * bits uint32 words.  Lane l = 16 g + rho owns d*bits/64 consecutive words
    and holds tokens {rho, rho + 16} (tau = 0, 1) of channels g*d/4 + 8 s + j
    (s < d/32, j < 8).  In each word, j even sits in bits 0..15 and j odd in
    bits 16..31, at a slot (bits-wide field) chosen per case below.
    """
    tau, rho = divmod(t, 16)
    g, r = divmod(c, d // 4)
    s, j = divmod(r, 8)
    i, e = divmod(j, 2)
    per_lane = d * bits // 64
    if (d, bits) == (128, 2):
        lw, slot = i, 4 * tau + s
    elif (d, bits) == (128, 4):
        lw, slot = 4 * tau + i, s
    elif (d, bits) == (64, 2):
        lw, slot = i & 1, 4 * (i >> 1) + 2 * tau + s
    elif (d, bits) == (64, 4):
        lw, slot = i, 2 * tau + s
    else:
        raise ValueError((d, bits))
    return (16 * g + rho) * per_lane + lw, 16 * e + bits * slot


def value_code_position(d: int, bits: int, t: int, c: int):
    """(word, bit) of value code (window token t, channel c) in a window block.

    Lane l = 16 g + rho holds channels 16 u + rho (u < d/16) of the eight
    tokens {4g .. 4g+3, 16+4g .. 16+4g+3} (index j = 0..7 in that order).  The
    codes of tokens j = 2i and 2i + 1 of one channel form a pair p = 4 u + i of
    2*bits bits (the even token in the low half of the pair); the lane's words
    hold 16/bits pairs each, pair p in word p // (16/bits) at bit
    2*bits*(p % (16/bits)).
    """
    u, rho = divmod(c, 16)
    if t < 16:
        g, j = divmod(t, 4)
    else:
        g, j = divmod(t - 16, 4)
        j += 4
    if (d, bits) not in ((64, 2), (64, 4), (128, 2), (128, 4)):
        raise ValueError((d, bits))
    p = 4 * u + j // 2
    ppw = 16 // bits
    per_lane = d * bits // 64
    return (16 * g + rho) * per_lane + p // ppw, 2 * bits * (p % ppw) + bits * (j % 2)


def _position_table(fn, d: int, bits: int):
    word = np.empty((WINDOW, d), dtype=np.int64)
    bit = np.empty((WINDOW, d), dtype=np.int64)
    for t in range(WINDOW):
        for c in range(d):
            word[t, c], bit[t, c] = fn(d, bits, t, c)
    return word, bit


_TABLES = {}


def position_table(kind: str, d: int, bits: int):
    key = (kind, d, bits)
    if key not in _TABLES:
        fn = key_code_position if kind == "key" else value_code_position
        _TABLES[key] = _position_table(fn, d, bits)
    return _TABLES[key]


def pack_windows(codes: np.ndarray, kind: str, bits: int) -> np.ndarray:
    """codes [..., 32, d] (ints < 2^bits) -> uint32 words [..., d*bits]."""
    d = codes.shape[-1]
    word, bit = position_table(kind, d, bits)
    lead = codes.shape[:-2]
    c = codes.reshape(-1, WINDOW * d).astype(np.uint64)
    out = np.zeros((c.shape[0], d * bits), dtype=np.uint64)
    shifted = c << bit.reshape(-1).astype(np.uint64)
    for k in range(WINDOW * d):          # positions are disjoint: OR == add
        out[:, word.flat[k]] |= shifted[:, k]
    return out.astype(np.uint32).reshape(*lead, d * bits)


def unpack_windows(words: np.ndarray, kind: str, d: int, bits: int) -> np.ndarray:
    """uint32 words [..., d*bits] -> codes uint8 [..., 32, d]."""
    word, bit = position_table(kind, d, bits)
    lead = words.shape[:-1]
    w = words.reshape(-1, d * bits).astype(np.uint64)
    vals = (w[:, word.reshape(-1)] >> bit.reshape(-1).astype(np.uint64)) & np.uint64(2**bits - 1)
    return vals.astype(np.uint8).reshape(*lead, WINDOW, d)


# ----------------------------------------------------------------------------- key codec
def key_window_quantize(y: np.ndarray, bits: int):
    """One window's range metadata and codes from rotated keys y: fp32 [..., 32, d].

    Returns (codes uint8 [..., 32, d], m fp16 bits [..., d], s fp16 bits [..., d]).
    """
    L = 2**bits - 1
    y = np.asarray(y, dtype=F32)
    mn = y.min(axis=-2) + F32(0)     # "+ 0": a zero extreme is +0
    mx = y.max(axis=-2) + F32(0)
    step = (mx - mn) / F32(L)
    m16, s16 = f16_bits(mn), f16_bits(step)
    m, s = f16_to_f32(m16), f16_to_f32(s16)
    codes = np.zeros(y.shape, dtype=np.uint8)
    for j in range(L):
        theta = m + s * F32(j + 0.5)
        codes += (y >= theta[..., None, :]).astype(np.uint8)
    return codes, m16, s16


# ----------------------------------------------------------------------------- MXFP4 metadata
# E2M1 element values by code (sign bit 3 clear), from the element format: code bits
# (e1 e0 m), exponent bias 1, exponent 0 subnormal with value m / 2.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def mx_record_bytes(d: int) -> int:
    """Bytes of one window's MXFP4 metadata record for one vector (m or s): d/2 bytes
    of E2M1 codes (channel 2i in the low nibble of byte i), d/32 exponent bytes, then
    zero padding to a multiple of 16 bytes."""
    return (d // 2 + d // MX_BLOCK + 15) // 16 * 16


def mxfp4_encode(x: np.ndarray):
    """fp32 [..., n*32] -> (codes uint8 [..., n*32] in 0..15, exponent bytes uint8 [..., n]).

    Each block of 32 consecutive elements shares the exponent e = floor(log2 amax) - 2,
    stored as e + 127; every element is x * 2^-e rounded to the nearest E2M1 value with
    ties to the even code (values beyond 6 take 6), its sign in bit 3.
    """
    x = np.asarray(x, dtype=np.float64)   # fp32 inputs are exact in fp64
    shape = x.shape
    blocks = x.reshape(shape[:-1] + (shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, k = np.frexp(amax)                  # amax = f * 2^k, f in [0.5, 1): floor(log2 amax) = k - 1
    e = np.where(amax > 0, k - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    v = np.abs(blocks) * np.exp2(-e.astype(np.float64))[..., None]   # exact scaling
    dist = np.abs(v[..., None] - E2M1_VALUES)                         # [..., 32, 8]
    best = dist.min(axis=-1, keepdims=True)
    tie = dist == best
    # the nearest code; where two are equally near, the even one
    even_pick = np.where(tie[..., 0::2].any(axis=-1),
                         2 * np.argmax(tie[..., 0::2], axis=-1), -1)
    code = np.where(tie.sum(axis=-1) > 1, even_pick, np.argmax(tie, axis=-1))
    sign = np.signbit(blocks).astype(np.int64)
    codes = (code + 8 * sign).astype(np.uint8).reshape(shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp4_decode(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """Inverse of mxfp4_encode: float64 values (exact)."""
    codes = np.asarray(codes, dtype=np.int64)
    shape = codes.shape
    c = codes.reshape(shape[:-1] + (shape[-1] // MX_BLOCK, MX_BLOCK))
    mag = E2M1_VALUES[c & 7] * np.exp2(np.asarray(exps, np.float64) - 127.0)[..., None]
    return np.where(c & 8, -mag, mag).reshape(shape)


def mx_pack_record(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """Per-window record bytes [..., mx_record_bytes(d)] from codes [..., d], exps [..., d/32]."""
    codes = np.asarray(codes, np.uint8)
    d = codes.shape[-1]
    rec = np.zeros(codes.shape[:-1] + (mx_record_bytes(d),), np.uint8)
    rec[..., :d // 2] = codes[..., 0::2] | (codes[..., 1::2] << 4)
    rec[..., d // 2:d // 2 + d // MX_BLOCK] = exps
    return rec


def mx_unpack_record(rec: np.ndarray, d: int):
    """(codes [..., d], exps [..., d/32]) from record bytes."""
    rec = np.asarray(rec, np.uint8)
    codes = np.empty(rec.shape[:-1] + (d,), np.uint8)
    codes[..., 0::2] = rec[..., :d // 2] & 15
    codes[..., 1::2] = rec[..., :d // 2] >> 4
    return codes, rec[..., d // 2:d // 2 + d // MX_BLOCK]


def mx_record_values(rec: np.ndarray, d: int) -> np.ndarray:
    """Decoded float64 vector [..., d] of a record."""
    return mxfp4_decode(*mx_unpack_record(rec, d))


def key_window_quantize_mx(y: np.ndarray, bits: int):
    """key_window_quantize with MXFP4 metadata.  Returns (codes uint8 [..., 32, d],
    m record uint8 [..., R], s record uint8 [..., R]), R = mx_record_bytes(d)."""
    L = 2**bits - 1
    y = np.asarray(y, dtype=F32)
    mn = y.min(axis=-2) + F32(0)
    mx = y.max(axis=-2) + F32(0)
    step = (mx - mn) / F32(L)
    mc, me = mxfp4_encode(mn)
    sc, se = mxfp4_encode(step)
    m = mxfp4_decode(mc, me).astype(F32)   # exact: E2M1 times a power of two
    s = mxfp4_decode(sc, se).astype(F32)
    codes = np.zeros(y.shape, dtype=np.uint8)
    for j in range(L):
        theta = m + s * F32(j + 0.5)
        codes += (y >= theta[..., None, :]).astype(np.uint8)
    return codes, mx_pack_record(mc, me), mx_pack_record(sc, se)


def quantize_keys(k: np.ndarray, signs: np.ndarray, bits: int, meta: str = "fp16"):
    """Quantize a chunk of keys.  k: fp32 [B][n][Hkv][d], n a multiple of 32.

    Returns (k_codes uint32 [B][Hkv][n/32][d*bits], k_min, k_scale); the metadata are
    fp16 bits [B][Hkv][n/32][d] (meta "fp16") or MXFP4 records uint8
    [B][Hkv][n/32][mx_record_bytes(d)] (meta "mxfp4").  Window w of the result is
    window t0/32 + w of the cache.
    """
    B, n, H, d = k.shape
    assert n % WINDOW == 0 and meta in ("fp16", "mxfp4")
    y = rotate_keys_f32(k, signs)                                # [B][n][H][d]
    y = y.transpose(0, 2, 1, 3).reshape(B, H, n // WINDOW, WINDOW, d)
    quant = key_window_quantize if meta == "fp16" else key_window_quantize_mx
    codes, km, ks = quant(y, bits)
    return pack_windows(codes, "key", bits), km, ks


# ----------------------------------------------------------------------------- value codec
def lloyd_max_gaussian(n_levels: int, iters: int = 4000) -> np.ndarray:
    """Lloyd-Max levels for N(0,1) (float64, ascending).

    Alternates the two optimality conditions: every threshold is the midpoint
    of its neighbouring levels, every level is the conditional mean of N(0,1)
    between its thresholds, E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    """
    phi = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi) if math.isfinite(x) else 0.0
    Phi = lambda x: 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) if math.isfinite(x) else (1.0 if x > 0 else 0.0)
    lv = np.linspace(-2.0, 2.0, n_levels)
    for _ in range(iters):
        th = [-math.inf] + [0.5 * (lv[i] + lv[i + 1]) for i in range(n_levels - 1)] + [math.inf]
        lv = np.array([(phi(th[i]) - phi(th[i + 1])) / (Phi(th[i + 1]) - Phi(th[i]))
                       for i in range(n_levels)])
    return lv


def value_codebook_f16(bits: int) -> np.ndarray:
    """Fixed value codebook: Lloyd-Max levels for N(0,1) rounded to fp16 (bit patterns)."""
    return f16_bits(lloyd_max_gaussian(2**bits).astype(np.float32))


def value_boundaries_f32(levels16: np.ndarray) -> np.ndarray:
    """beta_j = (l_j + l_{j+1}) / 2 in fp32 from fp16 levels."""
    lv = f16_to_f32(levels16)
    return ((lv[:-1] + lv[1:]) / F32(2)).astype(F32)


def value_scale_f32(v: np.ndarray) -> np.ndarray:
    """sigma = sqrt(S/d), S = stride-halving tree sum of v_i^2, all fp32.  v: [..., d]."""
    v = np.asarray(v, dtype=F32)
    d = v.shape[-1]
    S = v * v
    w = d // 2
    while w >= 1:
        S = S[..., :w] + S[..., w:2 * w]
        w //= 2
    return np.sqrt(S[..., 0] / F32(d))


def rotate_values_f32(v: np.ndarray, U: np.ndarray) -> np.ndarray:
    """v'_i = sum_k U[k][i] v_k, k ascending, each product and sum rounded to fp32."""
    v = np.asarray(v, dtype=F32)
    U = np.asarray(U, dtype=F32)
    acc = np.zeros(v.shape, dtype=F32)
    for kk in range(v.shape[-1]):
        acc = acc + U[kk][None, :] * v[..., kk:kk + 1]
    return acc


def quantize_values(v: np.ndarray, tags: np.ndarray, U: np.ndarray, levels16: np.ndarray, bits: int):
    """Quantize a chunk of values.

    v: fp32 [B][n][Hkv][d]; tags: uint8 [B][n] modality of each token (rotation
    index); U: fp32 [M][d][d]; levels16: fp16 codebook bits [2^bits].
    Returns (v_codes uint32 [B][Hkv][n/32][d*bits], v_scale fp16 bits [B][Hkv][n]).
    """
    B, n, H, d = v.shape
    assert n % WINDOW == 0
    sigma16 = f16_bits(value_scale_f32(v))                      # [B][n][H]
    sig = f16_to_f32(sigma16)
    vr = np.empty_like(v, dtype=F32)
    for m in range(U.shape[0]):
        sel = tags == m
        if sel.any():
            vr[sel] = rotate_values_f32(v[sel], U[m])
    beta = value_boundaries_f32(levels16)
    codes = np.zeros(v.shape, dtype=np.uint8)
    for j in range(beta.shape[0]):
        theta = sig * beta[j]
        codes += (vr >= theta[..., None]).astype(np.uint8)
    codes = codes.transpose(0, 2, 1, 3).reshape(B, H, n // WINDOW, WINDOW, d)
    return pack_windows(codes, "value", bits), sigma16.transpose(0, 2, 1).copy()


# ----------------------------------------------------------------------------- dequantization
def dequantize_keys(k_codes, k_min, k_scale, signs, bits: int, length: Optional[int] = None):
    """Original-space keys x_hat = R^{-1}(m + s * code), float64 [B][Hkv][T][d].

    k_min, k_scale: fp16 bits (uint16 [B][Hkv][nw][d]) or MXFP4 records (uint8
    [B][Hkv][nw][mx_record_bytes(d)]), told apart by their dtype.
    """
    B, H, nw, _ = k_codes.shape
    d = np.asarray(signs).shape[-1]
    codes = unpack_windows(k_codes, "key", d, bits).astype(np.float64)   # [B][H][nw][32][d]
    if np.asarray(k_min).dtype == np.uint8:
        m, s = mx_record_values(k_min, d), mx_record_values(k_scale, d)
    else:
        m, s = f16_to_f64(k_min), f16_to_f64(k_scale)
    yhat = m[:, :, :, None, :] + s[:, :, :, None, :] * codes
    yhat = yhat.reshape(B, H, nw * WINDOW, d)
    if length is not None:
        yhat = yhat[:, :, :length]
    return inverse_key_rotation_f64(yhat, signs)


def dequantize_values(v_codes, v_scale, tags, U, levels16, bits: int, length: Optional[int] = None):
    """Original-space values v_hat = U_m (sigma * l[code]), float64 [B][Hkv][T][d]."""
    B, H, nw, _ = v_codes.shape
    d = U.shape[-1]
    T = nw * WINDOW if length is None else length
    codes = unpack_windows(v_codes, "value", d, bits).reshape(B, H, nw * WINDOW, d)[:, :, :T]
    lv = f16_to_f64(levels16)
    vprime = f16_to_f64(v_scale)[:, :, :T, None] * lv[codes]
    out = np.empty_like(vprime)
    for m in range(U.shape[0]):
        for b in range(B):
            sel = tags[b, :T] == m
            if sel.any():
                out[b][:, sel] = vprime[b][:, sel] @ np.asarray(U[m], np.float64).T
    return out


# ----------------------------------------------------------------------------- attention
def attention_f64(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q . k_t) . v_t for one query head; zeros when there is no token."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1])
    s = scale * (keys @ np.asarray(q, np.float64))
    p = np.exp(s - s.max())
    return (p @ values) / p.sum()


def decode_attention(q, seq_lens, cache: dict, signs, U, levels16, scale: Optional[float] = None,
                     rows: Optional[Sequence] = None):
    """Decode attention over the dequantized packed cache, float64.

    q: fp32 [B][Hq][d]; seq_lens: [B]; cache: dict with k_codes, k_min, k_scale,
    v_codes, v_scale, modality, key_bits, value_bits.  Query head h reads KV
    head h // (Hq/Hkv).  rows: optional list of (b, h) to compute (others 0).
    """
    B, Hq, d = q.shape
    Hkv = cache["k_min"].shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if not scale else float(scale)
    out = np.zeros((B, Hq, d))
    want = [(b, h) for b in range(B) for h in range(Hq)] if rows is None else list(rows)
    by_kv = {}
    for b, h in want:
        by_kv.setdefault((b, h // G), []).append(h)
    for (b, kv), heads in sorted(by_kv.items()):
        n = int(seq_lens[b])
        nw = (n + WINDOW - 1) // WINDOW
        sl = lambda a: a[b:b + 1, kv:kv + 1, :nw]
        keys = dequantize_keys(sl(cache["k_codes"]), sl(cache["k_min"]), sl(cache["k_scale"]),
                               signs, cache["key_bits"], length=n)[0, 0]
        vals = dequantize_values(sl(cache["v_codes"]), cache["v_scale"][b:b + 1, kv:kv + 1, :nw * WINDOW],
                                 cache["modality"][b:b + 1], U, levels16, cache["value_bits"],
                                 length=n)[0, 0]
        for h in heads:
            out[b, h] = attention_f64(q[b, h], keys, vals, scale)
    return out


# ----------------------------------------------------------------------------- streaming
def stream_packed_lengths(n: int):
    """(key_packed, value_packed): how many leading tokens of an n-token stream have
    quantized keys and values ([paper] §3.1 Implementation details, captioning).

    Keys are quantized every 128 tokens, as four 32-token groups: the first
    128 * floor(n / 128) tokens.  Values stay in a sliding FP16 window of the 128
    most recent tokens and are quantized once they leave it; with values packed
    in 32-token windows, a window is quantized when its last token has left, so
    32 * floor(max(0, n - 128) / 32) tokens (reading: the pages do not say how the
    sliding window meets the 32-token grouping).
    """
    n = int(n)
    return (n // 128) * 128, (max(0, n - 128) // WINDOW) * WINDOW


def decode_attention_streaming(q, seq_lens, cache: dict, k_recent, v_recent, signs, U, levels16,
                               scale: Optional[float] = None, rows: Optional[Sequence] = None):
    """Decode attention over a streamed cache, float64.

    Token t of sequence b attends with the dequantized packed key when
    t < key_packed and with k_recent[b, t, kv] (the stored key, as given)
    otherwise; values likewise with value_packed; (key_packed, value_packed) =
    stream_packed_lengths(seq_lens[b]).  k_recent, v_recent: [B][T][Hkv][d]
    indexed by absolute token position (only the unquantized tokens are read).
    """
    B, Hq, d = q.shape
    Hkv = cache["k_min"].shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if not scale else float(scale)
    out = np.zeros((B, Hq, d))
    want = [(b, h) for b in range(B) for h in range(Hq)] if rows is None else list(rows)
    by_kv = {}
    for b, h in want:
        by_kv.setdefault((b, h // G), []).append(h)
    for (b, kv), heads in sorted(by_kv.items()):
        n = int(seq_lens[b])
        kp, vp = stream_packed_lengths(n)
        keys = np.asarray(k_recent[b, :n, kv], np.float64).copy()
        vals = np.asarray(v_recent[b, :n, kv], np.float64).copy()
        if kp > 0:
            nw = kp // WINDOW
            sl = lambda a: a[b:b + 1, kv:kv + 1, :nw]
            keys[:kp] = dequantize_keys(sl(cache["k_codes"]), sl(cache["k_min"]), sl(cache["k_scale"]),
                                        signs, cache["key_bits"], length=kp)[0, 0]
        if vp > 0:
            nw = vp // WINDOW
            vals[:vp] = dequantize_values(cache["v_codes"][b:b + 1, kv:kv + 1, :nw],
                                          cache["v_scale"][b:b + 1, kv:kv + 1, :vp],
                                          cache["modality"][b:b + 1], U, levels16, cache["value_bits"],
                                          length=vp)[0, 0]
        for h in heads:
            out[b, h] = attention_f64(q[b, h], keys, vals, scale)
    return out


# ----------------------------------------------------------------------------- error metrics
# [paper] §3.3 "Error comparison" (Table 3 caption) compares the codecs by the key
# reconstruction MSE, the KL divergence between the attention distributions computed
# with original and with quantized keys, and the MSE of the attention output; the
# digest's key-results list gives the Table 3 values ([digest] 关键结果与论文证据).
# The pages print no formulas: the readings below are the plain definitions.
def key_reconstruction_mse(keys, keys_hat) -> float:
    """Mean over every element of (k_hat - k)^2 (float64)."""
    k = np.asarray(keys, np.float64)
    return float(np.mean((np.asarray(keys_hat, np.float64) - k) ** 2))


def _log_softmax(s):
    s = s - s.max(axis=-1, keepdims=True)
    return s - np.log(np.exp(s).sum(axis=-1, keepdims=True))


def attention_kl(q, keys, keys_hat, scale: float) -> float:
    """Mean over query rows of KL(p || p_hat), p = softmax(scale q . k_t) over the tokens t with
    the original keys and p_hat with the quantized keys.  q: [H][d]; keys: [T][d] (float64)."""
    q = np.asarray(q, np.float64)
    lp = _log_softmax(scale * (q @ np.asarray(keys, np.float64).T))
    lph = _log_softmax(scale * (q @ np.asarray(keys_hat, np.float64).T))
    return float(np.mean(np.sum(np.exp(lp) * (lp - lph), axis=-1)))


def attention_output_mse(q, keys, values, keys_hat, values_hat, scale: float) -> float:
    """Mean over every element of (o_hat - o)^2, o = softmax(scale q . k) v with the original
    keys and values, o_hat with the quantized ones.  q: [H][d]; keys, values: [T][d]."""
    q = np.asarray(q, np.float64)
    o = np.exp(_log_softmax(scale * (q @ np.asarray(keys, np.float64).T))) @ np.asarray(values, np.float64)
    oh = np.exp(_log_softmax(scale * (q @ np.asarray(keys_hat, np.float64).T))) @ np.asarray(values_hat, np.float64)
    return float(np.mean((oh - o) ** 2))


# ----------------------------------------------------------------------------- calibration
def calibrate_value_rotation(values: np.ndarray, weights: Optional[np.ndarray] = None) -> np.ndarray:
    """U_m for one modality from its calibration values, float64 [d][d].

    C = sum_t w_t v_t v_t^T / sum_t w_t (w_t = 1 when no weights are given; the pages
    weight by attention contribution); E = eigenvectors of C as columns, eigenvalues
    descending, each column's largest-magnitude entry (the first such) made positive;
    U = E H_d / sqrt(d).  Then v' = U^T v decorrelates v and spreads the result over
    the channels like the Hadamard rotation.
    """
    v = np.asarray(values, np.float64)
    n, d = v.shape
    w = np.ones(n) if weights is None else np.asarray(weights, np.float64)
    C = (v * w[:, None]).T @ v / w.sum()
    lam, E = np.linalg.eigh(C)
    E = E[:, np.argsort(-lam, kind="stable")]
    lead = np.argmax(np.abs(E), axis=0)
    E = E * np.sign(E[lead, np.arange(d)])[None, :]
    return E @ sylvester(d) / math.sqrt(d)


def value_codec_mse(v: np.ndarray, U: np.ndarray, bits: int = 2) -> float:
    """Mean squared error of the value codec (rotation U, per-token scale, fixed
    codebook) on values v [n][d], relative to the mean squared value."""
    v = np.asarray(v, F32)
    n, d = v.shape
    Us = np.asarray(U, F32)[None]
    tags = np.zeros((1, n), np.uint8)
    lv = value_codebook_f16(bits)
    vc, vs = quantize_values(v[None, :, None, :], tags, Us, lv, bits)
    vh = dequantize_values(vc, vs, tags, Us, lv, bits)[0, 0]
    return float(np.mean((vh - v) ** 2) / np.mean(np.asarray(v, np.float64) ** 2))
