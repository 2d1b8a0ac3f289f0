"""The pages' error metrics and the temporal-contiguity property, on the CPU oracle.

[paper] §3.3 "Error comparison" (Table 3 caption) compares codecs by the key
reconstruction MSE, the KL divergence between attention distributions with original
and quantized keys, and the attention-output MSE; [paper] §3.3 "Key adaptation"
(Table 6 caption) finds that window ranges need the stream's temporal contiguity:
shuffling tokens globally hurts most, shuffling within each modality partly, and the
contiguous order is best.  The metric functions are pinned here by closed forms and
invariances; the property by the oracle's codec on synthetic drift data whose keys
cluster by modality.  The pages' numbers themselves need real models and data: parity
unpinned.
"""
import math

import numpy as np
import pytest

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import synth


def _drift(cid, seed, T, offset=0.0, heads=1):
    cfg = synth.Config(**{**synth.CONFIGS[cid].__dict__, "batch": 1, "kv_heads": heads, "fp32_inputs": True})
    tags = synth.modality_layout(cfg, seed, T)
    k = synth.drifting_tensor(cfg, tags, seed, 0, 0, T, modality_offset=offset)
    v = synth.drifting_tensor(cfg, tags, seed, 1, 0, T, modality_offset=offset)
    return cfg, tags, k, v


def test_metrics_vanish_on_identical_caches():
    rng = np.random.default_rng(0)
    k, v, q = rng.standard_normal((50, 16)), rng.standard_normal((50, 16)), rng.standard_normal((3, 16))
    assert O.key_reconstruction_mse(k, k) == 0.0
    assert abs(O.attention_kl(q, k, k, 0.25)) < 1e-15
    assert O.attention_output_mse(q, k, v, k, v, 0.25) == 0.0


def test_key_mse_of_a_constant_offset():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((40, 8))
    for delta in (0.5, -0.125, 3.0):
        assert O.key_reconstruction_mse(k, k + delta) == pytest.approx(delta ** 2, rel=1e-12)


def test_attention_kl_ignores_a_shift_shared_by_every_key():
    """Adding the same vector to every key adds one constant to all scores of a query, which
    softmax removes: the distributions, and the KL, are unchanged."""
    rng = np.random.default_rng(2)
    k, q = rng.standard_normal((30, 8)), rng.standard_normal((4, 8))
    u = rng.standard_normal(8)
    assert abs(O.attention_kl(q, k, k + u, 0.7)) < 1e-12
    assert O.attention_kl(q, k, k + rng.standard_normal((30, 8)), 0.7) > 1e-3


def test_attention_kl_of_two_tokens_closed_form():
    """Two tokens with scores a, b; the quantized key raises token 0's score by d.  With
    p = 1/(1 + e^(b-a)) and p' = 1/(1 + e^(b-a-d)):
    KL(p || p') = p ln(p/p') + (1-p) ln((1-p)/(1-p'))  (direction: original over quantized)."""
    scale = 0.5
    q = np.array([[1.0, 0.0]])
    for a, b, d in ((0.3, -0.4, 0.8), (2.0, 1.0, -1.5), (-1.0, 0.5, 0.25)):
        k = np.array([[a / scale, 0.0], [b / scale, 0.0]])
        kh = np.array([[(a + d) / scale, 0.0], [b / scale, 0.0]])
        p = 1.0 / (1.0 + math.exp(b - a))
        ph = 1.0 / (1.0 + math.exp(b - a - d))
        ref = p * math.log(p / ph) + (1 - p) * math.log((1 - p) / (1 - ph))
        assert O.attention_kl(q, k, kh, scale) == pytest.approx(ref, rel=1e-12, abs=1e-15)


def test_attention_output_mse_closed_forms():
    """Original keys and every value shifted by delta: the softmax weights sum to one, so the
    output moves by delta and its MSE is delta^2.  A single token: the output is its value,
    whatever the keys, so the MSE is the values' MSE."""
    rng = np.random.default_rng(3)
    k, v, q = rng.standard_normal((20, 8)), rng.standard_normal((20, 8)), rng.standard_normal((5, 8))
    for delta in (0.25, -2.0):
        assert O.attention_output_mse(q, k, v, k, v + delta, 0.35) == pytest.approx(delta ** 2, rel=1e-10)
    k1, v1 = k[:1], v[:1]
    kh, vh = rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert O.attention_output_mse(q, k1, v1, kh, vh, 0.35) == pytest.approx(np.mean((vh - v1) ** 2), rel=1e-12)


def test_attention_output_mse_of_two_tokens_closed_form():
    """Two tokens, exact values, the quantized key raising token 0's score by d: the output
    moves from p v0 + (1-p) v1 to p' v0 + (1-p') v1, so its MSE is (p' - p)^2 mean((v0 - v1)^2)."""
    scale = 0.5
    q = np.array([[1.0, 0.0]])
    rng = np.random.default_rng(4)
    v = rng.standard_normal((2, 6))
    for a, b, d in ((0.3, -0.4, 0.8), (2.0, 1.0, -1.5)):
        k = np.array([[a / scale, 0.0], [b / scale, 0.0]])
        kh = np.array([[(a + d) / scale, 0.0], [b / scale, 0.0]])
        p = 1.0 / (1.0 + math.exp(b - a))
        ph = 1.0 / (1.0 + math.exp(b - a - d))
        ref = (ph - p) ** 2 * float(np.mean((v[0] - v[1]) ** 2))
        assert O.attention_output_mse(q, k, v, kh, v, scale) == pytest.approx(ref, rel=1e-10)


@pytest.mark.parametrize("cid", [2, 4])
def test_error_metrics_fall_from_two_to_four_bits(cid):
    """[paper] §3.3 Ablation studies (Table 5 caption): more bits, less error - for all three
    metrics, with the oracle's codec on drift data."""
    cfg, tags, k, v = _drift(cid, 5, 2048)
    signs = synth.rademacher_signs(128, 5)
    U = synth.value_rotations(128, 5)
    q = synth.queries(cfg, 5)[0, :cfg.group]
    scale = 1.0 / math.sqrt(128)
    res = {}
    for bits in (2, 4):
        lv = O.value_codebook_f16(bits)
        kc, km, ks = O.quantize_keys(k, signs, bits)
        vc, vs = O.quantize_values(v, tags, U, lv, bits)
        kh = O.dequantize_keys(kc, km, ks, signs, bits)[0, 0]
        vh = O.dequantize_values(vc, vs, tags, U, lv, bits)[0, 0]
        kk, vv = k[0, :, 0].astype(np.float64), v[0, :, 0].astype(np.float64)
        res[bits] = (O.key_reconstruction_mse(kk, kh), O.attention_kl(q, kk, kh, scale),
                     O.attention_output_mse(q, kk, vv, kh, vh, scale))
    assert all(b < a for a, b in zip(res[2], res[4])), res


@pytest.mark.parametrize("cid,seed", [(2, 0), (2, 1), (4, 2), (4, 3)])
def test_window_ranges_need_temporal_contiguity(cid, seed):
    """[paper] §3.3 Key adaptation (Table 6): the key reconstruction error of the window
    min-max codec is lowest on the stream in order, higher with the tokens shuffled within
    each modality, highest shuffled globally.  Drift data whose keys cluster by modality
    (a per-modality channel offset of 3 standard deviations); relative MSE, 5% margins."""
    T = 4096
    cfg, tags, k, _ = _drift(cid, seed, T, offset=3.0)
    signs = synth.rademacher_signs(128, seed)

    def rel(kk):
        kc, km, ks = O.quantize_keys(kk, signs, 2)
        kh = O.dequantize_keys(kc, km, ks, signs, 2)[0, 0]
        x = kk[0, :, 0].astype(np.float64)
        return O.key_reconstruction_mse(x, kh) / float(np.mean(x ** 2))

    rng = np.random.default_rng(100 + seed)
    within = np.arange(T)
    for m in range(3):
        idx = np.where(tags[0] == m)[0]
        within[idx] = rng.permutation(idx)
    contiguous, by_modality, shuffled = rel(k), rel(k[:, within]), rel(k[:, rng.permutation(T)])
    assert contiguous * 1.05 < by_modality and by_modality * 1.05 < shuffled, (contiguous, by_modality, shuffled)
