"""Shared plumbing of the GPU tests: device copies, contexts, error measures."""
import sys

import numpy as np

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import binding, synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint32:
        x = x.view(np.int32)
    elif x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def from_dev(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def bf16_tensor(x):
    """fp32 numpy holding bf16-exact values -> torch bf16 on the GPU."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


_CODEBOOKS = {}


def oracle_codebook(bits):
    """The oracle's own value codebook (fp16 bits), computed once per width.  Every parity
    reference dequantizes with this table, never with the one the library builds."""
    if bits not in _CODEBOOKS:
        _CODEBOOKS[bits] = O.value_codebook_f16(bits)
    return _CODEBOOKS[bits].copy()


def make_context(cfg, key_bits=None, value_bits=None, seed=0, key_meta="fp16", modalities=3):
    """A context with the configuration's seeded signs and rotations (the first `modalities`
    of them) and the library's built-in codebook.  Returns (ctx, signs, U, levels) with
    `levels` the oracle's codebook, which the references use."""
    d = cfg.head_dim
    signs = synth.rademacher_signs(d, seed)
    U = synth.value_rotations(d, seed, modalities)
    kb = cfg.key_bits if key_bits is None else key_bits
    vb = cfg.value_bits if value_bits is None else value_bits
    ctx = binding.Context(d, cfg.q_heads, cfg.kv_heads, kb, vb, signs, U, key_meta=key_meta)
    return ctx, signs, U, oracle_codebook(vb)


def cache_to_device(cache):
    out = {k: to_dev(cache[k]) for k in ("k_codes", "k_min", "k_scale", "v_codes", "v_scale", "modality")}
    out["t_cap"] = int(cache.get("t_cap", cache["v_scale"].shape[-1]))
    return out


def row_errors(got, ref):
    """Per (b, h) row: max_c |got - ref| / max_c |ref| (rows with a zero reference use 1)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den > 0, den, 1.0)
    return np.max(np.abs(got - ref), axis=-1) / den


def sampled_unit_rows(cfg, seed, units=3):
    """(b, h) rows of every query head of a few sampled (sequence, KV head) units, always
    including the first and the last unit.  The oracle's cost is per unit, so checking
    all G heads of a unit costs little more than one."""
    rng = np.random.default_rng(seed)
    picks = {(0, 0), (cfg.batch - 1, cfg.kv_heads - 1)}
    picks |= {(int(rng.integers(cfg.batch)), int(rng.integers(cfg.kv_heads))) for _ in range(units)}
    return sorted((b, kv * cfg.group + j) for b, kv in picks for j in range(cfg.group))
