"""Host-only checks of the C ABI: the library loads, exports what include/omnikv.h
declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from decode_attention_fwht_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "omnikv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libomnikv.so not built (run __graft_entry__.build())")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(omnikv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_operations():
    syms = declared_symbols()
    for s in ("omnikv_quantize_keys", "omnikv_quantize_values", "omnikv_decode_attention"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    L = binding.load()
    for s in declared_symbols():
        assert hasattr(L, s), s
    assert set(declared_symbols()) == set(binding.EXPORTED)


def _cfg(**kw):
    base = dict(head_dim=128, num_q_heads=16, num_kv_heads=2, key_bits=2, value_bits=2, window=32,
                num_modalities=3, key_meta=binding.META_FP16)
    base.update(kw)
    return binding._Config(*[base[f] for f, _ in binding._Config._fields_])


def _create(cfg, signs=None, rots=None, codebook=None):
    L = binding.load()
    d = cfg.head_dim if cfg.head_dim in (64, 128) else 128
    signs = np.ones(d, np.int8) if signs is None else signs
    rots = np.stack([np.eye(d, dtype=np.float32)] * 3) if rots is None else rots
    h = ctypes.c_void_p()
    cb = None if codebook is None else codebook.ctypes.data
    st = L.omnikv_create(ctypes.byref(cfg), signs.ctypes.data, rots.ctypes.data, cb, ctypes.byref(h))
    return st, h, L.omnikv_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(head_dim=96), binding.EUNSUPPORTED, "head_dim"),
    (dict(key_bits=3), binding.EUNSUPPORTED, "bits"),
    (dict(value_bits=1), binding.EUNSUPPORTED, "bits"),
    (dict(window=16), binding.EUNSUPPORTED, "window"),
    (dict(num_q_heads=15), binding.EINVAL, "multiple"),
    (dict(num_q_heads=32, num_kv_heads=2), binding.EUNSUPPORTED, "8 query heads"),
    (dict(num_modalities=4), binding.EINVAL, "num_modalities"),
    (dict(num_kv_heads=0), binding.EINVAL, "num_kv_heads"),
    (dict(key_meta=2), binding.EINVAL, "key_meta"),
])
def test_create_rejects_bad_config(kw, status, needle):
    st, h, msg = _create(_cfg(**kw))
    assert st == status and needle in msg and not h.value


def test_create_rejects_bad_signs_and_rotations():
    signs = np.ones(128, np.int8)
    signs[5] = 0
    st, h, msg = _create(_cfg(), signs=signs)
    assert st == binding.EINVAL and "key_signs[5]" in msg
    rots = np.stack([np.eye(128, dtype=np.float32)] * 3)
    rots[1, 0, 0] = 1.5
    st, h, msg = _create(_cfg(), rots=rots)
    assert st == binding.EINVAL and "value_rotations[1]" in msg and "orthogonal" in msg


def test_create_rejects_unsorted_codebook():
    cb = np.array([0x3C00, 0x3800, 0x4000, 0x4200], np.uint16)   # 1.0, 0.5, 2, 3
    st, h, msg = _create(_cfg(), codebook=cb)
    assert st == binding.EINVAL and "ascending" in msg


def test_null_context_and_null_out():
    L = binding.load()
    assert L.omnikv_quantize_keys(None, None, 0, 1, 0, 32, 32, None, None, None, None) == binding.EINVAL
    assert "NULL" in L.omnikv_last_error().decode()
    assert L.omnikv_decode_attention(None, *([None] * 2), 1, 0, *([None] * 6), 32, 0.0, 0, None, 0, None,
                                     None) == binding.EINVAL
    sz = ctypes.c_size_t()
    assert L.omnikv_decode_workspace_size(None, 1, 32, 0, ctypes.byref(sz)) == binding.EINVAL
    assert L.omnikv_create(None, None, None, None, None) == binding.EINVAL
    assert L.omnikv_destroy(None) == binding.OK
    assert L.omnikv_key_meta_bytes(None, ctypes.byref(sz)) == binding.EINVAL


def test_stream_schedule_host_function_matches_the_oracle():
    """omnikv_stream_packed_lengths (host arithmetic) against the oracle's schedule."""
    from oracle import omnikv_oracle as O
    for n in range(0, 2000, 7):
        assert binding.Context.stream_packed_lengths(n) == O.stream_packed_lengths(n), n
    L = binding.load()
    kp, vp = ctypes.c_int64(), ctypes.c_int64()
    assert L.omnikv_stream_packed_lengths(-1, ctypes.byref(kp), ctypes.byref(vp)) == binding.EINVAL


def test_streaming_calls_reject_a_null_context():
    L = binding.load()
    z = None
    st = L.omnikv_stream_append(z, z, z, binding.BF16, z, z, z, 1, z, z, 256, z, z, z, z, z, z, 32, z)
    assert st == binding.EINVAL
    st = L.omnikv_decode_attention_streaming(z, z, z, 1, 32, z, z, z, z, z, z, 32, z, z, binding.BF16, 256,
                                             0.0, 0, z, 0, z, z)
    assert st == binding.EINVAL


def test_calibration_rejects_bad_arguments():
    L = binding.load()
    out = np.zeros((128, 128), np.float32)
    assert L.omnikv_calibrate_value_rotation(None, binding.F32, None, 16, 96, out.ctypes.data, None) == binding.EUNSUPPORTED
    assert L.omnikv_calibrate_value_rotation(None, binding.F32, None, 0, 128, out.ctypes.data, None) == binding.EINVAL
    assert L.omnikv_calibrate_value_rotation(None, binding.F32, None, 16, 128, out.ctypes.data, None) == binding.EINVAL
    assert L.omnikv_calibrate_value_rotation(None, 7, None, 16, 128, out.ctypes.data, None) == binding.EINVAL
