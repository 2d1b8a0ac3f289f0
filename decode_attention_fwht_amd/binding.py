"""Thin ctypes binding of libomnikv (include/omnikv.h).

Argument marshalling only: tensors are passed as device pointers, the current
torch stream as the HIP stream; every step of the hot path runs in the HIP
kernels behind the C ABI.  If the library is not built this module raises; it
never falls back to a CPU implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libomnikv.so")

OK, EINVAL, EUNSUPPORTED, EHIP, ENOMEM = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
META_FP16, META_MXFP4 = 0, 1

EXPORTED = (
    "omnikv_create", "omnikv_destroy", "omnikv_value_codebook", "omnikv_quantize_keys",
    "omnikv_quantize_values", "omnikv_decode_workspace_size", "omnikv_decode_attention",
    "omnikv_decode_partial", "omnikv_decode_combine", "omnikv_stream_packed_lengths", "omnikv_stream_append",
    "omnikv_decode_attention_streaming", "omnikv_calibrate_value_rotation", "omnikv_key_meta_bytes",
    "omnikv_decode_attention_noalloc", "omnikv_last_error",
)


def calibrate_value_rotation(values, weights=None, stream=None) -> np.ndarray:
    """U_m (fp32 numpy [d][d]) from one modality's calibration values: a contiguous device
    tensor [n][d] (fp32 or bf16) and optional fp32 weights [n]."""
    import torch
    if values.dtype not in (torch.float32, torch.bfloat16) or not values.is_contiguous() or values.dim() != 2:
        raise ValueError("values must be a contiguous fp32 or bf16 tensor [n][d]")
    if weights is not None and (weights.dtype != torch.float32 or not weights.is_contiguous()):
        raise ValueError("weights must be a contiguous fp32 tensor [n]")
    n, d = int(values.shape[0]), int(values.shape[1])
    out = np.zeros((d, d), np.float32)
    dt = BF16 if values.dtype == torch.bfloat16 else F32
    _check(load().omnikv_calibrate_value_rotation(_ptr(values), dt, _ptr(weights), n, d, out.ctypes.data,
                                                  _stream(stream)))
    return out


class OmniKVError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"omnikv status {status}: {msg}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "head_dim", "num_q_heads", "num_kv_heads", "key_bits", "value_bits", "window", "num_modalities",
        "key_meta")]


_lib = None


def load() -> ctypes.CDLL:
    """Load libomnikv.so (built in the package directory) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    # torch first: its HIP runtime then provides the library's libamdhip64.so.7 too (same
    # soname), so device memory, streams and graphs all belong to one runtime.  Loaded the
    # other way round, torch would bind to the system runtime and find no GPU.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.omnikv_create.argtypes = [ctypes.POINTER(_Config), vp, vp, vp, ctypes.POINTER(vp)]
    L.omnikv_destroy.argtypes = [vp]
    L.omnikv_value_codebook.argtypes = [vp, vp]
    L.omnikv_key_meta_bytes.argtypes = [vp, ctypes.POINTER(sz)]
    L.omnikv_quantize_keys.argtypes = [vp, vp, ctypes.c_int, i32, i64, i64, i64, vp, vp, vp, vp]
    L.omnikv_quantize_values.argtypes = [vp, vp, ctypes.c_int, vp, i32, i64, i64, i64, vp, vp, vp]
    L.omnikv_decode_workspace_size.argtypes = [vp, i32, i64, i32, ctypes.POINTER(sz)]
    L.omnikv_decode_attention.argtypes = [vp, vp, vp, i32, i64, vp, vp, vp, vp, vp, vp, i64,
                                          ctypes.c_float, i32, vp, sz, vp, vp]
    L.omnikv_decode_partial.argtypes = [vp, vp, vp, i32, i64, vp, vp, vp, vp, vp, vp, i64,
                                        ctypes.c_float, i32, vp, sz, vp]
    L.omnikv_decode_attention_noalloc.argtypes = [vp, vp, vp, i32, i64, vp, vp, vp, vp, vp, vp, i64,
                                                  ctypes.c_float, i32, vp, vp]
    L.omnikv_decode_combine.argtypes = [vp, vp, i32, i64, i32, vp, sz, vp, vp]
    L.omnikv_stream_packed_lengths.argtypes = [i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.omnikv_stream_append.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, i32, vp, vp, i32,
                                       vp, vp, vp, vp, vp, vp, i64, vp]
    L.omnikv_calibrate_value_rotation.argtypes = [vp, ctypes.c_int, vp, i64, i32, vp, vp]
    L.omnikv_decode_attention_streaming.argtypes = [vp, vp, vp, i32, i64, vp, vp, vp, vp, vp, vp, i64,
                                                    vp, vp, ctypes.c_int, i32, ctypes.c_float, i32, vp, sz,
                                                    vp, vp]
    for name in EXPORTED:
        if name == "omnikv_last_error":
            continue
        getattr(L, name).restype = ctypes.c_int
    L.omnikv_last_error.restype = ctypes.c_char_p
    L.omnikv_last_error.argtypes = []
    _lib = L
    return L


def _check(status: int):
    if status != OK:
        raise OmniKVError(status, load().omnikv_last_error().decode())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


class Context:
    """An omnikv_ctx: attention shape, codec widths and the immutable tables."""

    def __init__(self, head_dim: int, num_q_heads: int, num_kv_heads: int, key_bits: int = 2,
                 value_bits: int = 2, key_signs=None, value_rotations=None, value_codebook=None,
                 num_modalities: Optional[int] = None, key_meta: str = "fp16"):
        L = load()
        signs = np.ascontiguousarray(key_signs, dtype=np.int8)
        rots = np.ascontiguousarray(value_rotations, dtype=np.float32)
        M = rots.shape[0] if num_modalities is None else num_modalities
        meta = {"fp16": META_FP16, "mxfp4": META_MXFP4}.get(key_meta, -1)
        cfg = _Config(head_dim, num_q_heads, num_kv_heads, key_bits, value_bits, 32, M, meta)
        cb = None if value_codebook is None else np.ascontiguousarray(value_codebook, dtype=np.uint16)
        h = ctypes.c_void_p()
        _check(L.omnikv_create(ctypes.byref(cfg), signs.ctypes.data, rots.ctypes.data,
                               None if cb is None else cb.ctypes.data, ctypes.byref(h)))
        self._h = h
        self.head_dim, self.num_q_heads, self.num_kv_heads = head_dim, num_q_heads, num_kv_heads
        self.key_bits, self.value_bits, self.num_modalities = key_bits, value_bits, M
        self.key_meta = key_meta
        nb = ctypes.c_size_t()
        _check(L.omnikv_key_meta_bytes(h, ctypes.byref(nb)))
        self.key_meta_bytes = nb.value   # per (sequence, KV head, window), each of k_min, k_scale

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            load().omnikv_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self) -> int:
        return self._h.value

    def value_codebook(self) -> np.ndarray:
        out = np.zeros(1 << self.value_bits, dtype=np.uint16)
        _check(load().omnikv_value_codebook(self._h, out.ctypes.data))
        return out

    # -- allocation helpers (device memory via torch; plain storage, no compute)
    def alloc_cache(self, batch: int, t_cap: int, device="cuda"):
        import torch
        d, H, nw = self.head_dim, self.num_kv_heads, t_cap // 32
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        # key metadata: fp16 bit patterns [B][H][nw][d], or MXFP4 byte records [B][H][nw][R]
        meta = ((batch, H, nw, d), torch.int16) if self.key_meta == "fp16" else \
            ((batch, H, nw, self.key_meta_bytes), torch.uint8)
        return dict(
            k_codes=z((batch, H, nw, d * self.key_bits), torch.int32),
            k_min=z(*meta),
            k_scale=z(*meta),
            v_codes=z((batch, H, nw, d * self.value_bits), torch.int32),
            v_scale=z((batch, H, t_cap), torch.int16),
            modality=z((batch, t_cap), torch.uint8),
            t_cap=t_cap,
        )

    # -- the three operations
    def quantize_keys(self, k, t0: int, cache: dict, stream=None):
        import torch
        dt = BF16 if k.dtype == torch.bfloat16 else F32
        if k.dtype not in (torch.bfloat16, torch.float32) or not k.is_contiguous():
            raise ValueError("k must be a contiguous fp32 or bf16 tensor [B][n][Hkv][d]")
        B, n = int(k.shape[0]), int(k.shape[1])
        _check(load().omnikv_quantize_keys(self._h, _ptr(k), dt, B, t0, n, cache["t_cap"],
                                           _ptr(cache["k_codes"]), _ptr(cache["k_min"]),
                                           _ptr(cache["k_scale"]), _stream(stream)))

    def quantize_values(self, v, t0: int, cache: dict, stream=None):
        import torch
        dt = BF16 if v.dtype == torch.bfloat16 else F32
        if v.dtype not in (torch.bfloat16, torch.float32) or not v.is_contiguous():
            raise ValueError("v must be a contiguous fp32 or bf16 tensor [B][n][Hkv][d]")
        B, n = int(v.shape[0]), int(v.shape[1])
        _check(load().omnikv_quantize_values(self._h, _ptr(v), dt, _ptr(cache["modality"]), B, t0, n,
                                             cache["t_cap"], _ptr(cache["v_codes"]), _ptr(cache["v_scale"]),
                                             _stream(stream)))

    def workspace_size(self, batch: int, max_len: int, num_splits: int = 0) -> int:
        out = ctypes.c_size_t()
        _check(load().omnikv_decode_workspace_size(self._h, batch, max_len, num_splits, ctypes.byref(out)))
        return out.value

    def decode(self, q, seq_lens, max_len: int, cache: dict, out=None, workspace=None,
               softmax_scale: float = 0.0, num_splits: int = 0, stream=None):
        import torch
        B = int(q.shape[0])
        if out is None:
            out = torch.empty((B, self.num_q_heads, self.head_dim), dtype=torch.float32, device=q.device)
        need = self.workspace_size(B, max_len, num_splits)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        _check(load().omnikv_decode_attention(
            self._h, _ptr(q), _ptr(seq_lens), B, max_len, _ptr(cache["k_codes"]), _ptr(cache["k_min"]),
            _ptr(cache["k_scale"]), _ptr(cache["v_codes"]), _ptr(cache["v_scale"]), _ptr(cache["modality"]),
            cache["t_cap"], softmax_scale, num_splits, _ptr(workspace), workspace.numel(), _ptr(out),
            _stream(stream)))
        return out

    def decode_noalloc(self, q, seq_lens, max_len: int, cache: dict, out, softmax_scale: float = 0.0,
                       num_splits: int = 0, stream=None):
        """omnikv_decode_attention_noalloc: the library's static scratch as the workspace; the
        caller passes the output."""
        _check(load().omnikv_decode_attention_noalloc(
            self._h, _ptr(q), _ptr(seq_lens), int(q.shape[0]), max_len, _ptr(cache["k_codes"]),
            _ptr(cache["k_min"]), _ptr(cache["k_scale"]), _ptr(cache["v_codes"]), _ptr(cache["v_scale"]),
            _ptr(cache["modality"]), cache["t_cap"], softmax_scale, num_splits, _ptr(out), _stream(stream)))
        return out

    def decode_partial(self, q, seq_lens, max_len: int, cache: dict, workspace, softmax_scale: float = 0.0,
                       num_splits: int = 0, stream=None):
        _check(load().omnikv_decode_partial(
            self._h, _ptr(q), _ptr(seq_lens), int(q.shape[0]), max_len, _ptr(cache["k_codes"]),
            _ptr(cache["k_min"]), _ptr(cache["k_scale"]), _ptr(cache["v_codes"]), _ptr(cache["v_scale"]),
            _ptr(cache["modality"]), cache["t_cap"], softmax_scale, num_splits, _ptr(workspace),
            workspace.numel(), _stream(stream)))

    def decode_combine(self, seq_lens, batch: int, max_len: int, workspace, out, num_splits: int = 0,
                       stream=None):
        _check(load().omnikv_decode_combine(self._h, _ptr(seq_lens), batch, max_len, num_splits,
                                            _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
        return out

    # -- streaming generation
    def alloc_rings(self, batch: int, ring_cap: int = 256, dtype=None, device="cuda"):
        """Rings of recent keys and values [B][ring_cap][Hkv][d] (plain storage)."""
        import torch
        dtype = torch.bfloat16 if dtype is None else dtype
        shape = (batch, ring_cap, self.num_kv_heads, self.head_dim)
        return dict(k=torch.zeros(shape, dtype=dtype, device=device), v=torch.zeros(shape, dtype=dtype, device=device),
                    cap=ring_cap)

    @staticmethod
    def stream_packed_lengths(n: int):
        kp, vp = ctypes.c_int64(), ctypes.c_int64()
        _check(load().omnikv_stream_packed_lengths(n, ctypes.byref(kp), ctypes.byref(vp)))
        return kp.value, vp.value

    def stream_append(self, k_new, v_new, tags_new, lens, lens_host, cache: dict, rings: dict, stream=None):
        """One token per sequence: k_new, v_new [B][Hkv][d]; tags_new uint8 [B]; lens int32 [B]
        (device) and lens_host (host sequence of ints) are the lengths before the append."""
        import torch
        if k_new.dtype != rings["k"].dtype or v_new.dtype != rings["v"].dtype:
            raise ValueError("k_new / v_new must have the rings' dtype")
        dt = BF16 if k_new.dtype == torch.bfloat16 else F32
        B = int(k_new.shape[0])
        lh = (ctypes.c_int64 * B)(*[int(x) for x in lens_host])
        _check(load().omnikv_stream_append(
            self._h, _ptr(k_new), _ptr(v_new), dt, _ptr(tags_new), _ptr(lens), lh, B, _ptr(rings["k"]),
            _ptr(rings["v"]), rings["cap"], _ptr(cache["k_codes"]), _ptr(cache["k_min"]), _ptr(cache["k_scale"]),
            _ptr(cache["v_codes"]), _ptr(cache["v_scale"]), _ptr(cache["modality"]), cache["t_cap"],
            _stream(stream)))

    def decode_streaming(self, q, seq_lens, max_len: int, cache: dict, rings: dict, out=None, workspace=None,
                         softmax_scale: float = 0.0, num_splits: int = 0, stream=None):
        import torch
        B = int(q.shape[0])
        if out is None:
            out = torch.empty((B, self.num_q_heads, self.head_dim), dtype=torch.float32, device=q.device)
        need = self.workspace_size(B, max_len, num_splits)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        dt = BF16 if rings["k"].dtype == torch.bfloat16 else F32
        _check(load().omnikv_decode_attention_streaming(
            self._h, _ptr(q), _ptr(seq_lens), B, max_len, _ptr(cache["k_codes"]), _ptr(cache["k_min"]),
            _ptr(cache["k_scale"]), _ptr(cache["v_codes"]), _ptr(cache["v_scale"]), _ptr(cache["modality"]),
            cache["t_cap"], _ptr(rings["k"]), _ptr(rings["v"]), dt, rings["cap"], softmax_scale, num_splits,
            _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
        return out
