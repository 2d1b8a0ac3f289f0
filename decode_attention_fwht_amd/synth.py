"""Seeded synthetic inputs shaped like the workloads of OmniKVQuant.

This module only draws random numbers and lays them out.  It holds none of the
codec's or the attention's arithmetic, so both the HIP path and the CPU oracle
may take their inputs from it.

The pages evaluate on audio-visual benchmarks and on Qwen2.5-Omni-3B /
Qwen3-Omni-30B-A3B ("OmniKVQuant: KV Cache Quantization for Omni-LLMs",
Sec. 3.1 Setup).  Neither the data nor the weights are available, so these
generators stand in for them with caches of the same shapes: a window-level
drift of the key/value statistics (the "temporal key drift" of Sec. 2.2), a
few large outlier channels (Sec. 1), and interleaved text/audio/video chunks
(modality ids 0 = text, 1 = audio, 2 = video).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

TEXT, AUDIO, VIDEO = 0, 1, 2
WINDOW = 32


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: attention shape, cache length and codec widths."""
    cid: int
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    context: int
    key_bits: int = 2
    value_bits: int = 2
    prefill: int = 0            # tokens per sequence quantized in one write-path call
    fp32_inputs: bool = False   # K/V handed over as fp32 (else bf16)
    layout: str = "interleaved"  # modality layout recipe
    drift_text: float = 0.2     # sigma of the LogNormal window scale, text windows
    drift_av: float = 0.5       # same for audio / video windows
    outliers: int = 4           # outlier channels per KV head
    outlier_gain: float = 10.0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


CONFIGS = {
    1: Config(1, "tiny", 1, 2, 1, 64, 256, prefill=256, fp32_inputs=True,
              layout="tiny", drift_text=0.3, drift_av=0.3, outliers=2, outlier_gain=8.0),
    2: Config(2, "qwen25omni3b-b1-10k", 1, 16, 2, 128, 10240, prefill=10240),
    3: Config(3, "qwen25omni3b-b16-32k", 16, 16, 2, 128, 32768, prefill=4096),
    4: Config(4, "qwen3omni30b-b8-64k", 8, 32, 4, 128, 65536, prefill=0, layout="random"),
    5: Config(5, "qwen3omni30b-b4-256k", 4, 32, 4, 128, 262144, prefill=65536, layout="random"),
}


def rng_for(cid: int, seed: int, stream: int) -> np.random.Generator:
    """Independent generator per (config, seed, purpose)."""
    return np.random.default_rng(np.random.SeedSequence([int(cid), int(seed), int(stream)]))


# --------------------------------------------------------------------------- layouts
def modality_layout(cfg: Config, seed: int = 0, length: Optional[int] = None) -> np.ndarray:
    """uint8 [batch][length] modality ids.

    tiny: text[0:32], audio[32:128], video[128:256] (then video).
    interleaved: 256 text tokens, then alternating audio chunks of 50 and video
        chunks of 250, the last chunk cut at the end; same for every sequence.
    random: chunk lengths drawn U{64..512}, modality drawn text/audio/video with
        probabilities 0.05 / 0.25 / 0.70, independently per sequence.
    """
    T = cfg.context if length is None else int(length)
    out = np.empty((cfg.batch, T), dtype=np.uint8)
    if cfg.layout == "tiny":
        row = np.full(T, VIDEO, dtype=np.uint8)
        row[:min(T, 32)] = TEXT
        row[32:min(T, 128)] = AUDIO
        out[:] = row
    elif cfg.layout == "interleaved":
        row = np.empty(T, dtype=np.uint8)
        pos = min(T, 256)
        row[:pos] = TEXT
        k = 0
        while pos < T:
            n, m = (50, AUDIO) if k % 2 == 0 else (250, VIDEO)
            row[pos:pos + n] = m
            pos += n
            k += 1
        out[:] = row
    elif cfg.layout == "random":
        rng = rng_for(cfg.cid, seed, 1)
        for b in range(cfg.batch):
            pos = 0
            while pos < T:
                n = int(rng.integers(64, 513))
                m = int(rng.choice(3, p=[0.05, 0.25, 0.70]))
                out[b, pos:pos + n] = m
                pos += n
    else:
        raise ValueError(cfg.layout)
    return out


# --------------------------------------------------------------------------- K / V
def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returned as fp32 values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def drifting_tensor(cfg: Config, tags: np.ndarray, seed: int, stream: int,
                         t0: int = 0, n: Optional[int] = None, modality_offset: float = 0.0) -> np.ndarray:
    """fp32 [batch][n][kv_heads][head_dim] keys or values with window drift.

    Per (sequence, KV head): z ~ N(0,1); for every 32-token window w a shift
    mu_w ~ N(0, 0.5^2) per channel and a scale lambda_w ~ LogNormal(0, s) with
    s = drift_text for a window that starts on a text token, else drift_av;
    x = lambda_w * (z + mu_w); a seeded set of outlier channels is multiplied
    by outlier_gain; bf16 configs round to bf16.  `stream` separates keys (0)
    from values (1); tokens [t0, t0+n) of the sequence are drawn.
    modality_offset > 0 adds a per-(KV head, modality) channel offset
    modality_offset * N(0, 1) to every token of that modality (keys that cluster by
    modality); 0 (the default) draws exactly as without it.
    """
    T = tags.shape[1]
    n = T - t0 if n is None else int(n)
    assert t0 % WINDOW == 0 and n % WINDOW == 0 and t0 + n <= T
    d, H, B = cfg.head_dim, cfg.kv_heads, cfg.batch
    nw = n // WINDOW
    out = np.empty((B, n, H, d), dtype=np.float32)
    for b in range(B):
        first = tags[b, t0:t0 + n:WINDOW]
        for h in range(H):
            r = rng_for(cfg.cid, seed, (stream * 7919 + b) * 131 + h + 17 * t0)
            outl = r.choice(d, size=cfg.outliers, replace=False)
            z = r.standard_normal((nw, WINDOW, d), dtype=np.float32)
            mu = 0.5 * r.standard_normal((nw, 1, d), dtype=np.float32)
            s = np.where(first == TEXT, cfg.drift_text, cfg.drift_av).astype(np.float32)
            lam = np.exp(s * r.standard_normal(nw, dtype=np.float32))[:, None, None]
            x = lam * (z + mu)
            x[:, :, outl] *= np.float32(cfg.outlier_gain)
            x = x.reshape(n, d)
            if modality_offset > 0:
                ro = rng_for(cfg.cid, seed, (stream * 7919 + b) * 131 + h + 100003)
                off = np.float32(modality_offset) * ro.standard_normal((3, d), dtype=np.float32)
                x = x + off[tags[b, t0:t0 + n].astype(np.int64)]
            out[b, :, h, :] = x
    if not cfg.fp32_inputs:
        out = to_bf16(out)
    return out


def queries(cfg: Config, seed: int = 0, batch: Optional[int] = None) -> np.ndarray:
    """fp32 [batch][q_heads][head_dim] ~ N(0, 1)."""
    B = cfg.batch if batch is None else batch
    return rng_for(cfg.cid, seed, 2).standard_normal(
        (B, cfg.q_heads, cfg.head_dim)).astype(np.float32)


def rademacher_signs(d: int, seed: int = 0) -> np.ndarray:
    """int8 [d] of +-1: the random sign diagonal of the randomized Hadamard rotation."""
    r = np.random.default_rng(np.random.SeedSequence([7, int(seed), d]))
    return np.where(r.integers(0, 2, d) == 0, -1, 1).astype(np.int8)


def random_orthogonal(d: int, seed: int, m: int) -> np.ndarray:
    """fp32 [d][d] orthogonal: Q of a seeded Gaussian QR with sign(diag R) folded in."""
    r = np.random.default_rng(np.random.SeedSequence([11, int(seed), d, int(m)]))
    a = r.standard_normal((d, d))
    q, rr = np.linalg.qr(a)
    q = q * np.sign(np.diag(rr))[None, :]
    return q.astype(np.float32)


def value_rotations(d: int, seed: int = 0, modalities: int = 3) -> np.ndarray:
    """fp32 [M][d][d]: one seeded orthogonal basis per modality."""
    return np.stack([random_orthogonal(d, seed, m) for m in range(modalities)])


def seq_lens(cfg: Config, ragged: bool = False, seed: int = 0) -> np.ndarray:
    """int32 [batch]: full context, or ragged lengths in (context/2, context]."""
    if not ragged:
        return np.full(cfg.batch, cfg.context, dtype=np.int32)
    r = rng_for(cfg.cid, seed, 3)
    return r.integers(cfg.context // 2 + 1, cfg.context + 1, cfg.batch).astype(np.int32)


# --------------------------------------------------------------------------- packed caches
def random_packed_cache(cfg: Config, seed: int = 0, key_bits: Optional[int] = None,
                        value_bits: Optional[int] = None, length: Optional[int] = None):
    """A synthetic packed cache drawn directly (no quantizer involved).

    Any bit pattern is a legal code array, so decode can be exercised at full
    size without running a quantizer first.  Metadata are drawn in the ranges a
    drifting N(0,1)-like cache produces: per window lambda ~ LogNormal(0, 0.4),
    key minimum ~ lambda * U(-3.5, -1.5), key step ~ lambda * U(0.6, 1.6) (2 bit;
    scaled by 3/15 for 4 bit), value scale ~ LogNormal(0, 0.4).  Returns a dict
    of numpy arrays in the library's storage shapes.
    """
    kb = cfg.key_bits if key_bits is None else key_bits
    vb = cfg.value_bits if value_bits is None else value_bits
    T = cfg.context if length is None else int(length)
    assert T % WINDOW == 0
    B, H, d = cfg.batch, cfg.kv_heads, cfg.head_dim
    nw = T // WINDOW
    r = rng_for(cfg.cid, seed, 4)
    k_words = d * kb          # 32-bit words per 32-token window
    v_words = d * vb
    k_codes = r.integers(0, 2**32, (B, H, nw, k_words), dtype=np.uint64).astype(np.uint32)
    v_codes = r.integers(0, 2**32, (B, H, nw, v_words), dtype=np.uint64).astype(np.uint32)
    lam = np.exp(0.4 * r.standard_normal((B, H, nw, 1)))
    kmin = lam * r.uniform(-3.5, -1.5, (B, H, nw, d))
    kstep = lam * r.uniform(0.6, 1.6, (B, H, nw, d)) * (3.0 / (2**kb - 1))
    vscale = np.exp(0.4 * r.standard_normal((B, H, T)))
    return dict(
        k_codes=k_codes, v_codes=v_codes,
        k_min=kmin.astype(np.float16).view(np.uint16),
        k_scale=kstep.astype(np.float16).view(np.uint16),
        v_scale=vscale.astype(np.float16).view(np.uint16),
        modality=modality_layout(cfg, seed, T),
        key_bits=kb, value_bits=vb, t_cap=T,
    )


# --------------------------------------------------------------------------- calibration clusters
def modality_clusters(d: int, seed: int, n: int = 8192, heavy_tail: bool = False):
    """Per-modality value clusters for the rotation-choice experiment.

    Modality m gets its own random orthogonal basis, a decaying spectrum
    lambda_i = exp(-i / (d / (4 + 3 m))) and a mean 0.7 * N(0, 1).  Returns
    (calibration, held_out): lists of three fp32 [n][d] arrays.
    """
    cal, held = [], []
    for m in range(3):
        r = np.random.default_rng(np.random.SeedSequence([13, int(seed), d, m]))
        basis = random_orthogonal(d, 1000 + seed, m).astype(np.float64)
        spec = np.exp(-np.arange(d) / (d / (4.0 + 3.0 * m)))
        mean = 0.7 * r.standard_normal(d)
        def draw(k):
            z = r.laplace(size=(k, d)) / np.sqrt(2.0) if heavy_tail else r.standard_normal((k, d))
            return ((z * np.sqrt(spec)) @ basis.T + mean).astype(np.float32)
        cal.append(draw(n))
        held.append(draw(n))
    return cal, held


def drifting_tensor_device(cfg: Config, tags, seed: int, stream: int, t0: int, n: int, device="cuda"):
    """Same recipe as drifting_tensor, drawn with torch's generator on `device`.

    Returns a contiguous [batch][n][kv_heads][head_dim] tensor (bf16, or fp32 for
    fp32 configs).  Draws differ from the numpy version; the distribution is
    the same.  `tags`: uint8 tensor or array [batch][>= t0+n].
    """
    import torch
    assert t0 % WINDOW == 0 and n % WINDOW == 0
    d, H, B = cfg.head_dim, cfg.kv_heads, cfg.batch
    nw = n // WINDOW
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([cfg.cid, seed, stream, t0]).generate_state(1)[0]))
    tg = torch.as_tensor(np.asarray(tags) if not isinstance(tags, torch.Tensor) else tags.cpu().numpy())
    first = tg[:, t0:t0 + n:WINDOW].to(device)                                   # [B][nw]
    z = torch.randn((B, nw, WINDOW, H, d), generator=g, device=device)
    mu = 0.5 * torch.randn((B, nw, 1, H, d), generator=g, device=device)
    sig = torch.where(first == TEXT, cfg.drift_text, cfg.drift_av).to(torch.float32)
    lam = torch.exp(sig[:, :, None] * torch.randn((B, nw, H), generator=g, device=device))
    x = lam[:, :, None, :, None] * (z + mu)
    gain = torch.ones((H, d), device=device)
    for h in range(H):
        idx = torch.randperm(d, generator=g, device=device)[: cfg.outliers]
        gain[h, idx] = cfg.outlier_gain
    x = (x * gain).reshape(B, n, H, d)
    return x.contiguous() if cfg.fp32_inputs else x.to(torch.bfloat16).contiguous()
