"""omnikv_decode_attention_noalloc (the decode step with the library's static scratch as its
workspace, for callers that cannot allocate) against omnikv_decode_attention with a caller
workspace, through the C ABI: two calls in a row, the second with a smaller input, each
bit-identical to the ordinary entry point's result; and a step too large for the scratch is
refused before anything is launched."""
import numpy as np
import pytest

from decode_attention_fwht_amd import binding, synth
from tests.gpu_helpers import cache_to_device, make_context, say, to_dev

pytestmark = pytest.mark.gpu


def _step(ctx, cfg, B, T, seed):
    import torch
    one = synth.Config(**{**cfg.__dict__, "batch": B})
    cache = cache_to_device(synth.random_packed_cache(one, seed, length=T))
    q = to_dev(synth.queries(one, seed))
    lens = to_dev(np.array([T - 5 * b for b in range(B)], np.int32))
    ref = ctx.decode(q, lens, T, cache)
    out = torch.full((B, cfg.q_heads, cfg.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    ctx.decode_noalloc(q, lens, T, cache, out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_the_workspace_entry_point_twice():
    import torch
    cfg = synth.CONFIGS[3]
    say("[noalloc] cfg3 16 x 32768 then 3 x 4096")
    ctx, signs, U, lv = make_context(cfg)
    ref, out = _step(ctx, cfg, 16, 32768, 41)
    assert torch.equal(out, ref)
    ref2, out2 = _step(ctx, cfg, 3, 4096, 42)   # smaller: the scratch keeps the first call's contents
    assert torch.equal(out2, ref2)
    ctx.close()


def test_noalloc_refuses_a_step_beyond_the_scratch():
    import torch
    cfg = synth.CONFIGS[3]
    say("[noalloc-limit] cfg3 with 1024 splits")
    ctx, signs, U, lv = make_context(cfg)
    T = 32768
    assert ctx.workspace_size(16, T, 1024) > (12 << 20)
    cache = cache_to_device(synth.random_packed_cache(cfg, 43, length=T))
    q = to_dev(synth.queries(cfg, 43))
    lens = to_dev(np.full(16, T, np.int32))
    out = torch.zeros((16, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.OmniKVError) as e:
        ctx.decode_noalloc(q, lens, T, cache, out, num_splits=1024)
    assert e.value.status == binding.EINVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not torch.any(out)
    ctx.close()
