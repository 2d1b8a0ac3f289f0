"""Value-rotation calibration through the C ABI against the oracle's definition
([paper] §2.3; [digest] 方法概览): weighted second moment on the GPU in float64,
eigenvectors on the host, composed with the normalized Hadamard.  Bar: U equal to the
oracle's (float64 eigh) within 1e-5 per entry, orthogonal to 1e-5."""
import numpy as np
import pytest

from oracle import omnikv_oracle as O
from decode_attention_fwht_amd import binding, synth
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,bf16,weighted", [(64, False, False), (128, False, True), (128, True, True),
                                             (64, True, False)])
def test_calibration_matches_oracle(d, bf16, weighted):
    import torch
    say(f"[calibrate] d={d} bf16={bf16} weighted={weighted}")
    cal, _ = synth.modality_clusters(d, 1, n=5000)
    rng = np.random.default_rng(d)
    for m in range(3):
        v = cal[m]
        if bf16:
            v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
        w = rng.uniform(0.1, 2.0, v.shape[0]).astype(np.float32) if weighted else None
        vt = torch.from_numpy(v).cuda()
        if bf16:
            vt = vt.to(torch.bfloat16).contiguous()
        wt = torch.from_numpy(w).cuda() if weighted else None
        U = binding.calibrate_value_rotation(vt, wt)
        ref = O.calibrate_value_rotation(v, w)
        err = np.max(np.abs(U - ref))
        say(f"    modality {m}: max |U - U_oracle| {err:.2e}")
        assert err <= 1e-5
        assert np.allclose(U.T.astype(np.float64) @ U, np.eye(d), atol=1e-5)


def test_calibrated_rotations_run_through_the_codec():
    """A context built from calibrated rotations quantizes each modality's values with
    lower error than one built from another modality's rotation (end to end on the GPU
    write path, errors measured with the oracle's dequantization)."""
    import torch
    d = 128
    cal, held = synth.modality_clusters(d, 2, n=4096)
    Us = np.stack([binding.calibrate_value_rotation(torch.from_numpy(c).cuda()) for c in cal])
    signs = synth.rademacher_signs(d, 0)
    lv = O.value_codebook_f16(2)
    n = 1024
    for rot_name, rots in (("matched", Us), ("shifted", np.roll(Us, 1, axis=0))):
        ctx = binding.Context(d, 8, 1, 2, 2, signs, np.ascontiguousarray(rots))
        errs = []
        for m in range(3):
            v = held[m][:n].astype(np.float32)
            cache = ctx.alloc_cache(1, n)
            cache["modality"].fill_(m)
            ctx.quantize_values(torch.from_numpy(v[None, :, None, :]).cuda().contiguous(), 0, cache)
            torch.cuda.synchronize()
            vc = cache["v_codes"].cpu().numpy().view(np.uint32)
            vs = cache["v_scale"].cpu().numpy().view(np.uint16)
            vh = O.dequantize_values(vc, vs, np.full((1, n), m, np.uint8), rots, lv, 2)[0, 0]
            errs.append(float(np.mean((vh - v) ** 2) / np.mean(v.astype(np.float64) ** 2)))
        say(f"    {rot_name}: relative MSE per modality {[round(e, 4) for e in errs]}")
        if rot_name == "matched":
            matched = errs
        else:
            assert all(a < b for a, b in zip(matched, errs))
        ctx.close()
