"""Checks of the compiled gfx950 code that the sources rely on (no GPU needed; hipcc
cross-compiles).

The decode kernel's global->LDS copies are inline asm that set M0 (the LDS base of the
copy) and declare it clobbered.  M0 is a reserved register to the compiler, so that
declaration is only sound while no compiler-generated instruction in the decode kernels
reads or writes M0 (movrel indexing, s_sendmsg, GWS, interpolation, ...).  The test
compiles decode.hip with the library's own flags and checks that every M0 reference is
one of the copies: `s_mov_b32 m0, <sgpr>`, a wait state, then `global_load_lds_*`.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from decode_attention_fwht_amd import build as B


def _have_hipcc() -> bool:
    try:
        h = B._hipcc()
    except RuntimeError:
        return False
    return os.path.exists(h) or shutil.which(h) is not None


pytestmark = pytest.mark.skipif(not _have_hipcc(), reason="hipcc not found")


def _decode_asm() -> str:
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "decode.s")
        cmd = [B._hipcc(), *B.FLAGS, *B.EXTRA["decode.hip"], "--cuda-device-only", "-S",
               os.path.join(B.CSRC, "decode.hip"), "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-2000:]
        return open(out).read()


def test_decode_m0_is_only_the_copies_lds_base():
    lines = [l.split(";")[0].strip() for l in _decode_asm().splitlines()]
    code = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    copies = 0
    for i, l in enumerate(code):
        if not re.search(r"\bm0\b", l):
            continue
        # the copy's own M0 write, followed by one wait state and the copy that reads M0
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"M0 used outside the LDS copies: {l!r}"
        assert code[i + 1] == "s_nop 0", code[i + 1]
        assert code[i + 2].startswith("global_load_lds_"), code[i + 2]
        copies += 1
    assert copies > 0
    # no instruction that reads M0 implicitly, other than the copies
    implicit = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws|v_interp|ds_append|ds_consume|s_ttracedata)")
    bad = [l for l in code if implicit.match(l)]
    assert not bad, bad[:5]
