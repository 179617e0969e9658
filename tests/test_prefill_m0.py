"""The prefill kernels' global->LDS copies set m0 (the LDS base of the copy)
in inline asm that the compiler does not see as a write of m0 (it reserves
the register and will not take it as a clobber).  That is sound only while
nothing else in those kernels uses m0.  This CPU test compiles prefill.hip to
gfx950 assembly with the library's flags and checks that every mention of m0
is one of those `s_mov_b32 m0, sN` immediately followed by its
global_load_lds_dword(x4), and that no instruction which reads m0 implicitly
(movrel, sendmsg, GWS, ordered count, append/consume, addtid, interpolation,
buffer->LDS loads) appears."""
import os
import re
import shutil
import subprocess

import pytest

from paged_kv_gqa_pkv_amd import build as B

IMPLICIT_M0 = re.compile(
    r"^\s*(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_ordered_count|ds_append|ds_consume|"
    r"ds_read_addtid|ds_write_addtid|v_interp|buffer_load_\w+ .*\blds\b|s_set_gpr_idx)")


def _device_asm(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "prefill.s"
    cmd = [hipcc, *[f for f in B.COMMON if f != "-fPIC"], *B.EXTRA.get("prefill.hip", []),
           "--cuda-device-only", "-S", "-x", "hip", os.path.join(B.CSRC, "prefill.hip"),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def _instructions(lines):
    for ln in lines:
        code = ln.split(";")[0].strip()
        if not code or code.startswith(".") or code.endswith(":"):
            continue
        yield code


def test_m0_only_feeds_the_lds_copies(tmp_path):
    ins = list(_instructions(_device_asm(tmp_path)))
    copies = 0
    for i, code in enumerate(ins):
        assert not IMPLICIT_M0.match(code), f"implicit m0 user in prefill: {code}"
        if re.search(r"\bm0\b", code):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", code), f"other use of m0: {code}"
            assert ins[i + 1].startswith("global_load_lds_dword"), \
                f"m0 set but not used by the next instruction: {code} / {ins[i + 1]}"
            copies += 1
    n_dma = sum(c.startswith("global_load_lds_dword") for c in ins)
    assert copies > 0 and copies == n_dma, (copies, n_dma)
