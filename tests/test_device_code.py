"""Properties of the generated gfx950 code that the kernels rely on, checked
on the CPU from hipcc's device assembly."""
import os
import re
import subprocess

import pytest

from mla_paged_kv_metadata_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Instructions that read M0 without naming it.
IMPLICIT_M0 = ("s_sendmsg", "s_movrel", "v_movrel", "v_interp", "ds_gws", "s_set_gpr_idx", "buffer_load_lds",
               "global_load_lds", "ds_append", "ds_consume")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "mla_decode.s")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([cc, *flags, "-x", "hip", "--offload-device-only", "-S", "-I", os.path.join(ROOT, "include"),
                    "-o", out, os.path.join(build.CSRC, "mla_decode.hip")], check=True, capture_output=True,
                   timeout=600)
    lines = []
    for raw in open(out):
        t = raw.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            lines.append(t)
    return lines


def test_m0_is_written_only_right_before_the_lds_copies(device_asm):
    """The LDS-DMA copy helpers set M0 in their own asm and list it as
    clobbered; that is only safe if no other code keeps a value in M0.  Every
    M0 write must be one helper's, followed by its wait state and copy, and
    every instruction that reads M0 implicitly must be such a copy."""
    writes = 0
    for i, t in enumerate(device_asm):
        op = t.split()[0]
        if re.search(r"\bm0\b", t):
            assert t.startswith("s_mov_b32 m0, s"), t
            assert device_asm[i + 1] == "s_nop 0", (t, device_asm[i + 1])
            assert device_asm[i + 2].startswith("global_load_lds_dwordx4"), (t, device_asm[i + 2])
            writes += 1
        elif op.startswith(IMPLICIT_M0):
            assert op == "global_load_lds_dwordx4" and device_asm[i - 2].startswith("s_mov_b32 m0, s"), t
    assert writes > 0


def test_no_packed_fp32_arithmetic(device_asm):
    """The device code is built without packed fp32 VALU forms."""
    bad = [t for t in device_asm if t.split()[0] in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")]
    assert not bad, bad[:3]

