"""Static check of the device code's LDS copies (global_load_lds_*), on the CPU: the kernels are
compiled to gfx950 assembly and every copy must be at least five wait states away from a vector
instruction that writes a scalar register it reads (its scalar base, or M0 with the LDS
address).  The copies are inline assembly, which the compiler's hazard checks do not look
into; a vector write of the base (v_readfirstlane) followed too closely by a copy makes the
copy read the register's old value, i.e. a wrong address."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_relation_distillation_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
NEEDED = 5  # wait states between a VALU write of an SGPR and a memory instruction reading it


def _sregs(op):
    op = op.strip()
    if op == "m0":
        return {"m0"}
    m = re.match(r"s\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", op)
    return {int(m.group(1))} if m else set()


def copy_hazards(asm_text):
    """(copies, hazards): every global_load_lds_* and the vector writes of its scalar operands
    (M0 included) that come fewer than NEEDED wait states before it."""
    ins = []
    for line in asm_text.splitlines():
        t = line.strip()
        if not t or t[0] in ";." or t.endswith(":"):
            continue
        ins.append(t)
    copies, hazards = 0, []
    for k, t in enumerate(ins):
        if not t.startswith("global_load_lds"):
            continue
        copies += 1
        used = {"m0"}
        if " " in t:
            for op in t.split(None, 1)[1].split(","):
                used |= _sregs(op)
        waits = 0
        for j in range(k - 1, max(-1, k - 16), -1):
            p = ins[j]
            if waits >= NEEDED:
                break
            if p.startswith("s_nop"):
                parts = p.split()
                waits += (int(parts[1], 0) + 1) if len(parts) > 1 else 1
                continue
            if p.startswith("v_") and " " in p:
                dst = p.split(None, 1)[1].split(",")[0]
                if _sregs(dst) & used:
                    hazards.append((p, t, waits))
            waits += 1
    return copies, hazards


def test_scanner_flags_a_close_vector_write():
    bad = "v_readfirstlane_b32 s8, v2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    good = "v_readfirstlane_b32 s8, v2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    m0 = "v_readfirstlane_b32 m0, v2\n\tglobal_load_lds_dwordx4 v1, off\n"
    salu = "s_mov_b32 m0, s3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    assert copy_hazards(bad) == (1, [("v_readfirstlane_b32 s8, v2", "global_load_lds_dwordx4 v1, s[8:9]", 1)])
    assert copy_hazards(good) == (1, [])
    assert len(copy_hazards(m0)[1]) == 1
    assert copy_hazards(salu) == (1, [])


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_kernel_copies_are_clear_of_vector_scalar_writes(tmp_path):
    out = tmp_path / "kernels.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, "relkl_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    copies, hazards = copy_hazards(out.read_text())
    assert copies > 100  # every kernel stages its tiles with these copies
    assert hazards == [], hazards[:5]
