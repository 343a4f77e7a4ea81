"""Host-side checks of the hand-scheduled 64-row prefill shape: the committed
header is what its generator writes, and in the compiled kernel no
instruction outside the inline-assembly statements touches the registers
those statements keep between them (every AGPR, and v192..v255 before the
epilogue reads the output back), which the shape's correctness relies on."""

import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_online_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
KERNEL = "_ZN2fa12_GLOBAL__N_115fwd_bf16_kernelINS0_3CfgILi128ELi64ELi2ELi2ELi2ELi1ELb0ELb1EEEEEvNS0_9FwdParamsE"


def test_generated_header_matches_generator():
    sys.path.insert(0, CSRC)
    try:
        import gen_fwd_tile_asm as g
    finally:
        sys.path.pop(0)
    with open(os.path.join(CSRC, "fa_fwd_tile_asm.h")) as f:
        assert f.read() == g.header()


def _regs(text):
    out = []
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", text):
        out += [(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)]
    for m in re.finditer(r"\b([va])(\d+)\b", text):
        out.append((m.group(1), int(m.group(2))))
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_compiled_kernel_leaves_the_fixed_registers_alone(tmp_path):
    out = tmp_path / "fwd.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-x", "hip", "--cuda-device-only",
           "-S", os.path.join(CSRC, "fa_fwd_bf16.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    lines = out.read_text().split("\n")
    start = next(i for i, ln in enumerate(lines) if ln.startswith(KERNEL + ":"))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    body = lines[start:end + 1]
    # the epilogue begins with the statement that reads the output back
    # (its first instruction after four s_nop 7)
    o_read = max(i for i, ln in enumerate(body) if "v_accvgpr_read_b32 v72, a0" in ln)
    in_asm, bad = False, []
    for i, ln in enumerate(body):
        if ";;#ASMSTART" in ln:
            in_asm = True
            continue
        if ";;#ASMEND" in ln:
            in_asm = False
            continue
        s = ln.split(";")[0].strip()
        if in_asm or not s or s.endswith(":") or s.startswith("."):
            continue
        for kind, n in _regs(s):
            if kind == "a" or (kind == "v" and n >= 192 and i < o_read):
                bad.append(s)
                break
    assert not bad, bad[:10]
