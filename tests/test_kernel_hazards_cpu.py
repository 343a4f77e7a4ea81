"""Host-side checks of the compiled kernels (gfx950 assembly from hipcc -S) for
two ordering properties that parity tests only catch when a schedule happens
to expose them, as wrong and run-to-run different outputs.

1. No workgroup barrier is reached while this wavefront still has LDS
   accesses outstanding. The K/V rings refill a stage right after a barrier;
   a read of that stage still in flight (the compiler may sink a read's
   consumers past the barrier and leave the read ahead of it) would then
   race the refill.
2. No instruction touches an MFMA's destination registers sooner after the
   MFMA than the compiler itself waits before a plain vector read of that
   MFMA's result (measured here on a probe kernel per MFMA shape). The
   compiler places 64-bit register moves (v_mov_b64) that read a scaled FP8
   MFMA's result one wait state earlier than that, and such a copy read
   stale rows on MI355X.

3. Every LDS-bound global load (global_load_lds_*, whose LDS address is M0)
   comes at least one wait state after the last scalar write of M0, as the
   ISA's table of manually inserted wait states asks and as the compiler
   does in its own code (s_nop 0 between the two).

Paths are followed over the control-flow graph of each kernel: one wait state
per instruction, N + 1 per s_nop N (inline assembly counted as written).
"""

import collections
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_online_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fp8.hip"]
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-x", "hip", "--cuda-device-only", "-S"]

# one kernel per MFMA shape the library uses: the MFMA, then a plain add of
# its last result register
PROBE = r"""
#include <hip/hip_runtime.h>
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__global__ void p_scale_32x32x64_f8f6f4(const i32x8* a, const i32x8* b, float* o, int s) {
  f32x16 c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[threadIdx.x], b[threadIdx.x], f32x16{}, 0, 0, 0, s, 0, 127);
  o[threadIdx.x] = c[15] + 1.f;
}
__global__ void p_32x32x16_bf16(const bf16x8* a, const bf16x8* b, float* o) {
  f32x16 c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], b[threadIdx.x], f32x16{}, 0, 0, 0);
  o[threadIdx.x] = c[15] + 1.f;
}
__global__ void p_16x16x32_bf16(const bf16x8* a, const bf16x8* b, float* o) {
  f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], b[threadIdx.x], f32x4{}, 0, 0, 0);
  o[threadIdx.x] = c[3] + 1.f;
}
"""


def _compile(src, out):
    subprocess.run([HIPCC, *FLAGS, src, "-o", out], check=True, capture_output=True)
    with open(out) as f:
        return f.read().split("\n")


def _functions(lines):
    """{kernel symbol: [instruction text]} and {kernel: {label: index}}."""
    funcs, labels, cur = {}, {}, None
    for ln in lines:
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            cur = m.group(1)
            funcs[cur], labels[cur] = [], {}
            continue
        if cur is None:
            continue
        s = ln.strip()
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        if not s or s.startswith(";"):
            continue
        m = re.match(r"^(\.LBB\S+):", s)
        if m:
            labels[cur][m.group(1)] = len(funcs[cur])
            continue
        if s.startswith(".") or re.match(r"^\w+:$", s):
            continue
        funcs[cur].append(s)
    return funcs, labels


def _successors(ins, labels, j):
    parts = ins[j].split()
    op = parts[0]
    if op in ("s_endpgm", "s_setpc_b64"):
        return []
    if op == "s_branch":
        return [labels[parts[1]]] if parts[1] in labels else []
    out = []
    if op.startswith("s_cbranch") and parts[1] in labels:
        out.append(labels[parts[1]])
    if j + 1 < len(ins):
        out.append(j + 1)
    return out


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", text):
        out |= {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in re.finditer(r"\b([va])(\d+)\b", text):
        out.add((m.group(1), int(m.group(2))))
    return out


def _wait_states(s):
    parts = s.split()
    return int(parts[1], 0) + 1 if parts[0] == "s_nop" else 1


def barriers_with_lds_outstanding(ins, labels):
    """[(instruction index, LDS accesses possibly outstanding)] for each s_barrier."""
    def run(j0, x, report=None):
        j = j0
        while True:
            s = ins[j]
            op = s.split()[0]
            if op.startswith("ds_"):
                x = min(x + 1, 15)  # the counter's range: issue stalls beyond it
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if op == "s_waitcnt" and m:
                x = min(x, int(m.group(1)))
            if op == "s_barrier" and report is not None and x > 0:
                report.append((j, x))
            nxt = _successors(ins, labels, j)
            if nxt != [j + 1] or (j + 1) in starts:
                return x, nxt
            j += 1
    starts = {0} | set(labels.values())
    for j in range(len(ins)):
        if ins[j].split()[0].startswith(("s_branch", "s_cbranch")) and j + 1 < len(ins):
            starts.add(j + 1)
    entry = {b: 0 for b in starts}
    changed = True
    while changed:
        changed = False
        for b in sorted(starts):
            x, nxt = run(b, entry[b])
            for t in nxt:
                if t in entry and x > entry[t]:
                    entry[t] = x
                    changed = True
    report = []
    for b in sorted(starts):
        run(b, entry[b], report)
    return report


def short_mfma_reads(ins, labels, bound):
    """[(wait states, bound, MFMA, instruction)] for each access to an MFMA's
    destination registers closer to it than `bound` (per MFMA opcode)."""
    bad = []
    for i, s in enumerate(ins):
        op = s.split()[0]
        if "mfma" not in op:
            continue
        assert op in bound, f"no probe for {op}"
        need = bound[op]
        dst = _regs(s.split(None, 1)[1].split(",")[0])
        stack = [(k, 0) for k in _successors(ins, labels, i)]
        seen = {}
        while stack:
            j, ws = stack.pop()
            if ws >= need or seen.get(j, need) <= ws:
                continue
            seen[j] = ws
            s2 = ins[j]
            op2 = s2.split()[0]
            rest = s2.split(None, 1)[1] if " " in s2 else ""
            # the next MFMA of an accumulation chain reads the result through
            # the matrix unit's own dependency check
            if "mfma" not in op2 and op2 != "s_nop" and _regs(rest) & dst:
                bad.append((ws, need, s[:60], s2[:60]))
                continue
            stack += [(k, ws + _wait_states(s2)) for k in _successors(ins, labels, j)]
    return bad


def m0_write_then_lds_dma(ins, labels):
    """[(index of the M0 write, the load)] where an LDS-bound global load
    follows a scalar write of M0 with no wait state between."""
    bad = []
    for i, s in enumerate(ins):
        if not re.match(r"^s_\w+\s+m0\s*,", s):
            continue
        for j in _successors(ins, labels, i):
            if ins[j].split()[0].startswith("global_load_lds"):
                bad.append((i, ins[j][:60]))
    return bad


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    d = tmp_path_factory.mktemp("asm")
    probe = d / "probe.hip"
    probe.write_text(PROBE)
    jobs = [(str(probe), str(d / "probe.s"))] + [(os.path.join(CSRC, s), str(d / (s + ".s"))) for s in SOURCES]
    with ThreadPoolExecutor(4) as ex:
        outs = list(ex.map(lambda j: _compile(*j), jobs))
    return outs[0], dict(zip(SOURCES, outs[1:]))


def _probe_bounds(probe_lines):
    funcs, _ = _functions(probe_lines)
    bound = {}
    for ins in funcs.values():
        i = next(k for k, s in enumerate(ins) if "mfma" in s.split()[0])
        ws = 0
        for s in ins[i + 1:]:
            if s.split()[0] == "v_add_f32_e32":
                break
            ws += _wait_states(s)
        bound[ins[i].split()[0]] = ws
    return bound


def test_probe_bounds_are_plausible(compiled):
    bound = _probe_bounds(compiled[0])
    assert set(bound) == {"v_mfma_scale_f32_32x32x64_f8f6f4", "v_mfma_f32_32x32x16_bf16", "v_mfma_f32_16x16x32_bf16"}
    # more passes, longer wait: the 64-deep FP8 shape outlasts the bf16 ones
    assert bound["v_mfma_scale_f32_32x32x64_f8f6f4"] > bound["v_mfma_f32_32x32x16_bf16"] > \
        bound["v_mfma_f32_16x16x32_bf16"] > 0


@pytest.mark.parametrize("src", SOURCES)
def test_no_barrier_with_lds_accesses_outstanding(compiled, src):
    funcs, labels = _functions(compiled[1][src])
    assert funcs
    bad = {k[:100]: r for k, ins in funcs.items() if (r := barriers_with_lds_outstanding(ins, labels[k]))}
    assert not bad, bad


@pytest.mark.parametrize("src", SOURCES)
def test_mfma_results_read_no_sooner_than_the_compiler_bound(compiled, src):
    bound = _probe_bounds(compiled[0])
    funcs, labels = _functions(compiled[1][src])
    bad = {}
    for k, ins in funcs.items():
        r = short_mfma_reads(ins, labels[k], bound)
        if r:
            bad[k[:100]] = collections.Counter((w, n, s.split()[0]) for w, n, _, s in r)
    assert not bad, bad


@pytest.mark.parametrize("src", SOURCES)
def test_lds_dma_waits_for_its_m0_write(compiled, src):
    funcs, labels = _functions(compiled[1][src])
    bad = {k[:100]: r for k, ins in funcs.items() if (r := m0_write_then_lds_dma(ins, labels[k]))}
    assert not bad, bad
