"""Static check of the gfx950 assembly of every kernel unit: no instruction
other than a matrix op reads or overwrites the destination registers of a
matrix op (MFMA) fewer wait states after it than the hardware requires.

The compiler inserts those wait states for the instructions it generates,
but not around inline asm, and the kernels hold hand-placed asm (the
biased-accumulator S MFMA, empty register pins).  An asm instruction that
touched a result still in flight would read stale data or be overwritten
without any error, so the assembly is scanned here.  The required wait
states per MFMA shape are those LLVM itself emits between an isolated MFMA
of that shape and a dependent add, compiled once in this test.  The scan
follows straight-line code: it drops its window at labels reached only by a
jump, after unconditional branches and at the end of a program.
"""
import os
import re
import shutil
import subprocess

import pytest

from bit_quantized_attention_sage_amd import build as B

HIPCC = B.HIPCC
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc is not installed")

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")

# one isolated MFMA of each shape the kernels use, followed by a dependent add
_CALIBRATION = r"""
#include <hip/hip_runtime.h>
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
__global__ void i8_32(const v4i* a, int* o) {
  v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[threadIdx.x], a[threadIdx.x + 64], v16i{}, 0, 0, 0);
  o[threadIdx.x] = c[0] + 1;
}
__global__ void f8_32(const v8i* a, float* o) {
  v16f c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[threadIdx.x], a[threadIdx.x + 64], v16f{}, 0, 0, 0, 127, 0, 127);
  o[threadIdx.x] = c[0] + 1.f;
}
__global__ void f8_16(const v8i* a, float* o) {
  v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[threadIdx.x], a[threadIdx.x + 64], v4f{}, 0, 0, 0, 127, 0, 127);
  o[threadIdx.x] = c[0] + 1.f;
}
__global__ void bf16_32(const v8bf* a, float* o) {
  v16f c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], a[threadIdx.x + 64], v16f{}, 0, 0, 0);
  o[threadIdx.x] = c[0] + 1.f;
}
__global__ void bf16_16(const v8bf* a, float* o) {
  v4f c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], a[threadIdx.x + 64], v4f{}, 0, 0, 0);
  o[threadIdx.x] = c[0] + 1.f;
}
__global__ void f16_32(const v8h* a, float* o) {
  v16f c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[threadIdx.x], a[threadIdx.x + 64], v16f{}, 0, 0, 0);
  o[threadIdx.x] = c[0] + 1.f;
}
__global__ void f16_16(const v8h* a, float* o) {
  v4f c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[threadIdx.x], a[threadIdx.x + 64], v4f{}, 0, 0, 0);
  o[threadIdx.x] = c[0] + 1.f;
}
"""


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _assemble(src_path, extra, out_path):
    cmd = [HIPCC] + B.COMMON + extra + ["--cuda-device-only", "-S", src_path, "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out_path).read().splitlines()


def _instructions(lines):
    """(kind, opcode, operand text) per line: label, instr or None."""
    for line in lines:
        t = line.split(";")[0].strip()
        if not t or t.startswith("."):
            if re.match(r"^\.LBB\w*:", t):
                yield "label", t, ""
            continue
        if re.match(r"^[A-Za-z_][\w.$]*:", t):
            yield "func", t[:-1], ""
            continue
        op = t.split()[0]
        yield "instr", op, t[len(op):]


@pytest.fixture(scope="module")
def required_waits(tmp_path_factory):
    """Wait states LLVM puts between each MFMA shape and a dependent VALU op."""
    d = tmp_path_factory.mktemp("cal")
    src = d / "cal.hip"
    src.write_text(_CALIBRATION)
    lines = _assemble(str(src), [], str(d / "cal.s"))
    need, last_mfma, waits = {}, None, 0
    for kind, op, rest in _instructions(lines):
        if kind != "instr":
            continue
        if op.startswith("v_mfma"):
            last_mfma, waits = op, 0
        elif last_mfma and op.startswith("v_add") and _regs(rest) & {2}:
            need[last_mfma] = waits
            last_mfma = None
        elif last_mfma:
            waits += int(rest.strip()) + 1 if op == "s_nop" else 1
    assert len(need) == 7, need
    return need


def _scan(lines, need):
    hits, pending, func = [], [], None
    for kind, op, rest in _instructions(lines):
        if kind == "func":
            func, pending = op, []
            continue
        if kind == "label":
            continue  # fall-through keeps the window
        adv = int(rest.strip()) + 1 if op == "s_nop" else 1
        if op.startswith("v_mfma"):
            parts = rest.split(",")
            pending = [(d, w + 1, q, x) for d, w, q, x in pending]
            pending.append((_regs(parts[0]), 0, need[op], op))
            continue
        if op != "s_nop":
            touched = _regs(rest)
            for d, w, q, x in pending:
                if d & touched and w < q:
                    hits.append(f"{func}: {op}{rest} {w} wait states after {x} (needs {q})")
        pending = [(d, w + adv, q, x) for d, w, q, x in pending if w + adv < q]
        if op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            pending = []
    return hits


def test_calibration_is_sane(required_waits):
    # 8-pass shapes need more than 4-pass ones, 16-pass more than 8-pass
    assert required_waits["v_mfma_f32_16x16x32_bf16"] < required_waits["v_mfma_i32_32x32x32_i8"]
    assert required_waits["v_mfma_i32_32x32x32_i8"] < required_waits["v_mfma_scale_f32_32x32x64_f8f6f4"]


def test_scanner_flags_an_early_read(required_waits):
    lines = ["k:", "v_mfma_i32_32x32x32_i8 v[2:17], v[20:23], v[24:27], 0",
             "v_add_u32_e32 v1, 1, v2", "s_endpgm",
             "k2:", "v_mfma_i32_32x32x32_i8 v[2:17], v[20:23], v[24:27], 0",
             f"s_nop {required_waits['v_mfma_i32_32x32x32_i8'] - 1}", "v_add_u32_e32 v1, 1, v2", "s_endpgm"]
    hits = _scan(lines, required_waits)
    assert len(hits) == 1 and hits[0].startswith("k:")


@pytest.mark.parametrize("unit", [u for u in B.UNITS if u.endswith(".hip")])
def test_no_mfma_result_hazards(unit, required_waits, tmp_path):
    lines = _assemble(os.path.join(B.CSRC, unit), B.UNITS[unit], str(tmp_path / "k.s"))
    unknown = {op for kind, op, _ in _instructions(lines)
               if kind == "instr" and op.startswith("v_mfma") and op not in required_waits}
    assert not unknown, f"MFMA shapes without a calibrated wait: {unknown}"
    hits = _scan(lines, required_waits)
    assert not hits, "\n".join(hits[:20])


def _softmax_phase_mfmas(lines):
    """Per fused-kernel function, the MFMAs found after a matrix phase's end
    (`s_setprio 0` then `s_barrier`) and before the next barrier, priority
    raise, branch or loop header, in text order."""
    out, func = {}, None
    instrs = list(_instructions(lines))
    for i, (kind, op, rest) in enumerate(instrs):
        if kind == "func":
            func = op
            continue
        if kind != "instr" or op != "s_setprio" or rest.strip() != "0" or "attn_fwd_kernel" not in str(func):
            continue
        if i + 1 >= len(instrs) or instrs[i + 1][1] != "s_barrier":
            continue
        for kind2, op2, _ in instrs[i + 2:]:
            if kind2 == "func" or op2 in ("s_barrier", "s_branch", "s_endpgm") or (op2 == "s_setprio"):
                break
            if kind2 == "instr" and op2.startswith("v_mfma"):
                out.setdefault(func, []).append(op2)
    return out


def test_scanner_finds_an_mfma_in_a_softmax_phase():
    lines = ["_ZN4sage15attn_fwd_kernelX:", "s_setprio 0", "s_barrier", "v_exp_f32_e32 v1, v1",
             "v_mfma_f32_32x32x16_bf16 v[2:17], v[20:23], v[24:27], v[2:17]", "s_barrier", "s_endpgm"]
    assert _softmax_phase_mfmas(lines) == {"_ZN4sage15attn_fwd_kernelX": ["v_mfma_f32_32x32x16_bf16"]}


def test_fused_kernel_phases_keep_their_mfmas(tmp_path):
    """The ping-pong kernel's matrix work belongs to its MFMA phase: the
    compiler may sink a pure MFMA past the phase barrier (it did, for the FP8
    P.V MFMAs of boundary-checked steps), which puts matrix work and its
    operand waits into the softmax phase.  No instantiation may have any."""
    lines = _assemble(os.path.join(B.CSRC, "attn.hip"), B.UNITS["attn.hip"], str(tmp_path / "a.s"))
    found = _softmax_phase_mfmas(lines)
    assert not found, {f: len(v) for f, v in found.items()}
