"""Source checks of the HIP kernels for a miscompiled builtin (no GPU).

hipcc of ROCm 7.2 compiles __builtin_bit_cast whose operand is an element of
an ext_vector_type vector (v[i]) as a read of element 0, whatever i is.  A
zero or finiteness test written that way looks at one float in four.  The
kernels take single-element bit patterns through by-value helpers
(kda::f32_bits, kda::bits_f32); the lint keeps every call site on them and the
probe shows that the helper reads the element it names.
"""
import glob
import os
import re
import shutil
import subprocess

import pytest

from gated_delta_rule_46_amd.build import HIPCC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_46_amd", "csrc")

# an operand that is an element access: name[...][...] or name.member
ELEMENT = re.compile(r"[A-Za-z_][\w.]*(\s*\[[^\[\]]+\])+|[A-Za-z_]\w*(\.\w+)+")


def bit_cast_operands(text):
    """(line, operand) of every __builtin_bit_cast(T, operand) in text."""
    out = []
    for m in re.finditer(r"__builtin_bit_cast\s*\(", text):
        depth, i, comma = 1, m.end(), None
        while depth:
            ch = text[i]
            if ch in "([":
                depth += 1
            elif ch in ")]":
                depth -= 1
            elif ch == "," and depth == 1 and comma is None:
                comma = i
            i += 1
        out.append((text.count("\n", 0, m.start()) + 1, text[comma + 1:i - 1].strip()))
    return out


def test_lint_finds_element_operands():
    """The lint flags the miscompiled forms and passes values and expressions."""
    src = """
        a = __builtin_bit_cast(uint32_t, x[c]);
        b = __builtin_bit_cast(uint32_t, S[r][n][i]) & 1u;
        c = __builtin_bit_cast(float, v.y);
        d = __builtin_bit_cast(float, w[j] << 16);
        e = __builtin_bit_cast(u32x4, f);
        g = __builtin_bit_cast(bf16x8, *(const uint4 *)&raw.k[8]);
    """
    flagged = [op for _, op in bit_cast_operands(src) if ELEMENT.fullmatch(op)]
    assert flagged == ["x[c]", "S[r][n][i]", "v.y"]


def test_kernels_take_element_bits_by_value():
    bad = []
    for path in sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(CSRC, "*.hip"))):
        text = open(path).read()
        for line, op in bit_cast_operands(text):
            if ELEMENT.fullmatch(op):
                bad.append(f"{os.path.basename(path)}:{line}: __builtin_bit_cast(..., {op})")
    assert not bad, "element operands of __builtin_bit_cast (use kda::f32_bits / bits_f32):\n" + \
        "\n".join(bad)


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                    reason="hipcc not installed")
def test_helper_reads_the_named_element(tmp_path):
    """Device IR of f32_bits(v[2]) extracts element 2 of the loaded vector."""
    src = tmp_path / "probe.hip"
    src.write_text(
        '#include "kda_internal.h"\n'
        "typedef float f32x4 __attribute__((ext_vector_type(4)));\n"
        "__global__ void probe(const f32x4 *p, unsigned *o) {\n"
        "    f32x4 x = p[threadIdx.x];\n"
        "    o[threadIdx.x] = kda::f32_bits(x[2]);\n"
        "}\n")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC,
                        "--cuda-device-only", "-S", "-emit-llvm", str(src), "-o", "-"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    body = r.stdout[r.stdout.index("define"):]
    assert re.search(r"extractelement <4 x (i32|float)> %\d+, i64 2", body), body[:2000]
