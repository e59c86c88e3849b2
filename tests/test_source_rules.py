"""Rules on the HIP sources that no compiler check enforces.

Every inline-asm statement that writes M0 (the LDS base of gfx950's
global -> LDS copies) must name it in its clobber list, so that the compiler
orders the statement against its own uses of M0. No hand-written packed FP32
arithmetic appears anywhere (the build also turns the compiler's own off).
"""

import glob
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "int8_hadamard_domain_amd", "csrc")


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")))


def _asm_statements(text):
    """Every `asm volatile(...)` / `asm(...)` statement of a source, whole."""
    out = []
    for m in re.finditer(r"\basm\s*(volatile\s*)?\(", text):
        i, depth = m.end() - 1, 0
        while True:
            c = text[i]
            if c == '"':                       # skip string literals (may hold parentheses)
                i += 1
                while text[i] != '"':
                    i += 2 if text[i] == "\\" else 1
            elif c == "(":
                depth += 1
            elif c == ")":
                depth -= 1
                if depth == 0:
                    break
            i += 1
        out.append(text[m.start():i + 1])
    return out


def _writes_m0(stmt):
    # the template strings: an instruction whose destination (first operand) is m0
    tmpl = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', stmt.split(":")[0]))
    return re.search(r"\b[sv]_\w+\s+m0\s*,", tmpl.replace("\\n", "\n").replace("\\t", " ")) is not None


def test_asm_writing_m0_declares_the_clobber():
    found = 0
    for path in _sources():
        with open(path) as f:
            text = f.read()
        for stmt in _asm_statements(text):
            if _writes_m0(stmt):
                found += 1
                clobbers = stmt.split(":")[-1]
                assert '"m0"' in clobbers, f"{os.path.basename(path)}: asm writes m0 without declaring it: {stmt}"
    assert found > 0   # the copy helpers exist, so the check is not vacuous


def test_checker_sees_a_missing_clobber():
    bad = 'asm volatile("s_mov_b32 m0, %1\\n\\tglobal_load_lds_dword %0, off" ::"v"(p), "s"(l) : "memory");'
    good = bad.replace(': "memory")', ': "memory", "m0")')
    (sb,), (sg,) = _asm_statements(bad), _asm_statements(good)
    assert _writes_m0(sb) and '"m0"' not in sb.split(":")[-1]
    assert _writes_m0(sg) and '"m0"' in sg.split(":")[-1]
    assert not _writes_m0('asm volatile("" : "+v"(x));')


def test_no_hand_written_packed_fp32():
    for path in _sources():
        with open(path) as f:
            text = f.read()
        assert not re.search(r"v_pk_(add|mul|fma)_f32", text), os.path.basename(path)
