"""Rules the HIP sources keep, checked on the text (CPU only).

An inline-asm vector load with a register output is unsafe: the compiler takes the output as
written when the asm statement ends and may copy or reuse the register before the load's data
arrives. The library's asm loads write LDS directly (no register output); register loads go
through compiler builtins, whose waits the compiler places itself."""
import os
import re

CSRC = os.path.join(os.path.dirname(__file__), "..", "mx_quantized_grouped_amd", "csrc")

_ASM = re.compile(r"\basm\s+(?:volatile\s*)?\((.*?)\)\s*;", re.S)


def _sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name)) as f:
                yield name, f.read()


def _asm_statements(text):
    return [m.group(1) for m in _ASM.finditer(text)]


def _outputs(stmt):
    """Constraint strings of the statement's output operands (the list after the first ':')."""
    parts = stmt.split(":")
    if len(parts) < 2:
        return []
    return re.findall(r'"(=[^"]*)"', parts[1])


def test_no_asm_load_with_register_output():
    bad = []
    for name, text in _sources():
        for stmt in _asm_statements(text):
            if re.search(r"\b(buffer|global|flat|scratch)_load", stmt) and _outputs(stmt):
                bad.append((name, stmt.split("\n")[0][:80]))
    assert not bad, bad


def test_checker_sees_asm_outputs():
    # the checker itself: a register-output load is found, an LDS-only load and a wait are not
    reg = 'asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x) : "v"(p));'
    lds = 'asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(o), "s"(r), "s"(s) : "m0");'
    wait = 'asm volatile("s_waitcnt vmcnt(0)" ::: "memory");'
    assert [bool(_outputs(s)) for s in _asm_statements(reg + lds + wait)] == [True, False, False]


def test_library_has_asm_loads_to_check():
    found = sum(1 for _, text in _sources() for stmt in _asm_statements(text) if "_load" in stmt)
    assert found >= 1
