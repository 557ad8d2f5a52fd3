"""CPU guard on the inline assembly of the HIP sources.

The compiler's hazard recognizer does not look inside inline assembly.  A
VALU write of an SGPR (a v_readlane that reloads a spilled buffer
descriptor, say) needs 5 wait states before a vector memory instruction may
read that SGPR, and the compiler is free to place such a write right before
an asm block.  So every asm block that issues a vector memory instruction
(buffer_*, global_*, flat_*, scratch_*, including the direct-to-LDS loads)
must open with `s_nop 4` or longer.  This test parses csrc/ and fails on any
block that does not.
"""
import glob
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "hstu_sequential_transducer_causal_amd", "csrc")
VMEM = re.compile(r"^\s*(buffer_|global_|flat_|scratch_|tbuffer_)\w*")
NOP = re.compile(r"^\s*s_nop\s+(\d+)\s*$")


def _asm_blocks(text):
    """Yield (line number, template string) of every asm statement."""
    for m in re.finditer(r"\basm\s*(?:volatile\s*)?\(", text):
        i = m.end()
        depth, parts, cur, in_str, esc = 1, [], None, False, False
        while i < len(text) and depth:
            ch = text[i]
            if in_str:
                if esc:
                    esc = False
                elif ch == "\\":
                    esc = True
                elif ch == '"':
                    in_str = False
                    parts.append(cur)
                    cur = None
                    i += 1
                    continue
                cur += ch
            elif ch == '"':
                in_str, cur = True, ""
            elif ch == "(":
                depth += 1
            elif ch == ")":
                depth -= 1
            elif ch == ":" and depth == 1:
                break          # end of the template; operands follow
            i += 1
        line = text.count("\n", 0, m.start()) + 1
        yield line, "".join(parts).encode().decode("unicode_escape")


def violations(text, name="<text>"):
    out = []
    for line, tmpl in _asm_blocks(text):
        insts = [s.strip() for s in re.split(r"[\n;]", tmpl.replace("\t", " ")) if s.strip()]
        if not any(VMEM.match(s) for s in insts):
            continue
        first = NOP.match(insts[0])
        if not first or int(first.group(1)) < 4:
            out.append(f"{name}:{line}: vector memory asm block must open with s_nop 4: {tmpl!r}")
    return out


def test_every_vmem_asm_block_opens_with_wait_states():
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
    assert files
    bad, nblocks = [], 0
    for f in files:
        text = open(f).read()
        nblocks += sum(1 for _ in _asm_blocks(text))
        bad += violations(text, os.path.basename(f))
    assert nblocks > 0
    assert not bad, "\n".join(bad)


def test_checker_flags_a_block_without_the_wait_states():
    good = 'asm volatile("s_nop 4\\n\\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(a), "s"(r), "s"(o));'
    short = 'asm volatile("s_nop 1\\n\\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(a), "s"(r));'
    none = 'asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(a), "s"(r));'
    split = 'asm volatile("s_waitcnt vmcnt(0)\\n\\t"\n  "global_load_dword %0, %1, off" : "=v"(x) : "v"(p));'
    not_mem = 'asm volatile("s_waitcnt lgkmcnt(0)\\n\\ts_barrier" ::: "memory");'
    assert violations(good) == []
    assert violations(not_mem) == []
    assert len(violations(short)) == 1
    assert len(violations(none)) == 1
    assert len(violations(split)) == 1
