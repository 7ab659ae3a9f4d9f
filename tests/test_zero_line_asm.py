"""The line-zeroing asm block of the fold (zero_line in leapq_fold.hip), read
from the source and run by a small interpreter of its scalar branch tree:
for every row pick (block p = 0..3), every column pick (entry m = 0..15 of
the owning wave) and no pick (-1), exactly the tile registers of that line
are selected to 0, each once, under the right lane mask (rows: the lanes
of the picked row; columns: the lane half of the picked column).  The tile
registers are the asm operands %0..%63 in the order S[p][m] -> 16 p + m.
CPU only: a change to the block that breaks the tree fails here before it
reaches a GPU."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "quantized_recurrent_state_amd", "csrc", "leapq_fold.hip")


def zero_line_asm():
    text = open(SRC).read()
    start = text.index("__device__ __forceinline__ void zero_line(")
    body = text[start:text.index("\n}\n", start)]
    asm = body[body.index("asm volatile(") + len("asm volatile("):]
    # the template: the string literals up to the first ':' outside them
    end, inside, i = None, False, 0
    while i < len(asm):
        ch = asm[i]
        if inside and ch == "\\":
            i += 2
            continue
        if ch == '"':
            inside = not inside
        elif ch == ":" and not inside:
            end = i
            break
        i += 1
    lits = re.findall(r'"((?:[^"\\]|\\.)*)"', asm[:end])
    code = "".join(lits).replace("\\n", "\n").replace("\\t", "\t")
    # the output operand list: "+v"(S[p][m]) in order
    outs = re.findall(r'"\+v"\(S\[(\d)\]\[(\d+)\]\)', body)
    return code, [(int(p), int(m)) for p, m in outs]


def parse(code):
    prog, labels = [], {}
    for raw in code.split("\n"):
        line = raw.strip()
        if not line:
            continue
        m = re.fullmatch(r"(\d+):", line)
        if m:
            labels.setdefault(int(m.group(1)), []).append(len(prog))
            continue
        op, *rest = line.split(None, 1)
        args = [a.strip() for a in rest[0].split(",")] if rest else []
        prog.append((op, args))
    return prog, labels


def run(prog, labels, pr, mm):
    """Returns [(operand, mask)] in execution order for scalar inputs pr, mm."""
    regs = {"%[pr]": pr, "%[mm]": mm}
    scc, pc, out, steps = False, 0, [], 0

    def target(ref):
        n, d = int(ref[:-1]), ref[-1]
        assert d == "f", "only forward local labels are expected"
        nxt = [i for i in labels[n] if i >= pc + 1]
        assert nxt, f"label {ref} not found after {pc}"
        return min(nxt)

    while pc < len(prog):
        steps += 1
        assert steps < 1000, "the branch tree does not end"
        op, a = prog[pc]
        if op == "s_cmp_lt_i32":
            scc = regs[a[0]] < int(a[1])
        elif op == "s_bitcmp1_b32":
            scc = bool((regs[a[0]] >> int(a[1])) & 1)
        elif op == "s_cbranch_scc1":
            if scc:
                pc = target(a[0])
                continue
        elif op == "s_branch":
            pc = target(a[0])
            continue
        elif op == "v_cndmask_b32_e64":
            dst, src0, src1, mask = a
            assert dst == src0 and src1 == "0", (op, a)
            out.append((int(dst[1:]), mask))
        else:
            raise AssertionError(f"unexpected instruction {op}")
        pc += 1
    return out


@pytest.fixture(scope="module")
def tree():
    code, outs = zero_line_asm()
    assert outs == [(p, m) for p in range(4) for m in range(16)], "operands %0..%63 are S[p][m] in order"
    return parse(code)


@pytest.mark.parametrize("pr", [-1, 0, 1, 2, 3])
@pytest.mark.parametrize("mm", [-1] + list(range(16)))
def test_zero_line_selects_exactly_the_line(tree, pr, mm):
    prog, labels = tree
    got = run(prog, labels, pr, mm)
    want = []
    if pr >= 0:
        want += [(16 * pr + m, "%[rl]") for m in range(16)]
    if mm >= 0:
        want += [(16 * p + mm, "%[cl]") for p in range(4)]
    assert sorted(got) == sorted(want), (pr, mm, got)
    assert len(set(o for o, _ in got)) == len(got) or (pr >= 0 and mm >= 0), "an operand selected twice"
