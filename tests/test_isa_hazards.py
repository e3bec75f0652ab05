"""MFMA data hazards in the decode kernel's generated gfx950 code.

The decode kernel issues its matrix products as inline asm (so that the
compiler keeps their order and register classes), which also means the
compiler does not insert the wait states the hardware needs around them.  This
test compiles the kernel to assembly and checks, along every control-flow
path, the rules the kernel relies on (CDNA3/CDNA4 ISA, dependency rules for
MFMA):
  * a VALU instruction that writes a register an MFMA reads (A, B or C
    operand) is at least 2 wait states ahead of the product;
  * a non-MFMA instruction that reads or writes a register an MFMA writes is
    at least 18 wait states behind the product (an MFMA counts as one wait
    state here, far below what it really takes);
  * an MFMA reads another product's result only as its accumulator, over
    exactly the same registers.
Wait states: one per instruction, N + 1 for s_nop N.  CPU only (cross-compiles).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "head_latent_attention_absorb_amd", "csrc", "decode_mfma.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

VALU_TO_MFMA = 2
MFMA_TO_OTHER = 18

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")


def regs(op):
    out = set()
    for m in REG.finditer(op):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def split_ops(text):
    parts, depth, cur = [], 0, ""
    for ch in text:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            parts.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        parts.append(cur.strip())
    return parts


class Inst:
    def __init__(self, mnem, ops):
        self.mnem = mnem
        self.ops = ops
        self.is_mfma = mnem.startswith("v_mfma")
        self.is_valu = mnem.startswith("v_") and not self.is_mfma
        self.writes, self.reads = set(), set()
        if self.is_mfma:
            self.writes = regs(ops[0])
            self.src_ab = regs(ops[1]) | regs(ops[2])
            self.src_c = regs(ops[3]) if len(ops) > 3 else set()
            self.reads = self.src_ab | self.src_c
        elif self.is_valu or mnem.startswith(("ds_read", "ds_load", "global_load", "buffer_load")):
            if mnem.startswith(("global_load_lds", "buffer_load")) and "lds" in mnem:
                self.reads = set().union(*(regs(o) for o in ops)) if ops else set()
            elif ops:
                self.writes = regs(ops[0])
                self.reads = set().union(*(regs(o) for o in ops[1:])) if len(ops) > 1 else set()
        else:
            self.reads = set().union(*(regs(o) for o in ops)) if ops else set()
        m = re.match(r"s_nop\s*$", mnem)
        self.wait = int(ops[0], 0) + 1 if m and ops else 1


def parse_kernels(asm):
    """-> {kernel name: list of items}; an item is ('label', name) or ('inst', Inst)."""
    kernels, cur, name = {}, None, None
    for line in asm.splitlines():
        line = line.split(";")[0].rstrip()
        if not line.strip():
            continue
        m = re.match(r"^(_Z\w*decode_mfma_kernel\w*):", line)
        if m:
            name, cur = m.group(1), []
            kernels[name] = cur
            continue
        if cur is None:
            continue
        if re.match(r"^\.Lfunc_end", line):
            cur, name = None, None
            continue
        m = re.match(r"^(\.?\w+):\s*$", line)
        if m:
            cur.append(("label", m.group(1)))
            continue
        s = line.strip()
        if s.startswith("."):
            continue
        mnem, _, rest = s.partition(" ")
        cur.append(("inst", Inst(mnem, split_ops(rest))))
    return kernels


def cfg_edges(items):
    labels = {it[1]: i for i, it in enumerate(items) if it[0] == "label"}
    succ = []
    for i, it in enumerate(items):
        nxt = [i + 1] if i + 1 < len(items) else []
        if it[0] == "inst":
            mn = it[1].mnem
            if mn == "s_endpgm":
                nxt = []
            elif mn.startswith("s_branch"):
                nxt = [labels[it[1].ops[0]]]
            elif mn.startswith("s_cbranch"):
                nxt = nxt + [labels[it[1].ops[0]]]
        succ.append(nxt)
    pred = [[] for _ in items]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return succ, pred


def walk(items, edges, start, limit, visit):
    """Visit (index, wait states strictly between start and it) along edges
    while fewer than `limit` wait states separate them."""
    best = {}
    stack = [(j, 0) for j in edges[start]]
    while stack:
        i, ws = stack.pop()
        if ws >= limit or best.get(i, limit) <= ws:
            continue
        best[i] = ws
        it = items[i]
        if it[0] == "inst":
            visit(it[1], ws)
            ws += it[1].wait
        stack.extend((j, ws) for j in edges[i])


def check(items):
    succ, pred = cfg_edges(items)
    problems = []
    for k, it in enumerate(items):
        if it[0] != "inst" or not it[1].is_mfma:
            continue
        m = it[1]

        def back(inst, ws, m=m, k=k):
            if inst.is_valu and inst.writes & m.reads:
                problems.append(f"VALU {inst.mnem} {inst.ops} writes a source of "
                                f"{m.mnem} {m.ops} with {ws} wait states between")
        walk(items, pred, k, VALU_TO_MFMA, back)

        def fwd(inst, ws, m=m):
            if inst.is_mfma:
                if inst.src_ab & m.writes:
                    problems.append(f"{inst.mnem} {inst.ops} reads the result of {m.ops} as A/B")
                if inst.src_c & m.writes and inst.src_c != m.writes:
                    problems.append(f"{inst.mnem} {inst.ops} partly overlaps the result of {m.ops}")
                return
            if (inst.reads | inst.writes) & m.writes:
                problems.append(f"{inst.mnem} {inst.ops} touches the result of {m.mnem} "
                                f"{m.ops} {ws} wait states after it")
        walk(items, succ, k, MFMA_TO_OTHER, fwd)
    return problems


@pytest.fixture(scope="module")
def kernels():
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from head_latent_attention_absorb_amd.build import FLAGS
    r = subprocess.run([HIPCC, *FLAGS, "--cuda-device-only", "-S", SRC, "-o", "-"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    ks = parse_kernels(r.stdout)
    # 128-row groups: contiguous / paged x (bf16 / low-bit rows) split
    # partials, and contiguous / paged bf16 direct; 64-row groups: contiguous
    # / paged bf16 x (partials, direct)
    assert len(ks) == 10, sorted(ks)
    return ks


def test_decode_kernel_has_no_mfma_hazards(kernels):
    for name, items in kernels.items():
        n_mfma = sum(1 for it in items if it[0] == "inst" and it[1].is_mfma)
        assert n_mfma > 60, name  # the 64-row form issues 18 + 34 + 16
        problems = check(items)
        assert not problems, f"{name}:\n" + "\n".join(problems[:20])


def test_checker_catches_planted_hazards():
    """A VALU write right in front of a product, a VALU read right behind one,
    and a product reading another's result as A: all three are reported."""
    asm = """
_Z18decode_mfma_kernelILb0EEvv:
\tv_mov_b32 v4, v0
\tv_mfma_f32_32x32x16_bf16 v[10:25], v[4:7], v[30:33], v[10:25]
\tv_add_f32 v1, v10, v2
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[12:15], v[30:33], a[0:15]
\ts_nop 7
\ts_nop 7
\ts_nop 3
\tv_mov_b32 v2, v40
\ts_nop 0
\ts_nop 0
\tv_mfma_f32_32x32x16_bf16 a[16:31], v[40:43], v[2:5], a[16:31]
\ts_endpgm
.Lfunc_end0:
"""
    items = parse_kernels(asm)["_Z18decode_mfma_kernelILb0EEvv"]
    problems = check(items)
    assert any("v_mov_b32" in p and "writes a source" in p for p in problems)
    assert any("v_add_f32" in p and "touches the result" in p for p in problems)
    assert any("as A/B" in p for p in problems)
    # The third product is preceded by a VALU write with exactly 2 wait states
    # between: allowed.
    assert not any("'v2'" in p and "v[40:43]" in p for p in problems)
