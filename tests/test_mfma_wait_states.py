"""Wait states around the logit GEMM's MFMAs, checked in the generated gfx950
assembly (CPU; needs hipcc).

The GEMM and the top-k tile-logits kernel issue v_mfma_f32_16x16x32_bf16 in
inline assembly (the compiler's builtin of that instruction copies its
accumulator between registers on most uses), so the compiler does not know
those instructions are MFMAs and inserts none of the wait states it would
insert around them.  The kernels supply their own (after zeroing the
accumulators, at the end of every K-loop iteration, before the epilogue);
this test checks, over every path of the control-flow graph, that

- a VALU write of a VGPR or AGPR comes at least 3 wait states before an MFMA
  reads it (as operand A, B or accumulator C),
- an MFMA's result is read by a non-MFMA instruction at least 11 wait states
  after the MFMA (the documented requirement for this 4-pass instruction is
  smaller; the margin covers an extra pass of latency),
- an accumulator an MFMA reads is not overwritten by a non-MFMA instruction
  within 4 wait states,

counting one wait state per instruction and n + 1 for `s_nop n`, with the
minimum distance over all paths into each basic block (a forward dataflow
iterated to its fixed point).  It also checks that no K loop copies an
accumulator (v_accvgpr_mov / _read / _write inside a loop with MFMAs would
mean the compiler moved one between registers).
"""

import os
import re
import subprocess

import pytest

from invariant_selected_token_amd import build as B

VALU_TO_MFMA = 3
MFMA_TO_READ = 11
SRCC_TO_WRITE = 4
CAP = 16   # above every limit below

REG = re.compile(r"\b([av])(?:\[(\d+):(\d+)\]|(\d+)\b)")
BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\.LBB\w+)")


def _regs(text):
    out = []
    for m in REG.finditer(text):
        if m.group(4) is not None:
            out.append((m.group(1), int(m.group(4))))
        else:
            out.extend((m.group(1), x) for x in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _functions(asm):
    names = re.findall(r"\.type\s+(\S+),@function", asm)
    for name in names:
        i = asm.find("\n" + name + ":")
        if i < 0:
            continue
        body = asm[i + 1:]
        yield name, body[: body.index(".Lfunc_end")]


def _blocks(body):
    """Basic blocks: list of (label or None, [instructions]), successor lists."""
    lines = []
    for raw in body.split("\n")[1:]:
        t = raw.split(";")[0].strip()
        if not t:
            continue
        if re.match(r"^\.LBB\w+:$", t) or (t.endswith(":") and t.startswith(".")):
            lines.append(("label", t[:-1]))
        elif t.startswith("."):
            continue
        else:
            lines.append(("inst", t))
    blocks, cur, label = [], [], None
    for kind, t in lines:
        if kind == "label":
            if cur or label is not None:
                blocks.append((label, cur))
            cur, label = [], t
            continue
        cur.append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append((label, cur))
            cur, label = [], None
    if cur or label is not None:
        blocks.append((label, cur))
    index = {lab: k for k, (lab, _) in enumerate(blocks) if lab is not None}
    succ = []
    for k, (_, insts) in enumerate(blocks):
        s = []
        last = insts[-1] if insts else ""
        m = BRANCH.match(last)
        if m and m.group(2) in index:
            s.append(index[m.group(2)])
        if not last.startswith(("s_branch", "s_endpgm", "s_setpc")) and k + 1 < len(blocks):
            s.append(k + 1)
        succ.append(s)
    return blocks, succ


def _check(name, body):
    """Violations as strings; also the count of accumulator moves in MFMA loops."""
    blocks, succ = _blocks(body)
    n = len(blocks)
    # state: three dicts register -> wait states since the event (min over paths)
    entry = [None] * n
    entry[0] = ({}, {}, {})
    bad = []

    def step(state, inst, report):
        valu_w, mfma_w, srcc_r = state
        mn = inst.split()[0]
        ops = [o.strip() for o in inst[len(mn):].split(",")] if len(inst) > len(mn) else []
        ws = int(ops[0], 0) + 1 if mn == "s_nop" else 1
        for d in (valu_w, mfma_w, srcc_r):
            for r in list(d):
                v = d[r] + ws
                if v >= CAP:
                    del d[r]   # past every limit: no longer a hazard on any path
                else:
                    d[r] = v
        if mn == "s_nop":
            return
        if mn.startswith("v_mfma"):
            dst, srcs = _regs(ops[0]), _regs(",".join(ops[1:3]))
            c = _regs(ops[3]) if len(ops) > 3 else []
            for r in srcs + c:
                if r in valu_w and valu_w[r] < VALU_TO_MFMA and report:
                    bad.append(f"{name}: {inst} reads {r} {valu_w[r]} wait states after a VALU write")
            for r in c:
                srcc_r[r] = 0
            for r in dst:
                mfma_w[r] = 0
                valu_w.pop(r, None)
            return
        is_store = "store" in mn or mn.startswith("ds_write")
        srcs = _regs(",".join(ops)) if is_store else _regs(",".join(ops[1:]))
        dsts = [] if is_store else (_regs(ops[0]) if ops else [])
        for r in srcs:
            if r[0] == "a" and r in mfma_w and mfma_w[r] < MFMA_TO_READ and report:
                bad.append(f"{name}: {inst} reads {r} {mfma_w[r]} wait states after an MFMA")
        for r in dsts:
            if r[0] == "a" and r in srcc_r and srcc_r[r] < SRCC_TO_WRITE and report:
                bad.append(f"{name}: {inst} overwrites {r} {srcc_r[r]} wait states after an MFMA read it")
            if mn.startswith("v_"):
                valu_w[r] = 0
                mfma_w.pop(r, None)
                srcc_r.pop(r, None)

    def merge(a, b):
        if a is None:
            return tuple(dict(x) for x in b)
        out = []
        for x, y in zip(a, b):
            z = dict(x)
            for r, v in y.items():
                z[r] = min(v, z.get(r, CAP))
            out.append(z)
        return tuple(out)

    changed = True
    while changed:
        changed = False
        for k in range(n):
            if entry[k] is None:
                continue
            st = tuple(dict(x) for x in entry[k])
            for inst in blocks[k][1]:
                step(st, inst, False)
            for s in succ[k]:
                m = merge(entry[s], st)
                if m != entry[s]:
                    entry[s] = m
                    changed = True
    for k in range(n):
        if entry[k] is None:
            continue
        st = tuple(dict(x) for x in entry[k])
        for inst in blocks[k][1]:
            step(st, inst, True)
    # accumulator moves inside loops that hold MFMAs (a back edge to an earlier block)
    moves = 0
    for k in range(n):
        for s in succ[k]:
            if s <= k:
                insts = [i for b in blocks[s:k + 1] for i in b[1]]
                if any(i.startswith("v_mfma") for i in insts) and _innermost(succ, s, k):
                    moves += sum(i.startswith("v_accvgpr") for i in insts)
    return bad, moves


def _innermost(succ, s, k):
    """True when no other back edge lies strictly inside [s, k] (an innermost loop)."""
    for j in range(s, k + 1):
        for t in succ[j]:
            if t <= j and (t, j) != (s, k) and s <= t and j <= k:
                return False
    return True


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    flags = [f for f in B.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [cc, *flags, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC,
           os.path.join(B.CSRC, "kernels.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_mfma_kernels_present(asm):
    names = [n for n, body in _functions(asm) if "v_mfma" in body]
    assert any("gemm_kernel" in n for n in names)
    assert any("tile_logits_kernel" in n for n in names)


def test_mfma_wait_states(asm):
    bad = []
    for name, body in _functions(asm):
        if "v_mfma" not in body:
            continue
        b, _ = _check(name, body)
        bad += b
    assert not bad, "\n".join(bad[:20])


def test_no_accumulator_copies_in_k_loops(asm):
    for name, body in _functions(asm):
        if "v_mfma" not in body:
            continue
        _, moves = _check(name, body)
        assert moves == 0, f"{name}: {moves} accumulator moves inside an MFMA loop"


def test_checker_catches_a_planted_hazard():
    """The checker itself: a VALU write right before an MFMA that reads it,
    and an MFMA result read at once, in a two-block function with a loop."""
    body = "\n".join([
        "f:",
        "\tv_accvgpr_write_b32 a0, 0",
        ".LBB0_1:",
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
        "\ts_cbranch_scc1 .LBB0_1",
        "\tv_accvgpr_read_b32 v8, a1",
        "\ts_endpgm",
    ])
    bad, _ = _check("f", body)
    assert any("after a VALU write" in x for x in bad)
    assert any("after an MFMA" in x and "reads" in x for x in bad)
    ok = body.replace("\tv_accvgpr_write_b32 a0, 0", "\tv_accvgpr_write_b32 a0, 0\n\ts_nop 4") \
             .replace("\tv_accvgpr_read_b32 v8, a1", "\ts_nop 7\n\ts_nop 7\n\tv_accvgpr_read_b32 v8, a1")
    bad, _ = _check("f", ok)
    assert not bad, bad
