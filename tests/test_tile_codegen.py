"""Generated-code check of the tile GEMM's hand-issued weight loads.

With LDS-DMA loads in flight the compiler waits for every outstanding load before the first use
of a register load, so the tile kernel issues its weight loads as instructions of its own and
orders them before their use with its per-stage vmcnt wait only.  Nothing in the compiler keeps
it from reading, copying or reusing such a destination register before that wait.  This test
compiles the GEMM source for gfx950 and walks the control-flow graph of every kernel from each of
those loads: on every path, no instruction may name the destination registers before an
`s_waitcnt vmcnt(n)` that the load has completed by (at least n vector memory instructions issued
after it on that path).  It needs hipcc (no GPU).
"""
import os
import re
import shutil
import subprocess

import pytest

from quantized_expert_layer_amd import build as qbuild

MARK = "; weight load"
VMEM = ("global_", "buffer_", "flat_", "scratch_")
BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\.L\w+)")
VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")


def _regs(text):
    out = set()
    for m in VREG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _functions(asm_lines):
    """Yield (name, [(opcode, operand text, raw line)], {label: index}) per kernel body."""
    name, body, labels = None, [], {}
    for raw in asm_lines:
        line = raw.rstrip()
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body, labels = m.group(1), [], {}
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            yield name, body, labels
            name = None
            continue
        s = line.strip()
        lm = re.match(r"^(\.L\w+):", s)
        if lm:
            labels[lm.group(1)] = len(body)
            continue
        if not s or s.startswith((";", ".", "//")):
            continue
        code = s.split(";", 1)[0].strip()
        op, _, rest = code.partition(" ")
        body.append((op, rest, s))


def _successors(body, labels, i):
    op, rest, _ = body[i]
    if op in ("s_endpgm", "s_setpc_b64", "s_trap"):
        return []
    m = BRANCH.match(f"{op} {rest}")
    if m:
        tgt = labels[m.group(2)]
        if op == "s_branch":
            return [tgt]
        return [tgt, i + 1] if i + 1 < len(body) else [tgt]
    return [i + 1] if i + 1 < len(body) else []


def _vmcnt(op, rest):
    if op != "s_waitcnt":
        return None
    m = re.search(r"vmcnt\((\d+)\)", rest)
    return int(m.group(1)) if m else None


def _check_load(body, labels, i):
    """Violations on paths from weight load i: instructions naming its registers too early."""
    dest = _regs(body[i][1].split(",")[0])
    bad = []
    seen = set()
    stack = [(j, 0) for j in _successors(body, labels, i)]
    while stack:
        j, after = stack.pop()
        key = (j, min(after, 64))
        if key in seen:
            continue
        seen.add(key)
        op, rest, raw = body[j]
        n = _vmcnt(op, rest)
        if n is not None and after >= n:
            continue                       # the load has completed on this path
        if j == i:
            bad.append((j, "the load is issued again before its wait"))
            continue
        if _regs(rest) & dest:
            bad.append((j, raw))
            continue
        if op.startswith(VMEM):
            after += 1
        stack.extend((k, after) for k in _successors(body, labels, j))
    return bad


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    src = os.path.join(qbuild.CSRC, "gemm.hip")
    flags = [f for f in qbuild.HIPCC_FLAGS if f not in ("-fPIC",)]
    subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", src, "-o", str(out)],
                   check=True, capture_output=True, timeout=600)
    return out.read_text().splitlines()


def test_weight_loads_are_not_touched_before_their_wait(gemm_asm):
    kernels = loads = 0
    problems = []
    for name, body, labels in _functions(gemm_asm):
        idx = [i for i, (_, _, raw) in enumerate(body) if MARK in raw]
        if not idx:
            continue
        kernels += 1
        loads += len(idx)
        for i in idx:
            for j, what in _check_load(body, labels, i):
                problems.append(f"{name}: load `{body[i][2]}` -> `{what}`")
    assert kernels > 0 and loads > 0, "no hand-issued weight loads found in the tile kernels"
    assert not problems, "\n".join(problems[:20])


def test_checker_flags_an_early_read():
    """The checker itself: a read of the destination before the wait is reported, a read after a
    wait the load has completed by is not, and a wait too shallow for the load does not count."""
    asm = [
        "_Zk:",
        "\tglobal_load_dwordx4 v[4:7], v[0:1], off ; weight load",
        "\tglobal_load_dwordx4 v[8:11], v[0:1], off",
        "\ts_waitcnt vmcnt(2)",
        "\tv_add_u32_e32 v12, v5, v12",
        "\ts_waitcnt vmcnt(1)",
        "\tv_add_u32_e32 v13, v6, v13",
        "\ts_endpgm",
        ".Lfunc_end0:",
    ]
    (name, body, labels), = list(_functions(asm))
    bad = _check_load(body, labels, 0)
    assert len(bad) == 1 and "v5" in bad[0][1]
    asm_ok = [a for a in asm if "v5" not in a]
    (name, body, labels), = list(_functions(asm_ok))
    assert _check_load(body, labels, 0) == []
