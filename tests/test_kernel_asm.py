"""The decode kernel's QK waves issue their row loads from inline assembly and wait for them
with explicit counts; the compiler does not know those registers fill asynchronously.  This
CPU test compiles the kernel to gfx950 assembly and checks, for every such load block in the
QK waves' loop, that no instruction touches its destination registers between the block and
the first matrix instruction that consumes them (scanning the loop body cyclically), and that
an explicit wait sits in that window.  A copy or reuse of those registers while a load is in
flight would read or clobber data that has not landed (the failure this guards against: a row
address built from such a copy)."""
import os
import re
import subprocess
import tempfile

import pytest

from sparse_mla_attention_amd import build

SRC = os.path.join(build.CSRC, "smla_decode.hip")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return (parts[0] if parts else ""), set(), set()
    op, ops = parts[0], [o.strip() for o in parts[1].split(",")]
    if op.startswith(("ds_write", "global_store", "buffer_store", "s_")):
        src = set()
        for o in ops:
            src |= _regs(o.split()[0])
        return op, set(), src
    dst = _regs(ops[0].split()[0])
    src = set()
    for o in ops[1:]:
        src |= _regs(o.split()[0])
    return op, dst, src


def _blocks(lines):
    """(label, first line, end line, comment) of every basic block, in layout order."""
    starts = [i for i, l in enumerate(lines)
              if re.match(r"^(\.LBB\S+:|; %bb\.\d+:)", l)]
    out = []
    for k, i in enumerate(starts):
        end = starts[k + 1] if k + 1 < len(starts) else len(lines)
        lab = lines[i].split(":")[0].strip().lstrip(";").strip()
        # ".LBB0_20" is annotated as "Header=BB0_20"
        out.append((lab[2:] if lab.startswith(".L") else lab, i, end, lines[i]))
    return out


def _asm_loop(body):
    """The lines of the loop that holds the inline-assembly row loads: its header block and
    every block the compiler annotates as in that loop (or in a loop nested in it), in layout
    order (a rotated loop may place its latch before the header)."""
    lines = body.split("\n")
    blocks = _blocks(lines)
    for lab, i, end, head in blocks:
        if "Loop Header" not in head:
            continue
        members = {lab}
        grew = True
        while grew:
            grew = False
            for name, _, _, c in blocks:
                m = re.search(r"Header=(\S+)", c)
                if name not in members and m and m.group(1) in members:
                    members.add(name)
                    grew = True
        seg = []
        for l2, a, b, c in blocks:
            if l2 in members:
                seg.extend(lines[a:b])
        if any("ASMSTART" in x for x in seg) and any("global_load_dwordx4" in x for x in seg):
            return seg
    return None


def _check(body):
    seg = _asm_loop(body)
    assert seg is not None, "no loop with inline-assembly row loads"
    ins, in_asm = [], False
    for l in seg:
        s = l.strip()
        if "ASMSTART" in s:
            in_asm = True
            ins.append(("start", s))
        elif "ASMEND" in s:
            in_asm = False
            ins.append(("end", s))
        elif s and not s.startswith((";", ".")):
            ins.append(("asm" if in_asm else "cc", s))
    n, blocks, problems = len(ins), 0, []
    i = 0
    while i < n:
        if ins[i][0] == "start" and i + 1 < n and "global_load" in ins[i + 1][1]:
            d, j = set(), i + 1
            while ins[j][0] != "end":
                d |= _regs(ins[j][1].split()[1].rstrip(","))
                j += 1
            blocks += 1
            waited, k = False, (j + 1) % n
            for _ in range(n):
                kind, s = ins[k]
                if kind == "asm" and s.startswith("s_waitcnt vmcnt"):
                    waited = True
                elif kind == "asm" and "global_load" in s and _regs(s.split()[1].rstrip(",")) & d:
                    problems.append("reloaded before use: " + s)
                    break
                elif kind == "cc":
                    op, dst, src = _operands(s)
                    if op.startswith("v_mfma") and src & d:
                        if not waited:
                            problems.append("consumed before its wait: " + s)
                        break
                    if (dst | src) & d:
                        problems.append("touched in flight: " + s)
                k = (k + 1) % n
            i = j
        i += 1
    return blocks, problems


def test_async_row_loads_are_never_touched_in_flight():
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "decode.s")
        cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(r.stdout + r.stderr)
        text = open(out).read()
    # a kernel's body runs to its end label (an early return puts an s_endpgm before the loop)
    kernels = re.findall(r"^(_ZN\S*decode_kernel\S*):[^\n]*\n(.*?)^\.Lfunc_end", text,
                         re.S | re.M)
    assert len(kernels) == 6  # 3 row shapes x one/two-term P
    for name, body in kernels:
        blocks, problems = _check(body)
        assert blocks == 3, name
        assert not problems, (name, problems[:5])
    # the same kernels spill nothing (the compiler's waits for a spill reload do not know the
    # row loads in flight, so they would drain them)
    assert not re.search(r"\.vgpr_spill_count:\s+[1-9]", text)


def test_decode_kernels_spill_nothing():
    """Neither decode kernel spills registers: a spill reload's wait would also drain the row
    loads in flight, and scratch traffic would sit on the gather's memory path."""
    for src in ("smla_decode.hip", "smla_decode_g64.hip"):
        with tempfile.TemporaryDirectory() as tmp:
            out = os.path.join(tmp, "k.s")
            cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S",
                   os.path.join(build.CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                pytest.fail(r.stdout + r.stderr)
            text = open(out).read()
        counts = re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)
        assert counts, src
        assert all(int(c) == 0 for c in counts), (src, counts)


def test_pv_matrix_sequences_have_no_branches():
    """The 64-head kernel's P.V waves issue their matrix instructions as straight-line code
    (no branch or block boundary between neighbouring products), so the explicit pad before the
    accumulators' rescale is the one distance between a chunk's products and their reads that
    the schedule can change."""
    src = os.path.join(build.CSRC, "smla_decode_g64.hip")
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "g64.s")
        cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(r.stdout + r.stderr)
        text = open(out).read()
    kernels = re.findall(r"^(_ZN\S*decode_g64_kernel\S*):[^\n]*\n(.*?)^\.Lfunc_end", text,
                         re.S | re.M)
    assert kernels
    for name, body in kernels:
        ins = [l.strip() for l in body.split("\n")
               if l.strip() and not l.strip().startswith(";")]
        # the P.V products: FP8 on E4M3 rows, BF16 on 656-byte fp8_ds_mla rows
        idx = [i for i, l in enumerate(ins)
               if l.startswith(("v_mfma_scale_f32_32x32x64", "v_mfma_f32_32x32x16_bf16"))]
        assert idx, name
        for a, b in zip(idx, idx[1:]):
            if b - a < 12:
                seg = ins[a + 1:b]
                assert not any(s.startswith("s_cbranch") or s.endswith(":") for s in seg), \
                    (name, ins[a:b + 1])
