"""Checks on the gfx950 assembly of the flash kernels (CPU only: hipcc cross-compiles).

The tile copies of the bf16 kernels (absorbed prefill and decode, materialised prefill) are
written as inline asm (LDS-direct loads through M0) that the
compiler's wait tracking does not see; their correctness rests on properties of the
generated code that these tests pin:

* M0 is written only by those copy sequences (the asm clobbers M0, which the compiler
  does not preserve across it);
* no LDS-direct load carries a nonzero immediate offset (the offset would move the LDS
  destination as well as the source);
* no scratch (spill) access sits inside a tile loop that issues copies: the loop's hand
  placed vmcnt waits count only copies, and a spill reload there would also stall on
  every copy in flight.

The same copy properties are pinned for the Q8_0 decodes and the K + V^T decode.  The
split decode's score MFMAs are inline asm with VGPR accumulators, whose wait states the
compiler does not manage; the generated code must keep VALU writes away from their
sources and their results unread for 20 wait states after the last one.
"""
import os
import re
import shutil
import subprocess

import pytest

from deepseek_mla_amd import build as B

SRCS = [os.path.join(B.CSRC, f) for f in ("flash_mfma.hip", "decode_mfma.hip", "flash_mha.hip")]
BF16_KERNELS = ("flash_prefill_bf16_kernel", "flash_decode_kernelILb0E", "flash_mha_kernel")
# every kernel with LDS-direct tile copies: the bf16 ones, the Q8_0 split decode and the
# 128-head decodes (Q8_0, bf16, K + V^T)
COPY_KERNELS = BF16_KERNELS + ("flash_decode_kernelILb1E", "flash_decode_w_kernel")

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    texts = []
    for src in SRCS:
        out = d / (os.path.basename(src) + ".s")
        cmd = [B.HIPCC, *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S", src,
               "-o", str(out)]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        assert r.returncode == 0, r.stdout.decode(errors="replace")[-4000:]
        texts.append(out.read_text())
    return "\n".join(texts)


def kernel_bodies(text):
    """name -> list of instruction lines (label and comment lines kept for loop parsing)."""
    bodies, cur, name = {}, None, None
    for line in text.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, cur = m.group(1), []
            bodies[name] = cur
            continue
        if cur is not None:
            if line.strip().startswith(".Lfunc_end"):
                cur = None
                continue
            cur.append(line)
    return bodies


def bf16_bodies(text):
    b = {n: body for n, body in kernel_bodies(text).items() if any(k in n for k in BF16_KERNELS)}
    # the prefill in two forms (per-copy bounds, all tiles inside the cache) and the
    # materialised kernel in two shapes
    assert len(b) == 5, sorted(kernel_bodies(text))
    return b


def copy_bodies(text):
    b = {n: body for n, body in kernel_bodies(text).items() if any(k in n for k in COPY_KERNELS)}
    assert len(b) == 9, sorted(kernel_bodies(text))
    return b


def test_m0_written_only_by_copy_asm(asm):
    for name, body in copy_bodies(asm).items():
        in_asm = False
        for line in body:
            s = line.strip()
            if s.startswith(";;#ASMSTART"):
                in_asm = True
            elif s.startswith(";;#ASMEND"):
                in_asm = False
            elif not s.startswith(";") and re.search(r"\bm0\b", s):
                assert in_asm, f"{name}: compiler-generated M0 use: {s}"


def test_lds_loads_have_no_immediate_offset(asm):
    for line in asm.splitlines():
        s = line.strip()
        if s.startswith("global_load_lds") or s.startswith("buffer_load") and " lds" in s:
            m = re.search(r"offset:(0x[0-9a-fA-F]+|\d+)", s)
            assert m is None or int(m.group(1), 0) == 0, s


def test_no_spill_access_in_copy_loops(asm):
    for name, body in copy_bodies(asm).items():
        labels = {}
        for i, line in enumerate(body):
            m = re.match(r"^(\.LBB\w+):", line)
            if m:
                labels[m.group(1)] = i
        edges = []  # (header line, back-edge line) of every loop
        for i, line in enumerate(body):
            m = re.match(r"^\s*s_c?branch\w*\s+(\.LBB\w+)\s*$", line)
            if m and m.group(1) in labels and labels[m.group(1)] < i:
                edges.append((labels[m.group(1)], i))
        def instrs_of(h, e):
            return [l.strip() for l in body[h:e + 1]
                    if l.strip() and not l.strip().startswith((";", "."))]

        # tile loops: loops that issue copies and carry matrix work; the innermost of them
        # (an outer pass loop may spill around the tile loop)
        tile = [(h, e) for h, e in edges
                if any(x.startswith("global_load_lds") for x in instrs_of(h, e))
                and sum(x.startswith("v_mfma") for x in instrs_of(h, e)) >= 32]
        loops = 0
        for h, e in tile:
            if any(h <= h2 and e2 <= e and (h2, e2) != (h, e) for h2, e2 in tile):
                continue
            loops += 1
            spills = [x for x in instrs_of(h, e) if x.startswith("scratch_")]
            assert not spills, f"{name}: spill access in the tile loop: {spills[:3]}"
        assert loops >= 1, f"{name}: tile loop not found"


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def test_vgpr_accumulator_mfma_wait_states(asm):
    """In the split decode, around every MFMA that accumulates in VGPRs (the asm score
    MFMAs): no VALU instruction writes one of its sources in the 4 instructions before it,
    and no instruction other than an MFMA accumulating into the same registers reads or
    writes its result within 20 wait states after it (s_nop n counts n + 1)."""
    bodies = {n: b for n, b in kernel_bodies(asm).items() if "flash_decode_kernel" in n}
    assert len(bodies) == 2, sorted(bodies)
    for name, body in bodies.items():
        ins = []
        for line in body:
            t = line.split(";")[0].strip()
            if t and not t.startswith(".") and not t.endswith(":"):
                ins.append(t)
        found = 0
        for i, t in enumerate(ins):
            parts = t.split(None, 1)
            ops = [x.strip() for x in parts[1].split(",")] if len(parts) > 1 else []
            if not parts[0].startswith("v_mfma") or not ops or not ops[0].startswith("v"):
                continue
            found += 1
            dst = _vregs(ops[0])
            srcs = set().union(*[_vregs(x) for x in ops[1:4]])
            for j in range(max(0, i - 4), i):
                p = ins[j].split(None, 1)
                if p[0].startswith("v_") and not p[0].startswith("v_mfma") and len(p) > 1:
                    w = _vregs(p[1].split(",")[0].strip())
                    assert not (w & srcs), f"{name}: VALU write feeds an MFMA: {ins[j]} | {t}"
            ws = 0
            for j in range(i + 1, min(len(ins), i + 40)):
                p = ins[j].split(None, 1)
                if p[0] == "s_nop":
                    ws += int(p[1], 0) + 1
                    continue
                if ws >= 20:
                    break
                q = [x.strip() for x in p[1].split(",")] if len(p) > 1 else []
                used = set().union(*[_vregs(x) for x in q]) if q else set()
                if p[0].startswith("v_mfma"):
                    # a later MFMA may accumulate into exactly these registers (srcC = dst)
                    assert not (set().union(*[_vregs(x) for x in q[1:3]]) & dst), \
                        f"{name}: MFMA result used as a multiplicand: {t} | {ins[j]}"
                else:
                    assert not (used & dst), f"{name}: MFMA result touched after {ws} wait " \
                                             f"states: {t} | {ins[j]}"
                ws += 1
        assert found >= 36, f"{name}: {found} VGPR-accumulator MFMAs"
