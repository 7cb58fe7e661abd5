"""Invariants of the generated gfx950 code of the 384-row (tall) tiles (CPU only:
hipcc cross-compiles the kernels to assembly, nothing runs).

The tall kernels keep a third of their MFMA accumulators in VGPRs and issue
those MFMAs as inline assembly, which the compiler does not look inside.  The
hazard rules they rely on hold only if, in every basic block that holds such
MFMAs, no other instruction reads or writes the accumulator registers (the
compiler could otherwise copy them right after the MFMA that writes them),
and if the wait before the epilogue's first read is present.  A K-loop block
must also hold no scratch access: a scratch reload waits for every operand load
in flight.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_forward_amd", "csrc")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


pytestmark = pytest.mark.skipif(hipcc() is None, reason="hipcc not found")


def regs(txt):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", txt):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def kernels(asm):
    """(name, list of basic blocks (lists of instructions)) of every kernel that
    runs tall tiles."""
    for m in re.finditer(r"^(_Z\w*(?:tall|fused|k_grads)\w*):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        blocks, cur = [], []
        for line in asm[m.end():end].split("\n"):
            t = line.strip()
            if re.match(r"^\.LBB\w+:", t) or t.startswith("; %bb."):
                blocks.append(cur)
                cur = []
            t = t.split(";")[0].strip()
            if t:
                cur.append(t)
        blocks.append(cur)
        yield m.group(1), blocks


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in ("cce_forward.hip", "cce_backward.hip"):
        s = str(d / (src + ".s"))
        cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
               "--cuda-device-only", "-S", "-o", s, os.path.join(CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[src] = open(s).read()
    return out


def test_vgpr_accumulators_are_touched_only_by_their_mfmas(assembly):
    seen = 0
    for src, asm in assembly.items():
        for name, blocks in kernels(asm):
            for b in blocks:
                acc = set()
                for t in b:
                    if t.startswith("v_mfma"):
                        dst = t.split(None, 1)[1].split(",")[0].strip()
                        if dst.startswith("v"):
                            acc |= regs(dst)
                if not acc:
                    continue
                seen += 1
                bad = [t for t in b if not t.startswith("v_mfma") and not t.startswith("s_")
                       and regs(t) & acc]
                assert not bad, f"{name}: {bad[:3]}"
    # forward (2 kernels), recompute (4), fused (4) and k_grads (1) run tall K loops
    assert seen >= 40


def test_epilogue_waits_for_the_vgpr_mfmas(assembly):
    for src, asm in assembly.items():
        for name, blocks in kernels(asm):
            text = "\n".join("\n".join(b) for b in blocks)
            if not re.search(r"v_mfma\w* v\[", text):
                continue
            # the drain: three s_nop 7 (24 wait states) in one assembly statement
            assert re.search(r"s_nop 7\s+s_nop 7\s+s_nop 7", text), name


def test_no_scratch_in_mfma_blocks(assembly):
    for src, asm in assembly.items():
        for name, blocks in kernels(asm):
            for b in blocks:
                if any(t.startswith("v_mfma") for t in b):
                    assert not any("scratch_" in t for t in b), name
