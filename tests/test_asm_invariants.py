"""Invariants of the generated gfx950 code of the 384-row (tall) tiles and of the
forward's 64-wide K-slice loop (CPU only: hipcc cross-compiles the kernels to
assembly, nothing runs).

The tall kernels keep a third of their MFMA accumulators in VGPRs and issue
those MFMAs as inline assembly, which the compiler does not look inside.  The
hazard rules they rely on hold only if, in every basic block that holds such
MFMAs, no other instruction reads or writes the accumulator registers (the
compiler could otherwise copy them right after the MFMA that writes them),
and if the wait before the epilogue's first read is present; and no VALU
instruction may write one of their source registers in the two issue slots
before them.  A K-loop block
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


def accumulator_touches(assembly):
    """(blocks with VGPR-accumulator MFMAs, offending instructions)."""
    seen, bad = 0, []
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
                bad += [(name, t) for t in b if not t.startswith("v_mfma")
                        and not t.startswith("s_") and regs(t) & acc]
    return seen, bad


def test_vgpr_accumulators_are_touched_only_by_their_mfmas(assembly):
    seen, bad = accumulator_touches(assembly)
    assert not bad, bad[:3]
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


def instructions(asm):
    """(name, instruction list, label -> index) of every tall kernel, in program order."""
    for m in re.finditer(r"^(_Z\w*(?:tall|fused|k_grads)\w*):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        ins, labels = [], {}
        for line in asm[m.end():end].split("\n"):
            t = line.split(";")[0].strip()
            if not t:
                continue
            if re.match(r"^\.LBB\w+:$", t):
                labels[t[:-1]] = len(ins)
                continue
            if t.startswith("."):
                continue
            ins.append(t)
        yield m.group(1), ins, labels


def is_valu_write(t):
    return t.startswith("v_") and not t.startswith(
        ("v_mfma", "v_accvgpr_write", "v_readfirstlane", "v_readlane", "v_cmp"))


def source_hazards(assembly):
    """(assembly MFMAs checked, those with a VALU write of a source register in
    the 2 issue slots before them, following branches into their block)."""
    checked, bad = 0, []
    for src, asm in assembly.items():
        for name, ins, labels in instructions(asm):
            preds = {}
            for j, t in enumerate(ins):
                mm = re.match(r"s_(?:cbranch_\w+|branch) (\.LBB\w+)", t)
                if mm and mm.group(1) in labels:
                    preds.setdefault(labels[mm.group(1)], []).append(j)

            def clean(pos, srcregs, ws):
                j = pos - 1
                while j >= 0 and ws < 2:
                    p = ins[j]
                    if p.startswith("s_nop"):
                        ws += int(p.split()[1]) + 1
                    else:
                        if is_valu_write(p) and regs(p.split(None, 1)[1].split(",")[0]) & srcregs:
                            return False
                        ws += 1
                    j -= 1
                return True

            for i, t in enumerate(ins):
                if not t.startswith("v_mfma"):
                    continue
                ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
                if not ops[0].startswith("v"):
                    continue
                checked += 1
                srcregs = regs(ops[1]) | regs(ops[2]) | regs(ops[3])
                if not clean(i, srcregs, 0):
                    bad.append((name, t))
                for pos, js in preds.items():
                    if 0 <= i - pos < 2:
                        bad += [(name, t + " (branch)") for j in js
                                if not clean(j + 1, srcregs, i - pos)]
    return checked, bad


def test_no_valu_write_just_before_an_assembly_mfma_reads_it(assembly):
    """A VALU write of a VGPR needs 2 wait states before an MFMA reads it; the
    compiler does not count them for the MFMAs written as assembly."""
    checked, bad = source_hazards(assembly)
    assert not bad, bad[:3]
    assert checked >= 500


SYNTH = """_ZN3cce9k_fwd_tallE:
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[130:133], v[134:137], a[0:15]
\tv_mov_b32_e32 v140, v1
\tv_mfma_f32_32x32x16_bf16 v[2:17], v[138:141], v[134:137], v[2:17]
\ts_cbranch_scc1 .LBB0_2
.LBB0_1:
\tv_mfma_f32_32x32x16_bf16 v[18:33], v[130:133], v[134:137], v[18:33]
\tv_add_u32_e32 v20, 1, v20
.LBB0_2:
\tv_mov_b32_e32 v131, 0
\ts_branch .LBB0_3
.LBB0_3:
\tv_mfma_f32_32x32x16_bf16 v[34:49], v[130:133], v[142:145], v[34:49]
.Lfunc_end0:
"""


def test_checks_catch_planted_mistakes():
    """The checks themselves, on hand-written assembly with planted mistakes: an
    accumulator register written in the block of its MFMA (v20 in v[18:33]), a VALU write of
    a source register one slot before an MFMA (v140), and one that reaches the
    MFMA through a branch (v131)."""
    seen, bad = accumulator_touches({"synth": SYNTH})
    assert seen == 3 and [t for _, t in bad] == ["v_add_u32_e32 v20, 1, v20"]
    checked, bad = source_hazards({"synth": SYNTH})
    assert checked == 3
    msgs = [t for _, t in bad]
    assert any("v[138:141]" in t for t in msgs)
    assert any("v[142:145]" in t and "branch" in t for t in msgs)


def test_no_scratch_in_mfma_blocks(assembly):
    for src, asm in assembly.items():
        for name, blocks in kernels(asm):
            for b in blocks:
                if any(t.startswith("v_mfma") for t in b):
                    assert not any("scratch_" in t for t in b), name


def test_no_scratch_in_the_forward_64_wide_k_loop(assembly):
    """The forward's 64-wide K-slice loop (256x256 tiles; in every k_fwd built
    for aligned operands without a K tail, the only block with 128 MFMAs) holds
    no scratch access either."""
    asm = assembly["cce_forward.hip"]
    seen = 0
    for m in re.finditer(r"^(_Z\w*k_fwdILb1ELb0E\w*):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        for b in re.split(r"\n(?=\.LBB\w+:)", asm[m.end():end]):
            lines = [t.split(";")[0].strip() for t in b.split("\n")]
            if sum(t.startswith("v_mfma") for t in lines) >= 128:
                seen += 1
                assert not any("scratch_" in t for t in lines), m.group(1)
    assert seen >= 8
