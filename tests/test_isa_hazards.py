"""The dK/dV kernel accumulates dK and dV with an MFMA written as inline
assembly (so that the sums stay in the accumulation registers), which the
compiler does not recognise as an MFMA: it inserts no wait states around it.
The kernel is written so that none are needed; this test checks that claim
on the code the compiler actually emits for gfx950 (every instantiation of
dkdv_kernel, compiled with the library's own flags):

* no instruction other than another such MFMA (accumulating in place) reads
  or writes an accumulator register within 20 issue slots after an inline
  MFMA wrote it (an 8-pass XDL result needs about 11 before a vector read);
* no vector instruction writes a register that an inline MFMA reads as an
  operand within the 2 wait states before it;
* inside the hot step loop, nothing but the inline MFMAs touches the
  accumulation registers at all.

Runs on the CPU (hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess

import pytest

from head_chunked_context_amd import build as hb

pytestmark = pytest.mark.skipif(shutil.which(hb.HIPCC) is None and not os.path.exists(hb.HIPCC),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("isa") / "bwd.s")
    cmd = [hb.HIPCC] + hb.COMMON + hb.FLAGS.get("bwd.hip", []) + \
        ["--offload-device-only", "-S", "-x", "hip", os.path.join(hb.CSRC, "bwd.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read().split("\n")


def kernels(lines):
    """{name: [lines]} of every dkdv_kernel instantiation."""
    out, cur, name = {}, None, None
    for l in lines:
        m = re.match(r"^(_ZN2hc11dkdv_kernel\w+):", l)
        if m:
            name, cur = m.group(1), []
        if cur is not None:
            cur.append(l)
            if l.startswith(".Lfunc_end"):
                out[name] = cur
                cur = None
    return out


def regs(tok):
    """set of (file, index) registers named by an operand token"""
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def instructions(body):
    """(line index, opcode, operands, inside inline asm) for each instruction"""
    inasm = False
    for i, l in enumerate(body):
        t = l.strip()
        if t.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if t.startswith(";;#ASMEND"):
            inasm = False
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        yield i, parts[0], ops, inasm


def slots(op, ops):
    return int(ops[0]) + 1 if op == "s_nop" else 1


def hot_loop(body):
    """line range of the innermost loop holding the most MFMAs"""
    best = None
    for i, l in enumerate(body):
        if "Inner Loop Header" not in l:
            continue
        j = i
        while not re.match(r"^\.LBB\d+_\d+:", body[j]):
            j -= 1
        label = re.match(r"^\.L(BB\d+_\d+):", body[j]).group(1)
        last = max(k for k, x in enumerate(body) if ("Header=" + label + " ") in x)
        k = last + 1
        while k < len(body) and not body[k].startswith(".LBB") and not body[k].startswith("; %bb"):
            k += 1
        n = sum(1 for x in body[j:k] if "v_mfma" in x)
        if best is None or n > best[0]:
            best = (n, j, k)
    return best


def test_every_dkdv_instantiation_is_compiled(isa):
    ks = kernels(isa)
    # HD in {64, 128} x die-aware order x group loop
    assert len(ks) == 8, sorted(ks)


def early_reads(name, body):
    """accesses of an inline MFMA's accumulator within 20 slots of its write"""
    bad, recent, slot = [], [], 0   # (slot of the write, registers written)
    for i, op, ops, inasm in instructions(body):
        inline_mfma = inasm and op.startswith("v_mfma")
        touched = set()
        for o in ops:
            touched |= {r for r in regs(o) if r[0] == "a"}
        for w, rs in recent:
            if touched & rs and slot - w < 20:
                if inline_mfma and regs(ops[0]) == rs and regs(ops[3]) == rs:
                    continue  # the next accumulation into the same registers
                bad.append((name, i, body[i].strip(), slot - w))
        if inline_mfma:
            w = regs(ops[0])
            recent = [r for r in recent if not (r[1] & w)] + [(slot, w)]
        slot += slots(op, ops)
        recent = [r for r in recent if slot - r[0] < 20]
    return bad


def late_operands(name, body):
    """vector writes of an inline MFMA's operands in the 2 wait states before it"""
    bad, hist, slot = [], [], 0     # (slot of the write, registers written by VALU)
    for i, op, ops, inasm in instructions(body):
        if inasm and op.startswith("v_mfma"):
            read = regs(ops[1]) | regs(ops[2]) | regs(ops[3])
            for w, rs in hist:
                if read & rs and slot - w < 3:
                    bad.append((name, i, body[i].strip(), slot - w))
        if op.startswith("v_") and not op.startswith("v_mfma") and ops:
            hist.append((slot, regs(ops[0])))
        slot += slots(op, ops)
        hist = [h for h in hist if slot - h[0] < 3]
    return bad


# the checks themselves must see a hazard: hand-written bodies with one each
_MFMA = ["\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]", "\t;;#ASMEND"]


def test_checks_catch_planted_hazards():
    read_soon = _MFMA + ["\ts_nop 7", "\tv_accvgpr_read_b32 v8, a3"]
    assert early_reads("k", read_soon)
    assert not early_reads("k", _MFMA + ["\ts_nop 7"] * 3 + ["\tv_accvgpr_read_b32 v8, a3"])
    chained = _MFMA + ["\tv_add_u32_e32 v9, v9, v9"] + _MFMA
    assert not early_reads("k", chained)
    written_late = ["\tv_cvt_pk_bf16_f32 v5, v1, v2"] + _MFMA
    assert late_operands("k", written_late)
    assert not late_operands("k", ["\tv_cvt_pk_bf16_f32 v5, v1, v2", "\ts_nop 1"] + _MFMA)


def test_inline_mfma_results_are_not_read_early(isa):
    bad = [b for name, body in kernels(isa).items() for b in early_reads(name, body)]
    assert not bad, bad[:10]


def test_inline_mfma_operands_are_not_written_just_before(isa):
    bad = [b for name, body in kernels(isa).items() for b in late_operands(name, body)]
    assert not bad, bad[:10]


def test_hot_loop_moves_no_accumulator(isa):
    for name, body in kernels(isa).items():
        n, a, b = hot_loop(body)
        # most of a step's MFMAs (32 at D = 64, 64 at D = 128; the compiler
        # may rotate a few of them out of the loop's blocks)
        assert n >= (24 if "ILi64E" in name else 48), (name, n)
        moved = [l.strip() for l in body[a:b] if "v_accvgpr" in l or "scratch_" in l]
        assert not moved, (name, moved[:5])
