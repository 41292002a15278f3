"""Guard on the decode kernel's generated code (CPU only: compiles to gfx950
assembly with the library's flags, reads no GPU).

The kernel issues LDS operand reads from inline assembly and waits for them
with separate statements (s_waitcnt lgkmcnt(N)), so the compiler does not
know those registers are being written in the background.  This test walks
each kernel's instruction stream and checks that no instruction touches a
register of a read that is still in flight: LDS reads complete in order, so
after lgkmcnt(N) every LDS read except the newest N has landed.

The MFMAs are inline assembly too, so the compiler's hazard recognizer does
not see them either; the walk also checks the two MFMA data hazards the
kernel has to cover by hand (counted in wait states: one per instruction,
N + 1 for s_nop N):
  * a VALU write of a register an MFMA then reads needs 2 wait states;
  * an MFMA result read or overwritten by anything but the next MFMA of the
    same accumulation needs 12 after a 32x32x16 bf16 MFMA and 20 after a
    32x32x64 e4m3 one (what the compiler itself inserts on gfx950).
The walk follows the code in layout order, which for these straight-line
chains is execution order.
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from paged_kv_mla_req_amd import build as B

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

_REG = re.compile(r"(?<![\w.])([vas])(?:\[(\d+):(\d+)\]|(\d+))(?![\w])")


def _regs(text):
    out = set()
    for kind, lo, hi, one in _REG.findall(text):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    return out


def _kernels(asm: str, kernel: str = "mla_decode_kernel"):
    """name -> list of instruction lines, for each body of a kernel whose
    mangled name holds `kernel`."""
    bodies, cur, name = {}, None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*" + kernel + r"\S*):", line)
        if m:
            name, cur = m.group(1), []
            continue
        if cur is None:
            continue
        s = line.split(";")[0].strip()
        if s.startswith(".Lfunc_end") or s == "s_endpgm":
            bodies[name], cur = cur, None
            continue
        if not s or s.endswith(":") or s.startswith("."):
            continue
        cur.append(s)
    return bodies


def _check(instrs):
    """Instructions that touch a register an LDS read may still be writing,
    and partial lgkmcnt waits while a scalar load is outstanding (scalar loads
    also count in lgkmcnt but return out of order, so such a wait does not
    mean the older LDS reads have landed)."""
    inflight = []  # destination register sets of LDS reads, oldest first
    smem = False   # a scalar load issued since the last lgkmcnt(0)
    bad = []
    for i, ins in enumerate(instrs):
        op = ins.split()[0]
        if op.startswith("s_load") or op.startswith("s_buffer_load"):
            smem = True
            continue
        if op == "s_branch":
            # the next instruction in layout order is not this one's successor
            # (its block is reached from elsewhere, where the compiler's own
            # waits apply)
            smem = False
            continue
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", ins)
            if m:
                n = int(m.group(1))
                if n == 0:
                    smem = False
                elif smem and inflight:
                    bad.append((i, ins))
                inflight = inflight[len(inflight) - n:] if n < len(inflight) else inflight
            continue
        if op in ("s_nop", "s_barrier"):
            continue
        busy = set().union(*inflight) if inflight else set()
        operands = ins[len(op):]
        if op.startswith("ds_read") or op.startswith("ds_bpermute"):
            dst, _, rest = operands.partition(",")
            if busy & _regs(operands):
                bad.append((i, ins))
            inflight.append(_regs(dst))
            continue
        if op.startswith("ds_"):
            if busy & _regs(operands):
                bad.append((i, ins))
            inflight.append(set())  # counts in lgkmcnt, writes no register
            continue
        if busy & _regs(operands):
            bad.append((i, ins))
    return bad


def _split(ins):
    op = ins.split()[0]
    return op, [o.strip() for o in ins[len(op):].split(",")]


def _wait_states(ins):
    op, args = _split(ins)
    return int(args[0], 0) + 1 if op == "s_nop" else 1


VALU_TO_MFMA = 2
MFMA_TO_OTHER = 12      # 32x32x16 bf16: 8 passes
MFMA8_TO_OTHER = 20     # 32x32x64 f8f6f4 on e4m3 operands: 16 passes


def _mfma_hazards(instrs):
    bad = []
    for i, ins in enumerate(instrs):
        op, args = _split(ins)
        if not op.startswith("v_mfma"):
            continue
        # (1) VALU writes of the sources (scale registers included) shortly before
        srcs = set().union(*(_regs(a) for a in args[1:]))
        ws, j = 0, i - 1
        while j >= 0 and ws < VALU_TO_MFMA:
            pop, pargs = _split(instrs[j])
            if pop.startswith("v_") and not pop.startswith("v_mfma") and pargs and \
                    _regs(pargs[0]) & srcs:
                bad.append((i, ins, instrs[j]))
            ws += _wait_states(instrs[j])
            j -= 1
        # (2) uses of the result shortly after
        dst = _regs(args[0])
        need = MFMA8_TO_OTHER if "f8f6f4" in op else MFMA_TO_OTHER
        ws, j = 0, i + 1
        while j < len(instrs) and ws < need:
            nop, nargs = _split(instrs[j])
            if nop.startswith("v_mfma"):
                same_acc = len(nargs) > 3 and _regs(nargs[3]) == dst and _regs(nargs[0]) == dst
                if not same_acc and dst & set().union(*(_regs(a) for a in nargs)):
                    bad.append((i, ins, instrs[j]))
            elif nop != "s_nop" and dst & _regs(instrs[j][len(nop):]):
                bad.append((i, ins, instrs[j]))
            ws += _wait_states(instrs[j])
            j += 1
    return bad


def _compile(src):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, src.replace(".hip", ".s"))
        flags = [f for f in B.COMMON_FLAGS if f not in ("-fPIC",)]
        cmd = [HIPCC, *flags, *B.SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
               os.path.join(B.CSRC, src), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True, timeout=600)
        with open(out) as f:
            return f.read()


@pytest.fixture(scope="module")
def decode_asm():
    return _compile("decode.hip")


@pytest.fixture(scope="module")
def q8_asm():
    return _compile("decode_q8.hip")


@pytest.fixture(scope="module")
def all_bodies(decode_asm, q8_asm):
    """Every decode kernel body: the page kernel's two instances and the
    e4m3-query kernel."""
    bodies = dict(_kernels(decode_asm))
    bodies.update(_kernels(q8_asm, "mla_decode_q8_kernel"))
    return bodies


def test_all_kernels_present(decode_asm, q8_asm):
    """The page kernel in its two instances (bf16 cache, e4m3 cache; bf16
    MFMAs only) and the e4m3-query kernel (e4m3 MFMAs, scaled ones for the
    output)."""
    bodies = _kernels(decode_asm)
    assert len(bodies) == 2, list(bodies)
    assert all(not any("f8f6f4" in i for i in b) for b in bodies.values())
    q8 = _kernels(q8_asm, "mla_decode_q8_kernel")
    assert len(q8) == 1, list(q8)
    body = next(iter(q8.values()))
    assert sum("v_mfma_f32_32x32x64_f8f6f4" in i for i in body) > 0
    assert sum("v_mfma_scale_f32_32x32x64_f8f6f4" in i for i in body) > 0


def test_no_instruction_touches_an_in_flight_lds_read(all_bodies):
    for name, instrs in all_bodies.items():
        bad = _check(instrs)
        assert not bad, f"{name}: {len(bad)} instructions touch in-flight registers, e.g. {bad[:5]}"


def test_decode_kernels_have_no_scratch(decode_asm, q8_asm):
    """Every value stays in registers: no VGPR spills and no scratch memory (a
    spill reload would also wait on every page load in flight)."""
    for asm in (decode_asm, q8_asm):
        assert all(int(n) == 0 for n in re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm))
        assert "scratch_" not in asm


def test_q8_output_chain_waits_for_no_page_load(q8_asm):
    """The e4m3-query kernel's V reads are inline assembly: an LDS read the
    compiler knew of would get a wait for every page load in flight (vmcnt)
    in front of it, which puts the next page's load latency into every page.
    No vmcnt wait may lead into an output chain (its transposing V reads and
    scaled MFMAs), except the one after a piece's last page, which waits for
    the next piece's query loads just issued."""
    body = next(iter(_kernels(q8_asm, "mla_decode_q8_kernel").values()))
    for i, ins in enumerate(body):
        if not (ins.startswith("s_waitcnt") and "vmcnt" in ins):
            continue
        after = []
        for x in body[i + 1:i + 41]:
            if x.startswith("s_barrier"):
                break
            after.append(x)
        leads_in = any("ds_read_b64_tr_b8" in x or "v_mfma_scale" in x for x in after)
        query_wait = any(x.startswith("global_load") for x in body[max(0, i - 4):i])
        assert not leads_in or query_wait, (i, body[max(0, i - 4):i + 4])


def test_checker_flags_a_planted_use():
    """The walk itself: a use of a read's register before its wait is found,
    the same use after the wait is not."""
    good = ["ds_read_b128 v[4:7], v1", "s_waitcnt lgkmcnt(0)", "v_add_f32_e32 v8, v4, v5"]
    bad = ["ds_read_b128 v[4:7], v1", "v_add_f32_e32 v8, v4, v5", "s_waitcnt lgkmcnt(0)"]
    partial = ["ds_read_b128 v[4:7], v1", "ds_read_b128 v[8:11], v1", "s_waitcnt lgkmcnt(1)",
               "v_mov_b32_e32 v0, v5", "v_mov_b32_e32 v0, v9"]
    assert _check(good) == []
    assert len(_check(bad)) == 1
    assert [i for i, _ in _check(partial)] == [4]
    # a scalar load between an LDS read and a partial wait makes the wait unsafe
    smem = ["ds_read_b128 v[4:7], v1", "s_load_dword s4, s[0:1], 0x0",
            "ds_read_b128 v[8:11], v1", "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v0, v5"]
    assert [i for i, _ in _check(smem)] == [3]
    smem_drained = ["s_load_dword s4, s[0:1], 0x0", "s_waitcnt lgkmcnt(0)",
                    "ds_read_b128 v[4:7], v1", "ds_read_b128 v[8:11], v1",
                    "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v0, v5"]
    assert _check(smem_drained) == []


def test_no_unguarded_mfma_hazard(all_bodies):
    for name, instrs in all_bodies.items():
        bad = _mfma_hazards(instrs)
        assert not bad, f"{name}: {len(bad)} MFMA hazards, e.g. {bad[:3]}"


def test_hazard_walk_flags_planted_cases():
    mf = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"
    mf2 = "v_mfma_f32_32x32x16_bf16 a[0:15], v[12:15], v[8:11], a[0:15]"
    assert _mfma_hazards(["v_mov_b32_e32 v5, v1", mf]) != []
    assert _mfma_hazards(["v_mov_b32_e32 v5, v1", "s_nop 1", mf]) == []
    assert _mfma_hazards(["v_mov_b32_e32 v5, v1", "s_nop 0", mf]) != []
    assert _mfma_hazards(["v_mov_b32_e32 v30, v1", mf]) == []
    # accumulation into the same tile right after is fine, a read is not
    assert _mfma_hazards([mf, mf2]) == []
    assert _mfma_hazards([mf, "v_accvgpr_read_b32 v1, a3"]) != []
    assert _mfma_hazards([mf, "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v1, a3"]) == []
    # the e4m3 MFMA needs longer before its result is read
    f8 = "v_mfma_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15]"
    assert _mfma_hazards([f8, "s_nop 7", "s_nop 3", "v_mov_b32_e32 v40, v3"]) != []
    assert _mfma_hazards([f8, "s_nop 7", "s_nop 7", "s_nop 3", "v_mov_b32_e32 v40, v3"]) == []
