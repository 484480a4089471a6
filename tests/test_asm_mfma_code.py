"""The dense prefill projection's four-wave tiles issue their matrix instructions as inline asm
(accumulators tied in place to the matrix registers). The compiler does not see those as matrix
instructions, so it inserts none of the waits the hardware needs around them; the kernel is only
correct if the generated code keeps the gaps the instruction set requires. This test compiles
csrc/prefill_gemm.hip to gfx950 assembly with the library's own flags and checks them:

- no accumulator-register moves inside the k-loop (every MFMA accumulates in place);
- no vector-ALU write to an MFMA's A, B or C register within the 4 instructions before it (a
  VALU-to-MFMA read needs 2 wait states);
- no access of a matrix register within 19 wait states after the last MFMA (a 16-pass MFMA's
  result is not ready for other instructions earlier);
- no MFMA among the first 4 instructions of a basic block (so the look-back above sees the
  instructions that precede it at run time).

Host-only: needs hipcc, no GPU.
"""
import os
import re
import subprocess

import pytest

from dual_flow_shared_amd import build as dfx_build

QUAD_KERNEL = re.compile(r"^(_ZN3dfx19prefill_gemm_kernelINS_9DenseTileILi[0-9]+ELi8ELi2ELi2E\S+):", re.M)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        cc = dfx_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "prefill_gemm.s")
    flags = [f for f in dfx_build.FLAGS if f != "-fPIC"]
    src = os.path.join(dfx_build.CSRC, "prefill_gemm.hip")
    r = subprocess.run([cc, *flags, "--cuda-device-only", "-S", src, "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _functions(text):
    for m in QUAD_KERNEL.finditer(text):
        i = m.start()
        yield m.group(1), text[i:text.index(".Lfunc_end", i)].split("\n")


def _instructions(lines):
    """(opcode, operands, starts_block) per instruction."""
    out, new_block = [], True
    for raw in lines:
        t = raw.split(";")[0].strip()
        if re.match(r"^\.LBB\S*:", t):
            new_block = True
            continue
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        args = [a.strip() for a in t[len(op):].split(",")] if len(t.split()) > 1 else []
        out.append((op, args, new_block))
        new_block = False
    return out


def test_quad_tiles_present(asm):
    names = [n for n, _ in _functions(asm)]
    assert len(names) == 4, names  # 256- and 192-feature tiles, plain and gate/up epilogues


def test_asm_mfma_gaps(asm):
    for name, lines in _functions(asm):
        ins = _instructions(lines)
        mf = [k for k, x in enumerate(ins) if x[0].startswith("v_mfma")]
        assert mf, name
        first, last = mf[0], mf[-1]
        for k in range(first, last + 1):
            assert not ins[k][0].startswith("v_accvgpr"), (name, "accumulator move in the k-loop", ins[k])
        for k in mf:
            ops = set().union(*[_regs(a) for a in ins[k][1][1:4]])
            for q in range(max(0, k - 4), k):
                op, args, _ = ins[q]
                assert not (op.startswith("v_") and not op.startswith("v_mfma") and args and _regs(args[0]) & ops), \
                    (name, "VALU write just before an MFMA", ins[q], ins[k])
        run, since = 0, 4
        for op, _, starts in ins:
            since = 0 if starts else since
            if op.startswith("v_mfma"):
                assert since >= 4, (name, "MFMA near the start of a basic block")
            since += 1
        waited = 0
        for op, args, _ in ins[last + 1:]:
            if waited >= 19:
                break
            assert not any(r[0] == "a" for a in args for r in _regs(a)), \
                (name, f"matrix register accessed {waited} wait states after the last MFMA", op, args)
            waited += int(args[0]) + 1 if op == "s_nop" else 1
