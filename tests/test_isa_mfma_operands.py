"""Check the gfx950 assembly of the HIP sources for a clobbered MFMA operand.

With a runtime loop that carried W fragments in registers from one iteration
to the next, this toolchain (ROCm 7.2 clang) allocated other values into the
upper half of a live 128-bit A operand of v_mfma_f32_16x16x32_bf16 before the
MFMA read it; the kernel then returned non-finite sums.  The kernels are
written to avoid that shape, and this test compiles every source to assembly
and checks (with the library's own per-source flags), inside each basic block, that no MFMA A/B operand register tuple
is partly overwritten after being written as a whole or while live-in.

Compiles only (no GPU).  Reads the assembly of code built here.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from self_speculative_lm_amd.build import compile_flags

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "self_speculative_lm_amd", "csrc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

_NO_VGPR_DEST = ("global_store", "ds_write", "buffer_store", "scratch_store", "global_atomic", "ds_add", "s_")


def _range(op):
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return int(m.group(1)), int(m.group(2))
    m = re.match(r"v(\d+)$", op)
    if m:
        return int(m.group(1)), int(m.group(1))
    return None


def clobbered_operands(asm: str):
    """[(function, instruction)] for MFMAs whose A or B tuple was partly
    overwritten within the block: after a whole-tuple write, or while some of
    its registers are live-in (written before the block)."""
    fn, last, bad, n_mfma, stamp = None, {}, [], 0, 0
    for line in asm.splitlines():
        m = re.match(r"^(\S+):", line)
        if m and not line.startswith((" ", "\t")):
            if not m.group(1).startswith("."):
                fn = m.group(1)
            last = {}  # a label starts a basic block
            continue
        t = line.split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        parts = t.split(None, 1)
        op = parts[0]
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        if op.startswith("v_mfma"):
            n_mfma += 1
            for o in ops[1:3]:
                r = _range(o)
                if not r:
                    continue
                ws = [last.get(x) for x in range(r[0], r[1] + 1)]
                whole = {w for w in ws if w is not None and w[0] == r}
                partial = [w for w in ws if w is not None and w[0] != r]
                if (whole and any(w not in whole for w in ws)) or (partial and any(w is None for w in ws)):
                    bad.append((fn, t))
        if op.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
            last = {}
        elif ops and not op.startswith(_NO_VGPR_DEST):
            d = _range(ops[0])
            if d:
                stamp += 1
                for x in range(d[0], d[1] + 1):
                    last[x] = (d, stamp)
    return bad, n_mfma


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def test_checker_flags_a_clobbered_operand():
    good = """k:
    global_load_dwordx4 v[4:7], v[0:1], off
    v_mfma_f32_16x16x32_bf16 v[8:11], v[4:7], v[12:15], v[8:11]
"""
    clobbered = """k:
    global_load_dwordx4 v[4:7], v[0:1], off
    v_add_u32_e32 v6, 1, v2
    v_mfma_f32_16x16x32_bf16 v[8:11], v[4:7], v[12:15], v[8:11]
"""
    livein = """k:
.LBB0_1:
    v_add_u32_e32 v6, 1, v2
    v_mfma_f32_16x16x32_bf16 v[8:11], v[4:7], v[12:15], v[8:11]
"""
    packed = """k:
    v_cvt_pk_bf16_f32 v12, v1, v2
    v_cvt_pk_bf16_f32 v13, v1, v2
    v_cvt_pk_bf16_f32 v14, v1, v2
    v_cvt_pk_bf16_f32 v15, v1, v2
    global_load_dwordx4 v[4:7], v[0:1], off
    v_mfma_f32_16x16x32_bf16 v[8:11], v[4:7], v[12:15], v[8:11]
"""
    assert clobbered_operands(good)[0] == []
    assert len(clobbered_operands(clobbered)[0]) == 1
    assert len(clobbered_operands(livein)[0]) == 1
    assert clobbered_operands(packed)[0] == []  # a tuple built register by register is fine


@pytest.mark.parametrize("src", SOURCES)
def test_no_clobbered_mfma_operand(src):
    hipcc = _hipcc()
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, src + ".s")
        path = os.path.join(CSRC, src)
        cmd = [hipcc, *compile_flags(path), "--cuda-device-only", "-S", "-o", out, path]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        bad, n = clobbered_operands(open(out).read())
    assert not bad, f"{len(bad)} MFMA(s) with a clobbered operand in {src}, e.g. {bad[0]}"
