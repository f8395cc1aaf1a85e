"""Generated-code check of the matrix-core products (host only: compiles the
device code to gfx950 assembly, runs nothing).

A matrix-core instruction reads its A and B registers and writes its four
result registers over several passes after it issues.  If the register
allocator hands one of those registers to another value before the result
has been read (for instance a result register no FMA reads, when fewer than
four columns are live), the late write of the product clobbers that value.
The kernels fence each product (mfma_fence in dot_unit.h); this test checks
the compiled code: after every MFMA, no instruction writes its result or
source registers before some instruction reads the result.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_q4_q8_amd", "csrc")
SOURCES = ["qmv.hip", "ffn.hip", "moe.hip"]


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def _assembly(src, out):
    cmd = [_hipcc(), "-O3", "-std=c++17", "--offload-arch=gfx950", f"-I{ROOT}/include", f"-I{CSRC}",
           "-x", "hip", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


# instructions whose first operand is not a vector register they write
_NO_VDST = ("s_", "ds_write", "buffer_store", "global_store", "v_cmp", "v_cmpx")


def early_overwrites(asm_lines):
    """(mfma, offending instruction) pairs: a write to the product's result
    or source registers before any instruction reads the result (within the
    same straight-line block)."""
    insts = []
    fn = None
    for line in asm_lines:
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn = m.group(1)
        s = line.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            insts.append((fn, s))
    bad = []
    n = 0
    for k, (f, s) in enumerate(insts):
        if not s.startswith("v_mfma"):
            continue
        n += 1
        ops = s.split(None, 1)[1].split(",")
        d, a, b = _regs(ops[0]), _regs(ops[1]), _regs(ops[2])
        for f2, s2 in insts[k + 1:k + 400]:
            if f2 != f or s2.startswith(("s_endpgm", "s_branch", "s_cbranch")):
                break
            parts = s2.split(None, 1)
            if len(parts) < 2:
                continue
            op, rest = parts
            o = rest.split(",")
            srcs = set().union(*[_regs(x) for x in o[1:]]) if len(o) > 1 else set()
            if srcs & d:
                break
            if op.startswith(_NO_VDST):
                continue
            if _regs(o[0]) & (d | a | b):
                bad.append((f, s, s2))
                break
    return n, bad


def test_checker_flags_a_reused_result_register():
    asm = ["_Zk:",
           "  v_mfma_f32_16x16x32_f16 v[4:7], v[0:3], v[8:11], 0",
           "  v_mov_b32_e32 v7, 0",
           "  v_fma_f32 v12, v13, v4, v12",
           "  s_endpgm"]
    n, bad = early_overwrites(asm)
    assert n == 1 and len(bad) == 1
    ok = ["_Zk:",
          "  v_mfma_f32_16x16x32_f16 v[4:7], v[0:3], v[8:11], 0",
          "  v_fma_f32 v12, v13, v4, v12",
          "  v_mov_b32_e32 v7, 0",
          "  s_endpgm"]
    assert early_overwrites(ok) == (1, [])


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_no_register_reuse_under_matrix_core_products(tmp_path):
    outs = [str(tmp_path / (s + ".s")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(_assembly, SOURCES, outs))
    total = 0
    for src, out in zip(SOURCES, outs):
        with open(out) as fh:
            n, bad = early_overwrites(fh.readlines())
        total += n
        assert not bad, f"{src}: {len(bad)} products with an early overwrite, first: {bad[0]}"
    assert total > 0
