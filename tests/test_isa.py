"""Generated-code checks of the product kernels (host only: compiles the
device code to gfx950 assembly, runs nothing).

1. A matrix-core instruction reads its A and B registers and writes its four
   result registers over several passes after it issues.  If the register
   allocator hands one of those registers to another value before the result
   has been read (for instance a result register no FMA reads, when fewer
   than four columns are live), the late write of the product clobbers that
   value.  The kernels fence each product (mfma_fence in dot_unit.h); the
   check: after every MFMA, no instruction writes its result or source
   registers before some instruction reads the result.
2. The weight stream keeps several tiles of loads in flight per wave.  A
   wait for all outstanding vector memory operations (vmcnt(0)) inside a
   loop of products drains that pipeline every iteration (a column-map load
   inside the 16-column activation chunks once did exactly that).
3. A buffer load takes its range descriptor from scalar registers.  Where
   the compiler cannot prove a descriptor uniform it wraps each load in a
   loop over the lanes' distinct descriptors; every range here is the
   wave's, so no such loop may appear.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_q4_q8_amd", "csrc")
SOURCES = ["qmv.hip", "moe.hip"]


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


def _loops(asm_lines):
    """{(function, innermost loop header): [instructions]} from the
    compiler's loop annotations of the basic blocks."""
    loops = {}
    fn = cur = None
    for line in asm_lines:
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn, cur = m.group(1), None
            continue
        if re.match(r"^(\.LBB\w+|; %bb\.\d+):", line):
            lab = line.split(":")[0].replace(".LBB", "BB")
            h = re.search(r"in Loop: Header=(\S+)", line)
            cur = (fn, lab) if "Loop Header" in line else (fn, h.group(1)) if h else None
            continue
        s = line.split(";")[0].strip()
        if cur is not None and s and not s.startswith("."):
            loops.setdefault(cur, []).append(s)
    return loops


def full_waits_in_product_loops(asm_lines):
    """Innermost loops holding a matrix-core product and a vmcnt(0) wait."""
    return [k for k, ins in _loops(asm_lines).items()
            if any(i.startswith("v_mfma") for i in ins)
            and any(i.startswith("s_waitcnt") and re.search(r"vmcnt\(0\)", i) for i in ins)]


def per_lane_descriptor_loops(asm_lines):
    """Innermost loops that take a buffer descriptor from a lane
    (v_readfirstlane), issue a buffer access and iterate over the exec mask."""
    return [k for k, ins in _loops(asm_lines).items()
            if any(i.startswith("v_readfirstlane") for i in ins)
            and any(i.startswith(("buffer_load", "buffer_store", "buffer_atomic")) for i in ins)
            and any(re.match(r"s_xor_b64 exec, exec", i) for i in ins)]


def test_loop_checks_flag_their_patterns():
    drain = ["_Zk:",
             ".LBB0_1:                                ; =>This Inner Loop Header: Depth=1",
             "  buffer_load_dwordx4 v[0:3], v4, s[8:11], 0 offen",
             "  s_waitcnt vmcnt(0)",
             "  v_mfma_f32_16x16x32_f16 v[4:7], v[0:3], v[8:11], 0",
             "  s_cbranch_scc1 .LBB0_1",
             "  s_endpgm"]
    assert full_waits_in_product_loops(drain) == [("_Zk", "BB0_1")]
    ok = [l.replace("vmcnt(0)", "vmcnt(4)") for l in drain]
    assert full_waits_in_product_loops(ok) == []
    lanes = ["_Zk:",
             ".LBB0_2:                                ; =>This Inner Loop Header: Depth=1",
             "  v_readfirstlane_b32 s12, v18",
             "  v_readfirstlane_b32 s13, v19",
             "  v_cmp_eq_u64_e64 s[4:5], s[12:13], v[18:19]",
             "  s_and_saveexec_b64 s[4:5], s[4:5]",
             "  buffer_load_dwordx4 v[6:9], v15, s[12:15], 0 offen",
             "  s_xor_b64 exec, exec, s[4:5]",
             "  s_cbranch_execnz .LBB0_2",
             "  s_endpgm"]
    assert per_lane_descriptor_loops(lanes) == [("_Zk", "BB0_2")]
    assert per_lane_descriptor_loops([l for l in lanes if "s_xor" not in l]) == []


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


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if _hipcc() is None:
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("isa")
    outs = [str(d / (s + ".s")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(_assembly, SOURCES, outs))
    res = {}
    for src, out in zip(SOURCES, outs):
        with open(out) as fh:
            res[src] = fh.readlines()
    return res


def test_no_register_reuse_under_matrix_core_products(assembly):
    total = 0
    for src, lines in assembly.items():
        n, bad = early_overwrites(lines)
        total += n
        assert not bad, f"{src}: {len(bad)} products with an early overwrite, first: {bad[0]}"
    assert total > 0


def test_no_full_wait_in_product_loops(assembly):
    for src, lines in assembly.items():
        bad = full_waits_in_product_loops(lines)
        assert not bad, f"{src}: loops of products that wait for every load: {bad[:3]}"


def test_no_per_lane_descriptor_loops(assembly):
    for src, lines in assembly.items():
        bad = per_lane_descriptor_loops(lines)
        assert not bad, f"{src}: buffer accesses looped over per-lane descriptors: {bad[:3]}"
