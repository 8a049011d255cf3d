"""Static check of the matrix products that accumulate in VGPRs.

The S and dP products of the backward's dK/dV kernels (d <= 128 and
d = 256) and of the d = 256 dQ kernel are inline assembly
(v_mfma_f32_32x32x16_bf16 with a VGPR accumulator), which the compiler's
hazard tracking does not see. A kernel is only correct if no other
instruction reads or writes a product's result registers until the product
has finished (an 8-pass product needs about a dozen wait states), and no
instruction overwrites a separate accumulator input (C) that the product
may still be reading. This test compiles each kernel for gfx950 and checks,
in the generated assembly, that for WAIT_STATES wait states after each such
product (an instruction counts one, s_nop N counts N + 1) nothing but the
next product of the same accumulation chain (same registers as destination
and accumulator) touches the result registers, nothing writes a separate C
input, that no result overlaps the product's A, B or C operands, and that
a vector instruction that writes an operand is at least VALU_WAIT wait
states ahead of the product that reads it.
Runs on the CPU (hipcc cross-compiles).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = os.path.join(ROOT, "exact_io_aware_fa_amd", "csrc", "kernels")
SOURCES = ("fa_bwd_bf16.hip", "fa_bwd_dq_d256.hip", "fa_bwd_dkdv_d256.hip", "fa_bwd_dkdv_wide.hip")
WAIT_STATES = 20  # well above what an 8-pass product needs before its result is read
VALU_WAIT = 2     # a vector write of a register before a matrix product reads it


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _vgprs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _wait_states(inst):
    m = re.match(r"s_nop\s+(\d+)", inst)
    return int(m.group(1)) + 1 if m else 1


@pytest.fixture(scope="module", params=SOURCES)
def assembly(request, tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / (request.param + ".s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-munsafe-fp-atomics",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(KERNELS, request.param), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = [l.strip() for l in out.read_text().split("\n")]
    # Instructions only (no labels, directives or comments).
    return [l for l in lines
            if l and not l.startswith((";", ".")) and not l.endswith(":") and "//" not in l[:2]]


def test_vgpr_products_exist(assembly):
    n = sum(1 for l in assembly if l.startswith("v_mfma_f32_32x32x16_bf16 v["))
    assert n > 0, "no VGPR-accumulator products found: the check below would be vacuous"


def test_no_access_to_vgpr_product_results_in_flight(assembly):
    bad = []
    for i, line in enumerate(assembly):
        if not line.startswith("v_mfma_f32_32x32x16_bf16 v["):
            continue
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        dst = _vgprs(ops[0])
        src_c = _vgprs(ops[3])
        if dst & (_vgprs(ops[1]) | _vgprs(ops[2])):
            bad.append(("result overlaps A/B", line, ""))
        if src_c and src_c != dst and dst & src_c:
            bad.append(("result partly overlaps C", line, ""))
        separate_c = src_c if src_c != dst else set()
        waited = 0
        for nxt in assembly[i + 1:]:
            if waited >= WAIT_STATES:
                break
            waited += _wait_states(nxt)
            if nxt.startswith("s_"):
                continue  # scalar instructions touch no VGPRs
            nops = [o.strip() for o in nxt.split(None, 1)[1].split(",")] if " " in nxt else []
            if nops and _vgprs(nops[0]) & separate_c:
                bad.append(("C input overwritten while read", line, nxt))
                break
            if nxt.startswith("v_mfma") and len(nops) == 4 and \
                    _vgprs(nops[0]) == dst and _vgprs(nops[3]) == dst:
                break  # the chain's next product: accumulates in place
            if _vgprs(" ".join(nops)) & dst:
                bad.append(("touched while in flight", line, nxt))
                break
    assert not bad, bad[:5]


def test_no_vector_write_of_vgpr_product_operands_just_before(assembly):
    """A vector instruction that writes a register needs VALU_WAIT wait
    states before a matrix product may read it as A, B or C; the compiler
    inserts them for its own products only (the register allocator may put a
    v_accvgpr_read that brings an operand back from an AGPR right before an
    assembly product). For each operand register of an assembly product,
    the nearest earlier instruction that writes it (within WINDOW_BEFORE
    instructions) must either not be a vector ALU instruction (LDS loads and
    other products are waited for by counters and the hardware) or lie at
    least VALU_WAIT wait states back (an instruction counts one, s_nop N
    counts N + 1)."""
    WINDOW_BEFORE = 6
    bad = []
    for i, line in enumerate(assembly):
        if not line.startswith("v_mfma_f32_32x32x16_bf16 v["):
            continue
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        pending = _vgprs(ops[1]) | _vgprs(ops[2]) | (_vgprs(ops[3]) if ops[3] != ops[0] else set())
        waited = 0
        for prev in reversed(assembly[max(i - WINDOW_BEFORE, 0):i]):
            if not pending:
                break
            # Instructions whose first operand is a destination: vector ALU
            # and matrix instructions and loads (a store's first operand is
            # an address it reads).
            if prev.startswith(("v_", "ds_read", "buffer_load", "global_load", "scratch_load")) \
                    and " " in prev:
                written = _vgprs(prev.split(None, 1)[1].split(",")[0]) & pending
                if written:
                    if prev.startswith("v_") and not prev.startswith("v_mfma") \
                            and waited < VALU_WAIT:
                        bad.append((prev, line))
                        break
                    pending -= written
            waited += _wait_states(prev)
    assert not bad, bad[:5]


def test_vector_write_check_catches_a_write_right_before_a_product():
    """The check above on a hand-made sequence: an operand written by a
    v_accvgpr_read one instruction before the product is flagged; with an
    s_nop 1 in between it is not."""
    seq = ["v_accvgpr_read_b32 v41, a133", "s_waitcnt lgkmcnt(4)",
           "v_mfma_f32_32x32x16_bf16 v[16:31], v[160:163], v[38:41], 0"]
    with pytest.raises(AssertionError):
        test_no_vector_write_of_vgpr_product_operands_just_before(seq)
    ok = seq[:2] + ["s_nop 1"] + seq[2:]
    test_no_vector_write_of_vgpr_product_operands_just_before(ok)
