"""CPU tests of the C-ABI library: it loads, exports every symbol include/fa.h
declares, and validates arguments on the host (every call here fails
validation before anything would be enqueued; no compute runs without a
GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

from exact_io_aware_fa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from exact_io_aware_fa_amd.build import build
        build()
    return B.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*?\**\s*\b(fa_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_binding_surface():
    assert _declared() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (fa_\w+)$", out, flags=re.M))
    assert set(_declared()) <= exported


def test_abi_version_and_status_strings(lib):
    assert B.fa_abi_version() == B.ABI_VERSION == 6
    for code, tag in ((0, "FA_OK"), (1, "FA_E_NULLPTR"), (2, "FA_E_SHAPE"),
                      (3, "FA_E_UNSUPPORTED"), (4, "FA_E_WORKSPACE"), (5, "FA_E_ALIAS"),
                      (6, "FA_E_LAUNCH"), (7, "FA_E_ALIGN"), (8, "FA_E_SCRATCH")):
        assert B.fa_status_str(code).startswith(tag)
    assert B.fa_status_str(99) == "FA_E_UNKNOWN"


# Fake, well-separated, 256-byte-aligned device addresses; never dereferenced
# because every call below is rejected by validation.
Q, K, V, O, L, DO, DQ, DK, DV, WS, KVL = (0x1000_0000 * (i + 1) for i in range(11))
SHAPE = dict(batch=2, heads=3, n=64, d=64)


def fwd(**kw):
    a = dict(SHAPE, causal=0, softmax_scale=0.125, dtype=B.FA_BF16, q=Q, k=K, v=V,
             kv_len=None, o=O, lse=L, stream=None)
    a.update(kw)
    return B.fa_fwd(a["batch"], a["heads"], a["n"], a["d"], a["causal"], a["softmax_scale"],
                    a["dtype"], a["q"], a["k"], a["v"], a["kv_len"], a["o"], a["lse"],
                    a["stream"])


def ws_bytes(dtype=B.FA_BF16, **shape):
    s = dict(SHAPE, **shape)
    return B.fa_bwd_workspace_bytes(s["batch"], s["heads"], s["n"], s["d"], dtype)


def bwd(**kw):
    a = dict(SHAPE, causal=1, softmax_scale=0.125, dtype=B.FA_BF16, q=Q, k=K, v=V, o=O,
             d_o=DO, lse=L, kv_len=None, dq=DQ, dk=DK, dv=DV, workspace=WS,
             workspace_bytes=None, stream=None)
    a.update(kw)
    if a["workspace_bytes"] is None:
        a["workspace_bytes"] = ws_bytes(a["dtype"])
    return B.fa_bwd(a["batch"], a["heads"], a["n"], a["d"], a["causal"], a["softmax_scale"],
                    a["dtype"], a["q"], a["k"], a["v"], a["o"], a["d_o"], a["lse"],
                    a["kv_len"], a["dq"], a["dk"], a["dv"], a["workspace"],
                    a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), B.FA_E_UNSUPPORTED), (dict(d=32), B.FA_E_UNSUPPORTED),
    (dict(dtype=5), B.FA_E_UNSUPPORTED),
    (dict(softmax_scale=float("nan")), B.FA_E_UNSUPPORTED),
    (dict(softmax_scale=float("inf")), B.FA_E_UNSUPPORTED),
    (dict(batch=0), B.FA_E_SHAPE), (dict(heads=0), B.FA_E_SHAPE), (dict(n=0), B.FA_E_SHAPE),
    (dict(n=(1 << 22) + 1), B.FA_E_SHAPE), (dict(batch=1 << 16, heads=1 << 16), B.FA_E_SHAPE),
    (dict(q=None), B.FA_E_NULLPTR), (dict(o=None), B.FA_E_NULLPTR), (dict(lse=None), B.FA_E_NULLPTR),
    (dict(k=K + 8), B.FA_E_ALIGN), (dict(lse=L + 4), B.FA_E_ALIGN), (dict(kv_len=KVL + 2), B.FA_E_ALIGN),
    (dict(o=Q + 4096), B.FA_E_ALIAS), (dict(lse=O + 64), B.FA_E_ALIAS), (dict(o=V), B.FA_E_ALIAS),
    (dict(kv_len=O + 16), B.FA_E_ALIAS),
])
def test_fwd_validation(lib, kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), B.FA_E_UNSUPPORTED), (dict(batch=-1), B.FA_E_SHAPE),
    (dict(d_o=None), B.FA_E_NULLPTR), (dict(dk=None), B.FA_E_NULLPTR),
    (dict(workspace=None), B.FA_E_WORKSPACE),
    (dict(workspace_bytes=1024), B.FA_E_WORKSPACE),
    (dict(workspace=WS + 16), B.FA_E_ALIGN), (dict(dv=DV + 2), B.FA_E_ALIGN),
    (dict(dq=DK), B.FA_E_ALIAS), (dict(dk=L), B.FA_E_ALIAS), (dict(workspace=DQ), B.FA_E_ALIAS),
    (dict(dv=Q + 256), B.FA_E_ALIAS), (dict(kv_len=DQ + 4), B.FA_E_ALIAS),
])
def test_bwd_validation(lib, kw, code):
    assert bwd(**kw) == code


def fwd_gqa(heads_kv, **kw):
    a = dict(SHAPE, causal=0, softmax_scale=0.125, dtype=B.FA_BF16, q=Q, k=K, v=V,
             kv_len=None, o=O, lse=L, stream=None)
    a.update(kw)
    return B.fa_fwd_gqa(a["batch"], a["heads"], heads_kv, a["n"], a["d"], a["causal"],
                        a["softmax_scale"], a["dtype"], a["q"], a["k"], a["v"],
                        a["kv_len"], a["o"], a["lse"], a["stream"])


def bwd_gqa(heads_kv, **kw):
    a = dict(SHAPE, causal=1, softmax_scale=0.125, dtype=B.FA_BF16, q=Q, k=K, v=V, o=O,
             d_o=DO, lse=L, kv_len=None, dq=DQ, dk=DK, dv=DV, workspace=WS,
             workspace_bytes=None, stream=None)
    a.update(kw)
    if a["workspace_bytes"] is None:
        a["workspace_bytes"] = ws_bytes(a["dtype"])
    return B.fa_bwd_gqa(a["batch"], a["heads"], heads_kv, a["n"], a["d"], a["causal"],
                        a["softmax_scale"], a["dtype"], a["q"], a["k"], a["v"], a["o"],
                        a["d_o"], a["lse"], a["kv_len"], a["dq"], a["dk"], a["dv"],
                        a["workspace"], a["workspace_bytes"], a["stream"])


# SHAPE has 3 query heads: heads_kv must be 1 or 3. One K/V head of
# SHAPE is 64 * 64 * 2 = 8 KiB, so K + 8192 is the end of a one-head K.
@pytest.mark.parametrize("heads_kv,kw,code", [
    (0, {}, B.FA_E_SHAPE), (-1, {}, B.FA_E_SHAPE), (2, {}, B.FA_E_SHAPE),
    (4, {}, B.FA_E_SHAPE), (6, {}, B.FA_E_SHAPE),
    (1, dict(d=96), B.FA_E_UNSUPPORTED), (1, dict(k=None), B.FA_E_NULLPTR),
    (1, dict(v=V + 8), B.FA_E_ALIGN),
    (1, dict(o=K + 8192 - 16), B.FA_E_ALIAS),   # inside the one-head K
    (1, dict(lse=V + 4096), B.FA_E_ALIAS),
    (3, dict(o=K + 3 * 8192 - 16), B.FA_E_ALIAS),  # inside the three-head K
])
def test_fwd_gqa_validation(lib, heads_kv, kw, code):
    assert fwd_gqa(heads_kv, **kw) == code


@pytest.mark.parametrize("heads_kv,kw,code", [
    (0, {}, B.FA_E_SHAPE), (2, {}, B.FA_E_SHAPE), (5, {}, B.FA_E_SHAPE),
    (1, dict(dq=None), B.FA_E_NULLPTR), (1, dict(workspace_bytes=8), B.FA_E_WORKSPACE),
    (1, dict(dk=K + 8192 - 16), B.FA_E_ALIAS),   # dK overlaps the one-head K
    (1, dict(dv=DK + 8192 - 16), B.FA_E_ALIAS),  # dV overlaps the one-head dK
    (1, dict(dq=DV + 4096), B.FA_E_ALIAS),
    (3, dict(dv=DK + 3 * 8192 - 16), B.FA_E_ALIAS),
])
def test_bwd_gqa_validation(lib, heads_kv, kw, code):
    assert bwd_gqa(heads_kv, **kw) == code


def test_plain_entry_points_are_the_full_head_case(lib):
    # fa_fwd / fa_bwd behave as heads_kv = heads: the K range covers all
    # three heads, so an output placed inside the third head's K is caught.
    assert fwd(o=K + 3 * 8192 - 16) == B.FA_E_ALIAS
    assert bwd(dk=K + 3 * 8192 - 16) == B.FA_E_ALIAS


CU = 0x0c00_0000  # fake offsets array, below every tensor
PACKED = dict(num_seqs=3, heads=2, heads_kv=1, total=200, max_seqlen=90, d=64)


def fwd_varlen(**kw):
    a = dict(PACKED, cu=CU, causal=1, softmax_scale=0.125, dtype=B.FA_BF16, q=Q, k=K, v=V,
             o=O, lse=L, stream=None)
    a.update(kw)
    return B.fa_fwd_varlen(a["num_seqs"], a["heads"], a["heads_kv"], a["total"],
                           a["max_seqlen"], a["d"], a["cu"], a["causal"], a["softmax_scale"],
                           a["dtype"], a["q"], a["k"], a["v"], a.get("mask"), a["o"], a["lse"],
                           a["stream"])


def bwd_varlen(**kw):
    a = dict(PACKED, cu=CU, causal=1, softmax_scale=0.125, dtype=B.FA_BF16, q=Q, k=K, v=V,
             o=O, d_o=DO, lse=L, dq=DQ, dk=DK, dv=DV, workspace=WS, workspace_bytes=None,
             stream=None)
    a.update(kw)
    if a["workspace_bytes"] is None:
        a["workspace_bytes"] = B.fa_bwd_workspace_bytes(a["num_seqs"], a["heads"],
                                                        a["max_seqlen"], a["d"], a["dtype"])
    return B.fa_bwd_varlen(a["num_seqs"], a["heads"], a["heads_kv"], a["total"],
                           a["max_seqlen"], a["d"], a["cu"], a["causal"], a["softmax_scale"],
                           a["dtype"], a["q"], a["k"], a["v"], a["o"], a["d_o"], a["lse"],
                           a.get("mask"), a["dq"], a["dk"], a["dv"], a["workspace"],
                           a["workspace_bytes"], a["stream"])


# One head of PACKED is 200 * 64 * 2 = 25600 bytes; its LSE 800 bytes per head.
@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), B.FA_E_NULLPTR), (dict(num_seqs=0), B.FA_E_SHAPE),
    (dict(max_seqlen=0), B.FA_E_SHAPE), (dict(max_seqlen=201), B.FA_E_SHAPE),
    (dict(heads_kv=3), B.FA_E_SHAPE), (dict(d=80), B.FA_E_UNSUPPORTED),
    (dict(total=1 << 23, max_seqlen=1 << 22, d=256), B.FA_E_SHAPE),  # a head >= 2 GiB
    (dict(cu=CU + 2), B.FA_E_ALIGN), (dict(q=Q + 8), B.FA_E_ALIGN),
    (dict(o=K + 25600 - 16), B.FA_E_ALIAS),      # inside the one-head K
    (dict(o=Q + 2 * 25600 - 16), B.FA_E_ALIAS),  # inside the two-head Q
    (dict(lse=CU), B.FA_E_ALIAS),                # over the offsets
    (dict(lse=O + 256), B.FA_E_ALIAS),
])
def test_fwd_varlen_validation(lib, kw, code):
    assert fwd_varlen(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), B.FA_E_NULLPTR), (dict(max_seqlen=300), B.FA_E_SHAPE),
    (dict(dk=None), B.FA_E_NULLPTR), (dict(workspace_bytes=64), B.FA_E_WORKSPACE),
    (dict(cu=CU + 1), B.FA_E_ALIGN),
    (dict(dq=CU), B.FA_E_ALIAS), (dict(dv=DK + 25600 - 16), B.FA_E_ALIAS),
    (dict(workspace=L), B.FA_E_ALIAS),
])
def test_bwd_varlen_validation(lib, kw, code):
    assert bwd_varlen(**kw) == code


def test_varlen_workspace_is_per_sequence_and_head(lib):
    # num_seqs x heads slices of max_seqlen rows padded to 64: 3 x 2 x 128.
    assert B.fa_bwd_workspace_bytes(3, 2, 90, 64, B.FA_BF16) == 2 * 3072


def test_workspace_size_closed_form(lib):
    b, h, n, d = 2, 3, 100, 128
    rows = b * h * 128 * 4          # n padded to a multiple of 64 per head
    vec = (rows + 255) // 256 * 256
    assert ws_bytes(B.FA_FP32, batch=b, heads=h, n=n, d=d) == 2 * vec
    assert ws_bytes(B.FA_BF16, batch=b, heads=h, n=n, d=d) == 2 * vec
    assert ws_bytes(B.FA_BF16, d=48) == 0
    assert ws_bytes(B.FA_BF16, n=0) == 0


def test_loader_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


# ---------------------------------------------------------------------------
# FP8 entry points

def test_fp8_sizes_closed_form(lib):
    # np = n rounded up to 128; codes batch*heads*np*d bytes, scales 4 per block.
    assert B.fa_fp8_codes_bytes(2, 3, 300, 128) == 2 * 3 * 384 * 128
    assert B.fa_fp8_scales_bytes(2, 3, 300) == 2 * 3 * 3 * 4
    assert B.fa_fp8_codes_bytes(1, 1, 128, 64) == 128 * 64
    assert B.fa_fp8_codes_bytes(0, 1, 128, 64) == 0
    assert B.fa_fp8_scales_bytes(1, 1, 0) == 0


X8, C8, S8, SG = (0x2_0000_0000 * (i + 1) for i in range(4))


def quant(**kw):
    a = dict(batch=2, heads=3, n=300, d=128, layout=B.FA_FP8_ROWS, x=X8, signs=None,
             codes=C8, scales=S8, stream=None)
    a.update(kw)
    return B.fa_fp8_quantize(a["batch"], a["heads"], a["n"], a["d"], a["layout"], a["x"],
                             a["signs"], a["codes"], a["scales"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=32), B.FA_E_UNSUPPORTED), (dict(d=96), B.FA_E_UNSUPPORTED),
    (dict(d=512), B.FA_E_UNSUPPORTED), (dict(layout=2), B.FA_E_UNSUPPORTED),
    (dict(layout=B.FA_FP8_VT, signs=SG), B.FA_E_UNSUPPORTED),
    (dict(n=0), B.FA_E_SHAPE), (dict(batch=0), B.FA_E_SHAPE),
    (dict(x=None), B.FA_E_NULLPTR), (dict(codes=None), B.FA_E_NULLPTR),
    (dict(scales=None), B.FA_E_NULLPTR),
    (dict(x=X8 + 2), B.FA_E_ALIGN), (dict(codes=C8 + 8), B.FA_E_ALIGN),
    (dict(scales=S8 + 2), B.FA_E_ALIGN), (dict(signs=SG + 4), B.FA_E_ALIGN),
    (dict(codes=X8 + 4096), B.FA_E_ALIAS), (dict(scales=C8 + 64), B.FA_E_ALIAS),
    (dict(scales=X8), B.FA_E_ALIAS), (dict(signs=C8 + 16), B.FA_E_ALIAS),
])
def test_fp8_quantize_validation(lib, kw, code):
    assert quant(**kw) == code


Q8, K8, V8, QS, KS, VS, O8, L8, KL8 = (0x3_0000_0000 * (i + 1) for i in range(9))


def fwd8(**kw):
    a = dict(batch=2, heads=4, heads_kv=2, n=300, d=128, causal=1, softmax_scale=0.125,
             q8=Q8, qs=QS, k8=K8, ks=KS, v8=V8, vs=VS, kv_len=None, o=O8, lse=L8, stream=None)
    a.update(kw)
    return B.fa_fwd_fp8(a["batch"], a["heads"], a["heads_kv"], a["n"], a["d"], a["causal"],
                        a["softmax_scale"], a["q8"], a["qs"], a["k8"], a["ks"], a["v8"],
                        a["vs"], a["kv_len"], a["o"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=32), B.FA_E_UNSUPPORTED), (dict(d=96), B.FA_E_UNSUPPORTED),
    (dict(d=512), B.FA_E_UNSUPPORTED), (dict(softmax_scale=float("nan")), B.FA_E_UNSUPPORTED),
    (dict(heads_kv=3), B.FA_E_SHAPE), (dict(heads_kv=0), B.FA_E_SHAPE),
    (dict(heads_kv=8), B.FA_E_SHAPE), (dict(n=0), B.FA_E_SHAPE),
    (dict(n=(1 << 22) + 1), B.FA_E_SHAPE),
    (dict(q8=None), B.FA_E_NULLPTR), (dict(vs=None), B.FA_E_NULLPTR),
    (dict(o=None), B.FA_E_NULLPTR), (dict(lse=None), B.FA_E_NULLPTR),
    (dict(k8=K8 + 8), B.FA_E_ALIGN), (dict(o=O8 + 4), B.FA_E_ALIGN),
    (dict(ks=KS + 2), B.FA_E_ALIGN), (dict(kv_len=KL8 + 1), B.FA_E_ALIGN),
    (dict(o=Q8 + 1024), B.FA_E_ALIAS), (dict(lse=O8 + 16), B.FA_E_ALIAS),
    (dict(lse=VS), B.FA_E_ALIAS), (dict(o=KL8 - 16, kv_len=KL8), B.FA_E_ALIAS),
])
def test_fwd_fp8_validation(lib, kw, code):
    assert fwd8(**kw) == code


def test_bwd_noalloc_rejects_oversize_and_bad_shapes_before_any_hip_call(lib):
    """fa_bwd_noalloc checks sizes on the host first: a call whose workspace
    would exceed the static scratch returns FA_E_SCRATCH, bad shapes their
    usual codes; neither touches the HIP runtime (no GPU here)."""
    args = [Q, K, V, O, DO, L, None, DQ, DK, DV, None]
    assert B.fa_bwd_workspace_bytes(1, 80, 32768, 128, B.FA_BF16) > B.FA_NOALLOC_SCRATCH_BYTES
    assert B.fa_bwd_workspace_bytes(1, 32, 16384, 128, B.FA_BF16) <= B.FA_NOALLOC_SCRATCH_BYTES
    assert B.fa_bwd_noalloc(1, 80, 80, 32768, 128, 1, 0.1, B.FA_BF16, *args) == B.FA_E_SCRATCH
    assert B.fa_bwd_noalloc(1, 4, 3, 64, 64, 1, 0.1, B.FA_BF16, *args) == B.FA_E_SHAPE
    assert B.fa_bwd_noalloc(1, 4, 4, 64, 96, 1, 0.1, B.FA_BF16, *args) == B.FA_E_UNSUPPORTED
    assert B.fa_bwd_noalloc(0, 4, 4, 64, 64, 1, 0.1, B.FA_BF16, *args) == B.FA_E_SHAPE
