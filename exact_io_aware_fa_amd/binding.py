"""ctypes binding of the C ABI in include/fa.h -- argument marshalling only.

Every function here has the name and argument order of the C entry point it
wraps; tensors are passed as raw device addresses (ints). Nothing is
computed on the host. If the shared library has not been built the loader
raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FA_LIB", os.path.join(PKG, "libexact_fa.so"))

FA_BF16 = 0
FA_FP32 = 1

FA_OK = 0
FA_E_NULLPTR = 1
FA_E_SHAPE = 2
FA_E_UNSUPPORTED = 3
FA_E_WORKSPACE = 4
FA_E_ALIAS = 5
FA_E_LAUNCH = 6
FA_E_ALIGN = 7
FA_E_SCRATCH = 8

# Size of the static scratch fa_bwd_noalloc uses on each device.
FA_NOALLOC_SCRATCH_BYTES = 16 << 20

# Every symbol include/fa.h declares.
EXPORTED = ("fa_fwd", "fa_fwd_gqa", "fa_fwd_masked", "fa_fwd_varlen", "fa_bwd",
            "fa_bwd_gqa", "fa_bwd_masked", "fa_bwd_varlen", "fa_bwd_timed", "fa_bwd_noalloc",
            "fa_bwd_workspace_bytes", "fa_block_index_bytes", "fa_block_index_build",
            "fa_fp8_codes_bytes", "fa_fp8_scales_bytes", "fa_fp8_quantize", "fa_fwd_fp8",
            "fa_status_str", "fa_abi_version")

# The FA_ABI_VERSION this binding was written against.
ABI_VERSION = 6

FA_BLOCK = 128

# Layouts of encoded FP8 tensors.
FA_FP8_ROWS = 0
FA_FP8_VT = 1


class FaMask(ctypes.Structure):
    """fa_mask: window sides (-1 = unbounded) and a block index address."""
    _fields_ = [("window_left", ctypes.c_int64), ("window_right", ctypes.c_int64),
                ("block_index", ctypes.c_void_p)]


def mask_arg(window=(-1, -1), block_index=None):
    """A FaMask for ctypes calls, or None when no extra mask is asked for."""
    if tuple(window) == (-1, -1) and not block_index:
        return None
    return FaMask(int(window[0]), int(window[1]), block_index or None)

_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libexact_fa.so once (raises if it is missing)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m exact_io_aware_fa_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        L.fa_fwd.restype = ctypes.c_int
        L.fa_fwd.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                             ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.fa_bwd.restype = ctypes.c_int
        L.fa_bwd.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                             ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.fa_fwd_gqa.restype = ctypes.c_int
        L.fa_fwd_gqa.argtypes = L.fa_fwd.argtypes[:2] + [_i64] + L.fa_fwd.argtypes[2:]
        L.fa_bwd_gqa.restype = ctypes.c_int
        L.fa_bwd_gqa.argtypes = L.fa_bwd.argtypes[:2] + [_i64] + L.fa_bwd.argtypes[2:]
        # num_seqs, heads, heads_kv, total, max_seqlen, d, cu_seqlens, causal,
        # scale, dtype, then the tensors and the stream.
        _vl = [_i64, _i64, _i64, _i64, _i64, _i64, _vp, ctypes.c_int, ctypes.c_float,
               ctypes.c_int]
        _mp = ctypes.POINTER(FaMask)
        L.fa_fwd_varlen.restype = ctypes.c_int
        L.fa_fwd_varlen.argtypes = _vl + [_vp, _vp, _vp, _mp, _vp, _vp, _vp]
        L.fa_bwd_varlen.restype = ctypes.c_int
        L.fa_bwd_varlen.argtypes = _vl + [_vp] * 6 + [_mp] + [_vp] * 4 + [ctypes.c_size_t, _vp]
        L.fa_fwd_masked.restype = ctypes.c_int
        L.fa_fwd_masked.argtypes = L.fa_fwd_gqa.argtypes[:12] + [_mp] + L.fa_fwd_gqa.argtypes[12:]
        L.fa_bwd_masked.restype = ctypes.c_int
        L.fa_bwd_masked.argtypes = L.fa_bwd_gqa.argtypes[:15] + [_mp] + L.fa_bwd_gqa.argtypes[15:]
        L.fa_block_index_bytes.restype = ctypes.c_size_t
        L.fa_block_index_bytes.argtypes = [_i64]
        L.fa_block_index_build.restype = ctypes.c_int
        L.fa_block_index_build.argtypes = [_i64, _vp, _vp, _vp]
        L.fa_bwd_noalloc.restype = ctypes.c_int
        L.fa_bwd_noalloc.argtypes = L.fa_bwd_gqa.argtypes[:18] + [_vp]
        L.fa_bwd_timed.restype = ctypes.c_int
        L.fa_bwd_timed.argtypes = L.fa_bwd_gqa.argtypes + [ctypes.POINTER(_vp)]
        L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.fa_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
        L.fa_fp8_codes_bytes.restype = ctypes.c_size_t
        L.fa_fp8_codes_bytes.argtypes = [_i64, _i64, _i64, _i64]
        L.fa_fp8_scales_bytes.restype = ctypes.c_size_t
        L.fa_fp8_scales_bytes.argtypes = [_i64, _i64, _i64]
        L.fa_fp8_quantize.restype = ctypes.c_int
        L.fa_fp8_quantize.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                      _vp]
        L.fa_fwd_fp8.restype = ctypes.c_int
        L.fa_fwd_fp8.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.fa_status_str.restype = ctypes.c_char_p
        L.fa_status_str.argtypes = [ctypes.c_int]
        L.fa_abi_version.restype = ctypes.c_int
        L.fa_abi_version.argtypes = []
        if L.fa_abi_version() != ABI_VERSION:
            raise RuntimeError(
                f"{LIB_PATH} has ABI version {L.fa_abi_version()}, this binding "
                f"needs {ABI_VERSION}: rebuild it")
        _lib = L
        return L


def fa_fwd(batch, heads, n, d, causal, softmax_scale, dtype, q, k, v, kv_len,
           o, lse, stream) -> int:
    return lib().fa_fwd(batch, heads, n, d, int(causal), float(softmax_scale),
                        int(dtype), q, k, v, kv_len, o, lse, stream)


def fa_fwd_gqa(batch, heads, heads_kv, n, d, causal, softmax_scale, dtype, q, k,
               v, kv_len, o, lse, stream) -> int:
    return lib().fa_fwd_gqa(batch, heads, heads_kv, n, d, int(causal),
                            float(softmax_scale), int(dtype), q, k, v, kv_len, o,
                            lse, stream)


def _mref(mask):
    return None if mask is None else ctypes.byref(mask)


def fa_fwd_masked(batch, heads, heads_kv, n, d, causal, softmax_scale, dtype, q, k, v,
                  kv_len, mask, o, lse, stream) -> int:
    """``mask``: a FaMask (see ``mask_arg``) or None."""
    return lib().fa_fwd_masked(batch, heads, heads_kv, n, d, int(causal),
                               float(softmax_scale), int(dtype), q, k, v, kv_len,
                               _mref(mask), o, lse, stream)


def fa_bwd_masked(batch, heads, heads_kv, n, d, causal, softmax_scale, dtype, q, k, v, o,
                  d_o, lse, kv_len, mask, dq, dk, dv, workspace, workspace_bytes,
                  stream) -> int:
    return lib().fa_bwd_masked(batch, heads, heads_kv, n, d, int(causal),
                               float(softmax_scale), int(dtype), q, k, v, o, d_o, lse, kv_len,
                               _mref(mask), dq, dk, dv, workspace, int(workspace_bytes),
                               stream)


def fa_fwd_varlen(num_seqs, heads, heads_kv, total, max_seqlen, d, cu_seqlens, causal,
                  softmax_scale, dtype, q, k, v, mask, o, lse, stream) -> int:
    return lib().fa_fwd_varlen(num_seqs, heads, heads_kv, total, max_seqlen, d, cu_seqlens,
                               int(causal), float(softmax_scale), int(dtype), q, k, v,
                               _mref(mask), o, lse, stream)


def fa_bwd_varlen(num_seqs, heads, heads_kv, total, max_seqlen, d, cu_seqlens, causal,
                  softmax_scale, dtype, q, k, v, o, d_o, lse, mask, dq, dk, dv, workspace,
                  workspace_bytes, stream) -> int:
    return lib().fa_bwd_varlen(num_seqs, heads, heads_kv, total, max_seqlen, d, cu_seqlens,
                               int(causal), float(softmax_scale), int(dtype), q, k, v, o,
                               d_o, lse, _mref(mask), dq, dk, dv, workspace,
                               int(workspace_bytes), stream)


def fa_block_index_bytes(n) -> int:
    return int(lib().fa_block_index_bytes(n))


def fa_block_index_build(n, block_mask, index, stream) -> int:
    return lib().fa_block_index_build(n, block_mask, index, stream)


def fa_bwd(batch, heads, n, d, causal, softmax_scale, dtype, q, k, v, o, d_o,
           lse, kv_len, dq, dk, dv, workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd(batch, heads, n, d, int(causal), float(softmax_scale),
                        int(dtype), q, k, v, o, d_o, lse, kv_len, dq, dk, dv,
                        workspace, int(workspace_bytes), stream)


def fa_bwd_gqa(batch, heads, heads_kv, n, d, causal, softmax_scale, dtype, q, k,
               v, o, d_o, lse, kv_len, dq, dk, dv, workspace, workspace_bytes,
               stream) -> int:
    return lib().fa_bwd_gqa(batch, heads, heads_kv, n, d, int(causal),
                            float(softmax_scale), int(dtype), q, k, v, o, d_o, lse,
                            kv_len, dq, dk, dv, workspace, int(workspace_bytes),
                            stream)


def fa_bwd_noalloc(batch, heads, heads_kv, n, d, causal, softmax_scale, dtype, q, k, v, o,
                   d_o, lse, kv_len, dq, dk, dv, stream) -> int:
    return lib().fa_bwd_noalloc(batch, heads, heads_kv, n, d, int(causal),
                                float(softmax_scale), int(dtype), q, k, v, o, d_o, lse,
                                kv_len, dq, dk, dv, stream)


def fa_bwd_timed(batch, heads, heads_kv, n, d, causal, softmax_scale, dtype, q, k,
                 v, o, d_o, lse, kv_len, dq, dk, dv, workspace, workspace_bytes,
                 stream, events) -> int:
    """``events``: four raw hipEvent_t handles (ints or None), or None."""
    arr = None
    if events is not None:
        arr = (_vp * 4)(*[e if e else None for e in events])
    return lib().fa_bwd_timed(batch, heads, heads_kv, n, d, int(causal),
                              float(softmax_scale), int(dtype), q, k, v, o, d_o,
                              lse, kv_len, dq, dk, dv, workspace,
                              int(workspace_bytes), stream, arr)


def fa_bwd_workspace_bytes(batch, heads, n, d, dtype) -> int:
    return int(lib().fa_bwd_workspace_bytes(batch, heads, n, d, int(dtype)))


def fa_fp8_codes_bytes(batch, heads, n, d) -> int:
    return int(lib().fa_fp8_codes_bytes(batch, heads, n, d))


def fa_fp8_scales_bytes(batch, heads, n) -> int:
    return int(lib().fa_fp8_scales_bytes(batch, heads, n))


def fa_fp8_quantize(batch, heads, n, d, layout, x, signs, codes, scales, stream) -> int:
    return lib().fa_fp8_quantize(batch, heads, n, d, int(layout), x, signs, codes, scales,
                                 stream)


def fa_fwd_fp8(batch, heads, heads_kv, n, d, causal, softmax_scale, q8, q_scales, k8,
               k_scales, v8, v_scales, kv_len, o, lse, stream) -> int:
    return lib().fa_fwd_fp8(batch, heads, heads_kv, n, d, int(causal), float(softmax_scale),
                            q8, q_scales, k8, k_scales, v8, v_scales, kv_len, o, lse, stream)


def fa_status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def fa_abi_version() -> int:
    return int(lib().fa_abi_version())


def check(status: int) -> None:
    """Raise RuntimeError carrying the library's message for a non-OK status."""
    if status != FA_OK:
        raise RuntimeError(fa_status_str(status))
