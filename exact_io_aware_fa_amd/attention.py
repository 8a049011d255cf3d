"""PyTorch-facing calls: allocate outputs and workspace with torch, pass raw
pointers and torch's current HIP stream to the C ABI.

PyTorch supplies device memory and streams only; every step of the forward
and backward runs in the library's HIP kernels. There is no CPU or eager
fallback: a CPU tensor or a missing library is an error.
"""

from __future__ import annotations

import math

import torch

from . import binding as _b

_DTYPES = {torch.bfloat16: _b.FA_BF16, torch.float32: _b.FA_FP32}


def _on_device(ref, named, layout):
    """Every tensor in ``named`` must be a contiguous GPU tensor on ref's
    device (the library receives raw device pointers; a host pointer or a
    pointer into another GPU's memory would be read by the kernels)."""
    for name, t in named:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, q on {ref.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous {layout}")


def _check_qkv(q, k, v, devices=True):
    # Shapes and dtypes first, then devices: every check runs on the host
    # before anything is launched.
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [batch, heads, n, d] and k, v one "
                         "[batch, heads_kv, n, d] shape")
    b, h, n, d = q.shape
    hkv = k.shape[1]
    if k.shape[0] != b or k.shape[2:] != q.shape[2:] or hkv < 1 or h % hkv:
        raise ValueError("k and v need q's batch, n and d, and a head count "
                         "heads_kv that divides q's")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if devices:
        _on_device(q, (("q", q), ("k", k), ("v", v)), "[batch, heads, n, d]")
    return hkv


def _check_saved(q, k, v, o, lse, do, lse_shape):
    """The backward's extra inputs: o and do shaped and typed like q, lse the
    forward's float32 logsumexp of shape ``lse_shape``; then every tensor on
    q's device (after all shape checks, so that a wrong shape is reported
    before a wrong device)."""
    if o.shape != q.shape or do.shape != q.shape or o.dtype != q.dtype or do.dtype != q.dtype:
        raise ValueError("o and do must match q in shape and dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(lse_shape):
        raise ValueError(f"lse must be float32 of shape {list(lse_shape)} (the forward's)")
    _on_device(q, (("q", q), ("k", k), ("v", v)), "")
    for name, t in (("o", o), ("do", do), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")


def _kv_len_arg(kv_len, batch, n, device):
    """int32 device tensor of key lengths (checked to lie in [1, n]), or None."""
    if kv_len is None:
        return None
    t = torch.as_tensor(kv_len)
    if t.numel() != batch:
        raise ValueError(f"kv_len must have {batch} entries")
    host = t.detach().to("cpu", torch.int64).reshape(-1)
    if int(host.min()) < 1 or int(host.max()) > n:
        raise ValueError(f"kv_len entries must lie in [1, {n}]")
    return host.to(torch.int32).to(device)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def build_block_index(block_mask, n):
    """Block-sparse index (int32 GPU tensor) of a boolean block mask for
    sequences of length n: block_mask[i][j] keeps key block j (keys
    j*128 .. j*128+127) for query block i; both dimensions ceil(n / 128).
    Built on the GPU by the library; reuse it for every call with that mask."""
    nb = (int(n) + _b.FA_BLOCK - 1) // _b.FA_BLOCK
    if tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be [{nb}, {nb}] for n = {n}")
    if not block_mask.is_cuda:
        raise ValueError("block_mask must be a GPU tensor")
    m = block_mask.to(torch.uint8).contiguous()
    nbytes = _b.fa_block_index_bytes(int(n))
    if nbytes == 0:
        raise ValueError(f"block masks support n <= {1024 * _b.FA_BLOCK}")
    index = torch.empty(nbytes // 4, dtype=torch.int32, device=block_mask.device)
    _b.check(_b.fa_block_index_build(int(n), m.data_ptr(), index.data_ptr(), _stream()))
    return index


def _mask(window, block_index, n):
    if block_index is not None:
        if not block_index.is_cuda or block_index.dtype != torch.int32:
            raise ValueError("block_index must come from build_block_index")
        if block_index.numel() * 4 != _b.fa_block_index_bytes(int(n)):
            raise ValueError("block_index was built for another sequence length")
    window = (-1, -1) if window is None else tuple(int(x) for x in window)
    if len(window) != 2 or min(window) < -1:
        raise ValueError("window must be (left, right) with -1 for an unbounded side")
    return _b.mask_arg(window, None if block_index is None else block_index.data_ptr())


def flash_attn_fwd(q, k, v, causal=False, softmax_scale=None, kv_len=None, window=None,
                   block_index=None):
    """Forward: returns (o, lse); o like q, lse float32 [batch, heads, n].

    k and v may have fewer heads than q (grouped or multi-query attention):
    query head i then uses K/V head i // (heads // heads_kv). ``window`` =
    (left, right) keeps keys i-left .. i+right (-1: unbounded);
    ``block_index`` (from ``build_block_index``) applies a block mask."""
    hkv = _check_qkv(q, k, v)
    b, h, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    kvl = _kv_len_arg(kv_len, b, n, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    mask = _mask(window, block_index, n)
    _b.check(_b.fa_fwd_masked(b, h, hkv, n, d, causal, scale, _DTYPES[q.dtype],
                              q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              None if kvl is None else kvl.data_ptr(), mask,
                              o.data_ptr(), lse.data_ptr(), _stream()))
    return o, lse


def flash_attn_bwd(q, k, v, o, lse, do, causal=False, softmax_scale=None,
                   kv_len=None, window=None, block_index=None):
    """Backward from the saved LSE: returns (dq, dk, dv); dk, dv shaped like
    k, v (summed over each K/V head's group of query heads)."""
    hkv = _check_qkv(q, k, v, devices=False)
    b, h, n, d = q.shape
    _check_saved(q, k, v, o, lse, do, (b, h, n))
    o, do, lse = o.contiguous(), do.contiguous(), lse.contiguous()
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    kvl = _kv_len_arg(kv_len, b, n, q.device)
    dt = _DTYPES[q.dtype]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = _b.fa_bwd_workspace_bytes(b, h, n, d, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    mask = _mask(window, block_index, n)
    _b.check(_b.fa_bwd_masked(b, h, hkv, n, d, causal, scale, dt,
                              q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              do.data_ptr(), lse.data_ptr(),
                              None if kvl is None else kvl.data_ptr(), mask,
                              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                              ws.data_ptr(), ws_bytes, _stream()))
    return dq, dk, dv


def _check_packed(q, k, v, devices=True):
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("q must be [heads, total, d] and k, v one [heads_kv, total, d] shape")
    h, total, d = q.shape
    hkv = k.shape[0]
    if k.shape[1:] != q.shape[1:] or hkv < 1 or h % hkv:
        raise ValueError("k and v need q's total and d, and a head count heads_kv that "
                         "divides q's")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if devices:
        _on_device(q, (("q", q), ("k", k), ("v", v)), "[heads, total, d]")
    return hkv


def _cu_seqlens_arg(cu_seqlens, total, max_seqlen, device):
    """(device int32 offsets, num_seqs, max_seqlen), checked on the host:
    they start at 0, never decrease and end at total."""
    host = torch.as_tensor(cu_seqlens).detach().to("cpu", torch.int64).reshape(-1)
    if host.numel() < 2 or int(host[0]) != 0 or int(host[-1]) != total:
        raise ValueError(f"cu_seqlens must run from 0 to total = {total}")
    lens = host[1:] - host[:-1]
    if int(lens.min()) < 0:
        raise ValueError("cu_seqlens must be non-decreasing")
    longest = max(int(lens.max()), 1)
    if max_seqlen is None:
        max_seqlen = longest
    elif int(max_seqlen) < longest:
        raise ValueError(f"max_seqlen {max_seqlen} is below the longest sequence {longest}")
    return host.to(torch.int32).to(device), host.numel() - 1, int(max_seqlen)


def flash_attn_varlen_fwd(q, k, v, cu_seqlens, max_seqlen=None, causal=False,
                          softmax_scale=None, window=None, block_index=None):
    """Forward over a packed variable-length batch: q [heads, total, d], k, v
    [heads_kv, total, d]; sequence s is rows cu_seqlens[s]..cu_seqlens[s+1]-1
    of every head and attends only to itself. Returns (o like q, lse float32
    [heads, total])."""
    hkv = _check_packed(q, k, v)
    h, total, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    cu, nseq, mx = _cu_seqlens_arg(cu_seqlens, total, max_seqlen, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((h, total), dtype=torch.float32, device=q.device)
    mask = _mask(window, block_index, mx)
    _b.check(_b.fa_fwd_varlen(nseq, h, hkv, total, mx, d, cu.data_ptr(), causal, scale,
                              _DTYPES[q.dtype], q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              mask, o.data_ptr(), lse.data_ptr(), _stream()))
    return o, lse


def flash_attn_varlen_bwd(q, k, v, o, lse, do, cu_seqlens, max_seqlen=None, causal=False,
                          softmax_scale=None, window=None, block_index=None):
    """Backward of ``flash_attn_varlen_fwd`` from the saved LSE: returns
    (dq, dk, dv) shaped like q, k, v."""
    hkv = _check_packed(q, k, v, devices=False)
    h, total, d = q.shape
    _check_saved(q, k, v, o, lse, do, (h, total))
    o, do, lse = o.contiguous(), do.contiguous(), lse.contiguous()
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    cu, nseq, mx = _cu_seqlens_arg(cu_seqlens, total, max_seqlen, q.device)
    dt = _DTYPES[q.dtype]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = _b.fa_bwd_workspace_bytes(nseq, h, mx, d, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    mask = _mask(window, block_index, mx)
    _b.check(_b.fa_bwd_varlen(nseq, h, hkv, total, mx, d, cu.data_ptr(), causal, scale, dt,
                              q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              do.data_ptr(), lse.data_ptr(), mask, dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws_bytes,
                              _stream()))
    return dq, dk, dv


class FlashAttentionFunction(torch.autograd.Function):
    """Autograd wrapper: saves q, k, v, o and the LSE; recomputes P in the
    backward kernel."""

    @staticmethod
    def forward(ctx, q, k, v, causal, softmax_scale, kv_len, window, block_index):
        o, lse = flash_attn_fwd(q, k, v, causal, softmax_scale, kv_len, window, block_index)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (causal, softmax_scale, kv_len, window, block_index)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = flash_attn_bwd(q, k, v, o, lse, do.contiguous(), *ctx.args)
        return dq, dk, dv, None, None, None, None, None


def flash_attention(q, k, v, causal=False, softmax_scale=None, kv_len=None, window=None,
                    block_index=None):
    """O = softmax(scale * Q K^T + mask) V with autograd support."""
    return FlashAttentionFunction.apply(q, k, v, causal, softmax_scale, kv_len, window,
                                        block_index)


class FlashAttentionVarlenFunction(torch.autograd.Function):
    """Autograd wrapper of the packed variable-length calls."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, causal, softmax_scale, window,
                block_index):
        o, lse = flash_attn_varlen_fwd(q, k, v, cu_seqlens, max_seqlen, causal, softmax_scale,
                                       window, block_index)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (cu_seqlens, max_seqlen, causal, softmax_scale, window, block_index)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = flash_attn_varlen_bwd(q, k, v, o, lse, do.contiguous(), *ctx.args)
        return dq, dk, dv, None, None, None, None, None, None


def flash_attention_varlen(q, k, v, cu_seqlens, max_seqlen=None, causal=False,
                           softmax_scale=None, window=None, block_index=None):
    """Packed variable-length attention with autograd support."""
    return FlashAttentionVarlenFunction.apply(q, k, v, cu_seqlens, max_seqlen, causal,
                                              softmax_scale, window, block_index)


# ---------------------------------------------------------------------------
# FP8 (E4M3) forward: encode Q, K, V per 128-row block, then attend on the
# codes (page 2, "4. FlashAttention 深度剖析", 4.5.4).

def _fp8_rows(n):
    return (n + _b.FA_BLOCK - 1) // _b.FA_BLOCK * _b.FA_BLOCK


def hadamard_signs(d, generator=None, device="cuda"):
    """Random +-1 signs (int8 GPU tensor of length d) for the rotation
    diag(signs) H_d of Q and K; draw one vector per model and reuse it."""
    bits = torch.randint(0, 2, (d,), generator=generator, dtype=torch.int8)
    return (2 * bits - 1).to(torch.int8).to(device)


def fp8_quantize(x, signs=None, layout="rows"):
    """E4M3 codes and per-block scales of a bf16 tensor x [batch, heads, n, d].

    layout "rows": codes [batch, heads, np, d]; "vt": codes
    [batch, heads, np / 128, d, 128] (each block transposed, the V layout).
    scales: float32 [batch, heads, np / 128]. With ``signs`` (int8 [d]) the
    rows are rotated by diag(signs) H_d first (Q and K only)."""
    if not x.is_cuda or x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 GPU tensor [batch, heads, n, d]")
    b, h, n, d = x.shape
    np_ = _fp8_rows(n)
    vt = layout == "vt"
    if layout not in ("rows", "vt"):
        raise ValueError("layout must be 'rows' or 'vt'")
    shape = (b, h, np_ // _b.FA_BLOCK, d, _b.FA_BLOCK) if vt else (b, h, np_, d)
    codes = torch.empty(shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty((b, h, np_ // _b.FA_BLOCK), dtype=torch.float32, device=x.device)
    if signs is not None:
        if signs.dtype != torch.int8 or signs.numel() != d or not signs.is_cuda:
            raise ValueError(f"signs must be an int8 GPU tensor of {d} entries")
        signs = signs.contiguous()
    _b.check(_b.fa_fp8_quantize(b, h, n, d, _b.FA_FP8_VT if vt else _b.FA_FP8_ROWS,
                                x.data_ptr(), signs.data_ptr() if signs is not None else None,
                                codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def flash_attn_fp8_fwd_codes(q8, q_scales, k8, k_scales, v8, v_scales, n, causal=False,
                             softmax_scale=None, kv_len=None):
    """FP8 forward on encoded operands (``fp8_quantize`` layouts: q8, k8
    "rows", v8 "vt"). Returns (o bf16 [batch, heads, n, d], lse float32)."""
    if q8.dim() != 4 or k8.dim() != 4:
        raise ValueError("q8 and k8 must be [batch, heads, np, d] codes")
    b, h, np_, d = q8.shape
    hkv = k8.shape[1]
    if np_ != _fp8_rows(n) or k8.shape != (b, hkv, np_, d) or \
            v8.shape != (b, hkv, np_ // _b.FA_BLOCK, d, _b.FA_BLOCK):
        raise ValueError("codes do not match the fp8_quantize layouts for this n")
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if t.dtype != torch.uint8:
            raise ValueError(f"{name} must be uint8 E4M3 codes")
    nb = np_ // _b.FA_BLOCK
    for name, t, hh in (("q_scales", q_scales, h), ("k_scales", k_scales, hkv),
                        ("v_scales", v_scales, hkv)):
        if t.dtype != torch.float32 or tuple(t.shape) != (b, hh, nb):
            raise ValueError(f"{name} must be float32 of shape {[b, hh, nb]}")
    _on_device(q8, (("q8", q8), ("k8", k8), ("v8", v8), ("q_scales", q_scales),
                    ("k_scales", k_scales), ("v_scales", v_scales)), "(fp8_quantize layout)")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = torch.empty((b, h, n, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=q8.device)
    kl = _kv_len_arg(kv_len, b, n, q8.device)
    _b.check(_b.fa_fwd_fp8(b, h, hkv, n, d, causal, scale, q8.data_ptr(), q_scales.data_ptr(),
                           k8.data_ptr(), k_scales.data_ptr(), v8.data_ptr(),
                           v_scales.data_ptr(), kl.data_ptr() if kl is not None else None,
                           o.data_ptr(), lse.data_ptr(), _stream()))
    return o, lse


def flash_attn_fp8_fwd(q, k, v, causal=False, softmax_scale=None, kv_len=None, signs=None):
    """FP8 attention forward from bf16 q [batch, heads, n, d] and k, v
    [batch, heads_kv, n, d]: Q and K are encoded per block (rotated by
    diag(signs) H_d when ``signs`` is given), V per block in the transposed
    layout, then both products run on the E4M3 matrix cores. Returns
    (o bf16, lse float32)."""
    _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("the FP8 forward takes bfloat16 inputs")
    q8, qs = fp8_quantize(q, signs)
    k8, ks = fp8_quantize(k, signs)
    v8, vs = fp8_quantize(v, layout="vt")
    return flash_attn_fp8_fwd_codes(q8, qs, k8, ks, v8, vs, q.shape[2], causal, softmax_scale,
                                    kv_len)
