"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
(via the torch wrappers) and the fp64 oracle on identical seeded inputs, and
compare them under the stated tolerances.

Tolerances (floating point; masking and indexing are checked bit-exactly in
test_masks_gpu.py):
* fp32 path: normwise relative error ||g - o||_inf / ||o||_inf <= 1e-5 for O
  and for dQ, dK, dV; LSE within 1e-5 * max(1, |L|).
* bf16 path: O within 1e-2 absolute (max over elements) for unit-variance
  inputs; for peaky rows (Q, K with std 3) the final bf16 rounding alone
  exceeds 1e-2 once |O| >= 4, so there the bound is 1e-2 + 2^-8 |o|
  elementwise (one bf16 unit roundoff of the output cast). dQ, dK, dV within
  2e-2 normwise relative error. LSE within 1e-3 absolute.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from exact_io_aware_fa_amd import attention as fa
from exact_io_aware_fa_amd.inputs import make_inputs

BF16_O_ABS = 1e-2
BF16_GRAD_REL = 2e-2
BF16_LSE_ABS = 1e-3
FP32_REL = 1e-5


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).double().numpy()


def normwise_rel(got, ref) -> float:
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def to_gpu(inp: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_gpu(w, inp, backward=True, window=None, block_index=None):
    g = to_gpu(inp)
    o, lse = fa.flash_attn_fwd(g["q"], g["k"], g["v"], w.causal, w.softmax_scale, g["kv_len"],
                               window, block_index)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = fa.flash_attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], w.causal,
                                       w.softmax_scale, g["kv_len"], window, block_index)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def kv_len_of(inp, b):
    return None if inp["kv_len"] is None else int(inp["kv_len"][b])


def group_of(inp) -> int:
    """Query heads per K/V head (1 for ordinary multi-head inputs)."""
    return inp["q"].shape[1] // inp["k"].shape[1]


def _lse_close(got, ref, tol_abs=None, tol_rel=None):
    """LSE comparison: rows with no visible key must be -inf on both sides,
    the others within the tolerance."""
    empty = ref == -np.inf
    assert np.array_equal(got == -np.inf, empty), "rows without visible keys differ"
    g, r = got[~empty], ref[~empty]
    if tol_rel is not None:
        return bool(np.all(np.abs(g - r) <= tol_rel * np.maximum(1.0, np.abs(r))))
    return bool(np.all(np.abs(g - r) <= tol_abs))


def check_forward_head(w, inp, gpu, b, h, rows=None, peaky=False, window=(-1, -1),
                       block_mask=None):
    """Compare O and LSE of query head (b, h) (optionally only query
    ``rows``); K and V come from the K/V head that query head uses."""
    j = h // group_of(inp)
    q = f64(inp["q"][b, h])
    k, v = (f64(inp[x][b, j]) for x in ("k", "v"))
    ref = oracle.head_forward(q, k, v, w.softmax_scale, w.causal, kv_len_of(inp, b), rows=rows,
                              window=window, block_mask=block_mask)
    go = f64(gpu["o"][b, h])
    gl = gpu["lse"][b, h].cpu().double().numpy()
    if rows is not None:
        go, gl = go[rows], gl[rows]
    if w.dtype == "fp32":
        assert normwise_rel(go, ref["o"]) <= FP32_REL, (b, h, normwise_rel(go, ref["o"]))
        assert _lse_close(gl, ref["lse"], tol_rel=FP32_REL), (b, h)
    else:
        err = np.abs(go - ref["o"])
        bound = BF16_O_ABS + (2.0 ** -8) * np.abs(ref["o"]) if peaky else BF16_O_ABS
        assert np.all(err <= bound), (b, h, float(err.max()))
        assert _lse_close(gl, ref["lse"], tol_abs=BF16_LSE_ABS), (b, h)
    return ref


def check_backward_head(w, inp, gpu, b, h, window=(-1, -1), block_mask=None):
    """Compare dQ of query head (b, h) and dK, dV of the K/V head it uses.
    With grouped K/V heads the oracle runs every query head of that group
    and sums their dK and dV (the gradient of a shared head), and the dQ of
    each of them is compared too."""
    grp = group_of(inp)
    j = h // grp
    k, v = (f64(inp[x][b, j]) for x in ("k", "v"))
    tol = FP32_REL if w.dtype == "fp32" else BF16_GRAD_REL
    errs = {}
    dk = dv = 0.0
    for hh in range(j * grp, (j + 1) * grp):
        q, do = (f64(inp[x][b, hh]) for x in ("q", "do"))
        ref = oracle.head_backward(q, k, v, do, w.softmax_scale, w.causal, kv_len_of(inp, b),
                                   window, block_mask)
        errs[f"dq{hh}"] = normwise_rel(f64(gpu["dq"][b, hh]), ref["dq"])
        dk = dk + ref["dk"]
        dv = dv + ref["dv"]
    errs["dk"] = normwise_rel(f64(gpu["dk"][b, j]), dk)
    errs["dv"] = normwise_rel(f64(gpu["dv"][b, j]), dv)
    assert all(e <= tol for e in errs.values()), (b, h, errs)
    return errs


def workload_inputs(w):
    return make_inputs(w, with_grad_out=w.backward)
