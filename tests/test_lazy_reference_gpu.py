"""Parity for rows whose running maximum climbs far past the reference taken
on their first key tiles.

The per-block update of the online softmax (page 1, "FlashAttention
原理深入剖析（上篇）", section 六; page 2, "4. FlashAttention 深度剖析", 4.2.4:
merging two (m, l, O~) states rescales the one with the smaller m) lets the
bf16 forward kernels hold a row's reference fixed while its running max stays
within 64 (base 2) of it, and move it, rescaling O~ and l, only past that.
The fp8 forward does the same with the frame its accumulators are kept in.
Unit-variance inputs, and the std-3 ones of the long causal workload, never
take that branch: a row's max does not climb 64 binary orders after its
first tile. The inputs here are shaped so that it does: query rows are scaled
by 2^-6, 1, 2, 4 in turn and the keys by 1, 2, 4, 8, 16 over successive
blocks of 150 keys (powers of two, so bf16 values stay exact). About half
the rows then move their reference one to three times mid-row while the
rows beside them in the same 64-row tile do not. A host test counts the
moves on 64- and 128-key tiles to show that the shaping does force them.

Every forward kernel is covered: d = 64, 128 and 256 dense (causal or not,
key padding), d = 128 with a window, d = 128 and 256 block-sparse (their own
kernels), fp32 (which keeps no lazy reference; its bound below accounts for
fp32 score rounding at these magnitudes), and fp8 on the oracle's codes.
The bf16 backward, which recomputes P from the stored L = m + log l, is
compared too.
"""

import math

import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd.inputs import custom, make_inputs
from parity_utils import (FP32_REL, check_backward_head, check_forward_head, f64,
                          normwise_rel, run_gpu)

Q_SCALES = (2.0 ** -6, 1.0, 2.0, 4.0)   # per query row, in turn
K_BLOCK = 150
K_SCALES = (1.0, 2.0, 4.0, 8.0, 16.0)   # per block of K_BLOCK keys
LAZY = 64.0                              # the kernels' reference lag bound, base 2


def shape_inputs(inp):
    """Scale query rows and key blocks by powers of two (exact in bf16)."""
    n = inp["q"].shape[2]
    qs = torch.tensor([Q_SCALES[i % len(Q_SCALES)] for i in range(n)])
    ks = torch.tensor([K_SCALES[min(j // K_BLOCK, len(K_SCALES) - 1)] for j in range(n)])
    out = dict(inp)
    out["q"] = (inp["q"].float() * qs[None, None, :, None]).to(inp["q"].dtype)
    out["k"] = (inp["k"].float() * ks[None, None, :, None]).to(inp["k"].dtype)
    return out


def _moves(q, k, scale, causal, tile):
    """Reference moves per row of a kernel that walks keys in tiles of
    ``tile``, sets the reference to the running max (base 2) at its first
    visible tile and moves it to the running max when that runs more than
    LAZY above it."""
    n = q.shape[0]
    t = scale * (q @ k.T) / math.log(2.0)
    if causal:
        t = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], t, -np.inf)
    count = np.zeros(n, dtype=np.int64)
    for i in range(n):
        ref, m = None, -np.inf
        for j0 in range(0, n, tile):
            m = max(m, t[i, j0:j0 + tile].max())
            if not np.isfinite(m):
                continue
            if ref is None:
                ref = m
            elif m > ref + LAZY:
                ref, count[i] = m, count[i] + 1
    return count


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_shaped_inputs_force_reference_moves(d, causal):
    w = custom("lazy", 1, 1, 700, d, "bf16", causal, seed=3)
    inp = shape_inputs(make_inputs(w, with_grad_out=False))
    q, k = f64(inp["q"][0, 0]), f64(inp["k"][0, 0])
    for tile in (64, 128):
        c = _moves(q, k, w.softmax_scale, causal, tile)
        assert (c >= 2).sum() >= 10, tile            # rows that move more than once
        moving = [(c[g:g + 64] > 0).sum() for g in range(0, 700, 64)]
        # Tiles of 64 rows where some rows move and others do not.
        assert sum(0 < x < 64 for x in moving) >= (4 if causal else 10), (tile, moving)


BF16_CASES = [
    # (n, d, causal, padded, window, sparse)
    (700, 64, False, False, None, False),
    (700, 64, True, False, None, False),
    (700, 128, False, True, None, False),
    (700, 128, True, False, None, False),
    (700, 256, False, False, None, False),
    (700, 256, True, True, None, False),
    (1100, 64, True, False, None, False),
    (700, 128, True, False, (400, -1), False),
    (700, 128, True, False, None, True),
    (700, 256, False, False, None, True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("n,d,causal,padded,window,sparse", BF16_CASES)
def test_bf16_forward_and_backward_with_reference_moves(n, d, causal, padded, window, sparse):
    from exact_io_aware_fa_amd import attention as fa
    w = custom(f"lazy_n{n}_d{d}", 2, 2, n, d, "bf16", causal, seed=n + d + 31, padded=padded)
    inp = shape_inputs(make_inputs(w))
    nb = (n + 127) // 128
    bm = None
    if sparse:
        rng = np.random.default_rng(n + d)
        bm = rng.random((nb, nb)) < 0.7
        np.fill_diagonal(bm, True)
    print(f"[lazy] bf16 n={n} d={d} causal={causal} padded={padded} window={window} "
          f"sparse={sparse}", flush=True)
    idx = fa.build_block_index(torch.from_numpy(bm).cuda(), n) if sparse else None
    gpu = run_gpu(w, inp, window=window, block_index=idx)
    win = (-1, -1) if window is None else window
    for b, h in ((0, 0), (1, 1)):
        check_forward_head(w, inp, gpu, b, h, peaky=True, window=win, block_mask=bm)
        check_backward_head(w, inp, gpu, b, h, window=win, block_mask=bm)


@pytest.mark.gpu
@pytest.mark.parametrize("d,causal", [(64, True), (128, False), (256, True)])
def test_fp32_forward_with_large_score_jumps(d, causal):
    """fp32 forward on the shaped inputs. Its scores carry the rounding of an
    fp32 dot product, |dS_ij| <= E = gamma_d scale sum_k |q_ik k_jk| with
    gamma_d = d 2^-24 (the standard a-priori bound), and a score error of at
    most E moves each softmax weight by a factor within exp(+-2E), so O
    moves by at most 2E max|v| (to first order) on top of the fp32 bound
    used elsewhere."""
    import oracle
    w = custom(f"lazy32_d{d}", 1, 2, 600, d, "fp32", causal, seed=d + 7)
    inp = shape_inputs(make_inputs(w, with_grad_out=False))
    print(f"[lazy] fp32 d={d} causal={causal}", flush=True)
    gpu = run_gpu(w, inp, backward=False)
    for h in range(2):
        q, k, v = (f64(inp[x][0, h]) for x in ("q", "k", "v"))
        ref = oracle.head_forward(q, k, v, w.softmax_scale, causal)
        e = d * 2.0 ** -24 * abs(w.softmax_scale) * (np.abs(q) @ np.abs(k).T).max()
        tol = FP32_REL + 2.0 * e * np.abs(v).max() / np.abs(ref["o"]).max()
        err = normwise_rel(f64(gpu["o"][0, h]), ref["o"])
        assert err <= tol, (h, err, tol)
        lse = gpu["lse"][0, h].cpu().double().numpy()
        assert np.all(np.abs(lse - ref["lse"]) <= FP32_REL * np.maximum(1, np.abs(ref["lse"]))
                      + e), h


@pytest.mark.gpu
@pytest.mark.parametrize("d,causal", [(64, False), (128, True), (256, False)])
def test_fp8_forward_with_frame_moves(d, causal):
    """fp8 forward on the oracle's codes of the shaped inputs, under the same
    per-element bound as the other fp8 forward cases. The accumulators'
    frame moves by a power of two, so the result does not depend on when it
    moves."""
    from test_fp8_gpu import _check_head, _run_codes
    n = 700
    w = custom(f"lazy8_d{d}", 1, 2, n, d, "bf16", causal, seed=d + 11)
    inp = shape_inputs(make_inputs(w, with_grad_out=False))
    print(f"[lazy] fp8 d={d} causal={causal}", flush=True)
    sc = w.softmax_scale
    (qc, qs, kc, ks, vc, vs), o, lse = _run_codes(inp["q"], inp["k"], inp["v"], n, causal, sc,
                                                  None)
    for h in range(2):
        _check_head(o[0, h], lse[0, h], qc[0, h], qs[0, h], kc[0, h], ks[0, h], vc[0, h],
                    vs[0, h], n, sc, causal, None)
