"""GPU parity for sliding windows and block-sparse masks (page 4,
"FlashAttention 原理深入剖析（下篇）", section 六: the flash-attn call's
window_size; page 2, "4. FlashAttention 深度剖析", 4.8.1: Mistral's sliding
window; page 3, "深入浅出 FlashAttention", 第八部分: block-sparse attention with
a coarse block-level mask whose empty blocks are skipped).

A window (left, right) keeps keys i-left .. i+right; a block mask keeps the
128 x 128 blocks it sets. Small cases compare the HIP path through the C ABI
with the fp64 oracle head by head (O, LSE, dQ, dK, dV), over causal and key
padding, grouped heads, packed batches, d = 64/128/256, bf16 and fp32,
including rows that see no key at all. The block index the library builds
is compared entry by entry with one computed on the host. At the long
sizes (32 heads x 16384 rows, d = 128) seeded rows are compared with the
oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa_amd import attention as fa
from exact_io_aware_fa_amd import binding as B
from exact_io_aware_fa_amd.inputs import PackedWorkload, custom, make_inputs, make_packed_inputs
from parity_utils import (BF16_GRAD_REL, BF16_LSE_ABS, BF16_O_ABS, FP32_REL,
                          check_backward_head, check_forward_head, f64, normwise_rel, run_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _block_mask(n, seed, density=0.6):
    nb = (n + 127) // 128
    rng = np.random.default_rng(seed)
    bm = rng.random((nb, nb)) < density
    np.fill_diagonal(bm, True)
    return bm


def _host_index(bm):
    nb = bm.shape[0]
    row_ptr, col_idx, col_ptr, row_idx = [0], [], [0], []
    for r in range(nb):
        cols = [j for j in range(nb) if bm[r, j]]
        col_idx += cols
        row_ptr.append(len(col_idx))
    for c in range(nb):
        rows = [i for i in range(nb) if bm[i, c]]
        row_idx += rows
        col_ptr.append(len(row_idx))
    return row_ptr, col_idx, col_ptr, row_idx


@pytest.mark.parametrize("n,density", [(1, 1.0), (300, 0.5), (2000, 0.3), (9000, 0.4)])
def test_block_index_matches_host(n, density):
    bm = _block_mask(n, seed=n, density=density)
    idx = fa.build_block_index(torch.from_numpy(bm).cuda(), n)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    nb = bm.shape[0]
    row_ptr, col_idx, col_ptr, row_idx = _host_index(bm)
    assert list(got[:nb + 1]) == row_ptr
    assert list(got[nb + 1:nb + 1 + len(col_idx)]) == col_idx
    o = nb + 1 + nb * nb
    assert list(got[o:o + nb + 1]) == col_ptr
    assert list(got[o + nb + 1:o + nb + 1 + len(row_idx)]) == row_idx


CASES = [
    # (n, d, causal, dtype, padded, window, sparse, heads, heads_kv)
    (300, 64, False, "bf16", False, (37, 5), False, 2, 2),
    (300, 128, True, "bf16", True, (100, -1), False, 4, 2),
    (520, 256, False, "bf16", False, (-1, 60), False, 2, 1),
    (700, 64, True, "bf16", False, (-1, -1), True, 2, 2),
    (640, 64, True, "bf16", False, (200, -1), True, 4, 2),
    (520, 64, False, "bf16", True, (90, 90), True, 2, 1),
    (1500, 64, True, "bf16", True, (300, -1), True, 2, 1),
    (700, 128, False, "bf16", True, (150, 150), True, 2, 1),
    (640, 128, True, "bf16", False, (200, -1), True, 4, 4),
    (500, 256, True, "bf16", False, (-1, -1), True, 2, 2),
    (777, 256, False, "bf16", True, (200, 100), True, 2, 1),
    (900, 256, True, "bf16", False, (300, -1), True, 4, 2),
    (300, 64, True, "fp32", True, (40, -1), False, 2, 2),
    (400, 128, False, "fp32", False, (-1, 90), True, 2, 1),
    (390, 256, True, "fp32", False, (64, -1), True, 2, 2),
]


@pytest.mark.parametrize("n,d,causal,dtype,padded,window,sparse,heads,heads_kv", CASES)
def test_window_and_block_masks_against_oracle(n, d, causal, dtype, padded, window, sparse,
                                               heads, heads_kv):
    w = custom(f"mask_n{n}_d{d}", 2, heads, n, d, dtype, causal, seed=n + 3 * d, padded=padded,
               heads_kv=heads_kv)
    inp = make_inputs(w)
    bm = _block_mask(n, seed=n + d) if sparse else None
    idx = fa.build_block_index(torch.from_numpy(bm).cuda(), n) if sparse else None
    print(f"[parity] masks n={n} d={d} causal={causal} {dtype} padded={padded} window={window} "
          f"sparse={sparse} heads={heads}/{heads_kv}", flush=True)
    gpu = run_gpu(w, inp, window=window, block_index=idx)
    for b, h in ((0, 0), (1, heads - 1)):
        check_forward_head(w, inp, gpu, b, h, window=window, block_mask=bm)
        check_backward_head(w, inp, gpu, b, h, window=window, block_mask=bm)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rows_without_visible_keys(dtype):
    # Keys 0..49 only (padding), window 10 to the left, causal: rows >= 61 see
    # no key -> O = 0, LSE = -inf, zero dQ; dK, dV finite and still exact.
    w = custom("empty_rows", 1, 2, 200, 64, dtype, True, seed=9)
    inp = make_inputs(w)
    inp["kv_len"] = torch.tensor([50], dtype=torch.int32)
    gpu = run_gpu(w, inp, window=(10, -1))
    assert torch.all(gpu["o"][0, :, 61:] == 0)
    assert torch.all(gpu["lse"][0, :, 61:] == -float("inf"))
    assert torch.all(gpu["dq"][0, :, 61:] == 0)
    for name in ("dk", "dv"):
        assert torch.isfinite(gpu[name]).all()
    for h in range(2):
        check_forward_head(w, inp, gpu, 0, h, window=(10, -1))
        check_backward_head(w, inp, gpu, 0, h, window=(10, -1))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_packed_batch_with_window_and_block_mask(dtype):
    lengths = (300, 1, 0, 517, 129)
    w = PackedWorkload("varlen_masks", 4, 2, sum(lengths), (1, 1), 128, dtype, True, seed=21,
                       lengths=lengths)
    inp = make_packed_inputs(w)
    mx = max(lengths)
    bm = _block_mask(mx, seed=5, density=0.5)
    idx = fa.build_block_index(torch.from_numpy(bm).cuda(), mx)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"]
    window = (200, -1)
    o, lse = fa.flash_attn_varlen_fwd(q, k, v, cu, None, True, w.softmax_scale, window, idx)
    dq, dk, dv = fa.flash_attn_varlen_bwd(q, k, v, o, lse, do, cu, None, True, w.softmax_scale,
                                          window, idx)
    torch.cuda.synchronize()
    cuh = [int(x) for x in cu]
    args = [f64(inp[x]) for x in ("q", "k", "v")]
    ro, rl = oracle.varlen_fwd(*args, cuh, True, w.softmax_scale, window, bm)
    rdq, rdk, rdv = oracle.varlen_bwd(*args, f64(inp["do"]), cuh, True, w.softmax_scale, window, bm)
    tol = FP32_REL if dtype == "fp32" else BF16_GRAD_REL
    go, gl = f64(o), lse.cpu().double().numpy()
    for a, e in zip(cuh[:-1], cuh[1:]):
        if e == a:
            continue
        for h in range(4):
            if dtype == "fp32":
                assert normwise_rel(go[h, a:e], ro[h, a:e]) <= FP32_REL
            else:
                assert np.abs(go[h, a:e] - ro[h, a:e]).max() <= BF16_O_ABS
            fin = np.isfinite(rl[h, a:e])
            assert np.array_equal(np.isfinite(gl[h, a:e]), fin)
            assert np.abs(gl[h, a:e][fin] - rl[h, a:e][fin]).max(initial=0) <= BF16_LSE_ABS
            assert normwise_rel(f64(dq)[h, a:e], rdq[h, a:e]) <= tol
        for j in range(2):
            assert normwise_rel(f64(dk)[j, a:e], rdk[j, a:e]) <= tol
            assert normwise_rel(f64(dv)[j, a:e], rdv[j, a:e]) <= tol


def _local_global_mask(n, local=4, glob=2):
    # Each query block sees its `local` predecessors (itself included) and
    # the first `glob` blocks: a block-banded pattern with global tokens.
    nb = (n + 127) // 128
    bm = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        bm[i, max(0, i - local + 1):i + 1] = True
        bm[i, :glob] = True
    return bm


@pytest.mark.parametrize("kind", ["window", "sparse"])
def test_long_sequence_rows(kind):
    w = custom(f"long_{kind}", 1, 32, 16384, 128, "bf16", True, seed=44, qk_sigma=3.0)
    inp = make_inputs(w)
    window, bm, idx = (-1, -1), None, None
    if kind == "window":
        window = (4095, -1)
    else:
        bm = _local_global_mask(w.n)
        idx = fa.build_block_index(torch.from_numpy(bm).cuda(), w.n)
    print(f"[parity] long causal {kind}", flush=True)
    gpu = run_gpu(w, inp, window=window, block_index=idx)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.isfinite(gpu[name]).all(), name
    rng = np.random.default_rng(7)
    for h in (0, 17, 31):
        rows = np.sort(rng.choice(w.n, size=16, replace=False))
        rows[-1] = w.n - 1
        check_forward_head(w, inp, gpu, 0, h, rows=rows, peaky=True, window=window,
                           block_mask=bm)


def test_mask_argument_checks():
    x = torch.randn(1, 1, 300, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(x, x, x, window=(-2, 5))
    with pytest.raises(ValueError):
        fa.build_block_index(torch.ones(2, 2, dtype=torch.bool, device="cuda"), 300)
    idx = fa.build_block_index(torch.ones(3, 3, dtype=torch.bool, device="cuda"), 300)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(x, x, x, block_index=idx[:-1])
    # An all-ones block mask and an unbounded window equal the plain call.
    o1, l1 = fa.flash_attn_fwd(x, x, x, True, block_index=idx, window=(-1, -1))
    o2, l2 = fa.flash_attn_fwd(x, x, x, True)
    assert torch.allclose(o1.float(), o2.float(), atol=1e-2) and torch.allclose(l1, l2, atol=1e-3)
