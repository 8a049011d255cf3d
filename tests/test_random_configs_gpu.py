"""Parity on seeded random combinations of the options the boundary takes.

The other GPU tests pick their cases by hand; this file draws 26 more from a
fixed seed so that options meet in combinations nobody chose: head dimension
64/128/256, bf16 or fp32, causal or not, key padding, a sliding window of
either or both sides (page 4, "FlashAttention 原理深入剖析（下篇）", section
六: the window_size of the flash-attn call), a block-sparse mask (page 3,
"深入浅出 FlashAttention", 第八部分), grouped K/V heads and ragged lengths,
plus two d = 128 draws from 4096 rows (the 64-keys-per-wave dK/dV kernel).
Forward and backward of two heads per case are compared with the fp64
oracle under the same tolerances as every other parity test. The draws are
made once at import from their own generator, so case ids are stable.
"""

import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd import attention as fa
from exact_io_aware_fa_amd.inputs import custom, make_inputs
from parity_utils import check_backward_head, check_forward_head, run_gpu

pytestmark = pytest.mark.gpu


def _draw(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        dtype = "fp32" if rng.random() < 0.2 else "bf16"
        d = int(rng.choice([64, 128, 256]))
        sizes = [1, 7, 63, 64, 65, 200, 511] + ([] if dtype == "fp32" else [777, 1025, 1500])
        n = int(rng.choice(sizes))
        causal = bool(rng.random() < 0.5)
        padded = bool(rng.random() < 0.4)
        kind = int(rng.integers(0, 4))
        left, right = int(rng.integers(0, n + 1)), int(rng.integers(0, n + 1))
        window = [None, (left, -1), (left, right), (-1, right)][kind]
        sparse = bool(rng.random() < 0.3)
        heads, heads_kv = [(2, 2), (4, 2), (4, 1), (3, 3)][int(rng.integers(0, 4))]
        batch = 2 if padded else int(rng.integers(1, 3))
        out.append((n, d, dtype, causal, padded, window, sparse, batch, heads, heads_kv))
    return out


CASES = _draw(26, seed=2027) + [
    (4200, 128, "bf16", True, True, None, False, 2, 4, 2),
    (4500, 128, "bf16", False, False, None, False, 1, 2, 1),
]


def _block_mask(n, seed):
    nb = (n + 127) // 128
    bm = np.random.default_rng(seed).random((nb, nb)) < 0.6
    np.fill_diagonal(bm, True)
    return bm


@pytest.mark.parametrize("n,d,dtype,causal,padded,window,sparse,batch,heads,heads_kv", CASES)
def test_random_configuration(n, d, dtype, causal, padded, window, sparse, batch, heads,
                              heads_kv):
    w = custom(f"rand_n{n}_d{d}", batch, heads, n, d, dtype, causal, seed=3 * n + d + heads,
               padded=padded, heads_kv=heads_kv)
    inp = make_inputs(w)
    bm = _block_mask(n, seed=n + d) if sparse else None
    idx = fa.build_block_index(torch.from_numpy(bm).cuda(), n) if sparse else None
    print(f"[random] n={n} d={d} {dtype} causal={causal} padded={padded} window={window} "
          f"sparse={sparse} batch={batch} heads={heads}/{heads_kv}", flush=True)
    gpu = run_gpu(w, inp, window=window, block_index=idx)
    win = (-1, -1) if window is None else window
    for b, h in ((0, 0), (batch - 1, heads - 1)):
        check_forward_head(w, inp, gpu, b, h, window=win, block_mask=bm)
        check_backward_head(w, inp, gpu, b, h, window=win, block_mask=bm)
