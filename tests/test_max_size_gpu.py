"""The largest sequences the boundary accepts, checked through locality.

The C ABI takes up to 2^22 rows as long as one head's rows stay under 2 GiB
(rows x d x 2 bytes for bf16). At that size the fp64 oracle cannot run on a
whole head, but a sliding window makes every output local: with keys
i - left .. i + right visible to query i (page 4, "FlashAttention
原理深入剖析（下篇）", section 六: the window_size of the flash-attn call),
row i's O, LSE and dQ depend only on the rows and keys within
its window, and key j's dK and dV only on the queries that see it and on
their windows. The masks depend on i - j alone, so the oracle run on a
slice [a, e) of the sequence (positions shifted by a) gives exactly the
full problem's values for the rows and keys whose dependencies lie inside
the slice. Segments at the start, in the middle and at the very end of
the sequence (byte offsets past 4 GiB in the second head) are compared
that way; every output element is also checked to be finite.

Inputs come from torch's seeded generator on the GPU (the full tensors take
tens of GiB); the oracle reads the slices it needs back from them.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa_amd import attention as fa
from parity_utils import BF16_GRAD_REL, BF16_LSE_ABS, BF16_O_ABS, f64, normwise_rel

pytestmark = pytest.mark.gpu

CASES = [
    # (n, d, causal, window, batch, heads, heads_kv)
    ((1 << 22) - 37, 256, True, (200, -1), 1, 2, 1),   # 2^31 - 18944 bytes per head
    ((1 << 22) - 5, 128, False, (150, 150), 1, 2, 2),
    ((1 << 22) - 1, 64, True, (100, -1), 1, 4, 2),
]


def _segments(n, left, right):
    """(a, e) slices: the start, the middle and the end of the sequence."""
    span = 4 * (left + right) + 64
    mid = (n // 2) - span // 2
    return [(0, span), (mid, mid + span), (n - span, n)]


def _valid(n, a, e, left, right):
    """Rows whose O, LSE, dQ and keys whose dK, dV the slice [a, e) fixes."""
    f_lo = a if a == 0 else a + left
    f_hi = e if e == n else e - right
    k_lo = a if a == 0 else f_lo + right
    k_hi = e if e == n else f_hi - left
    return (f_lo, f_hi), (k_lo, k_hi)


@pytest.mark.parametrize("n,d,causal,window,batch,heads,heads_kv", CASES)
def test_max_rows_through_window_locality(n, d, causal, window, batch, heads, heads_kv):
    print(f"[max] n={n} d={d} causal={causal} window={window} heads={heads}/{heads_kv}",
          flush=True)
    g = torch.Generator(device="cuda").manual_seed(n % 1000 + d)
    shape_q = (batch, heads, n, d)
    shape_kv = (batch, heads_kv, n, d)
    q = torch.randn(shape_q, generator=g, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(shape_kv, generator=g, device="cuda", dtype=torch.bfloat16)
    v = torch.randn(shape_kv, generator=g, device="cuda", dtype=torch.bfloat16)
    do = torch.randn(shape_q, generator=g, device="cuda", dtype=torch.bfloat16)
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.flash_attn_fwd(q, k, v, causal, scale, None, window)
    dq, dk, dv = fa.flash_attn_bwd(q, k, v, o, lse, do, causal, scale, None, window)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name

    left = window[0]
    right = 0 if causal else window[1]
    group = heads // heads_kv
    for a, e in _segments(n, left, right):
        (f_lo, f_hi), (k_lo, k_hi) = _valid(n, a, e, left, right)
        print(f"[max] slice [{a}, {e}): rows [{f_lo}, {f_hi}), keys [{k_lo}, {k_hi})",
              flush=True)
        for hk in range(heads_kv):
            ks, vs = f64(k[0, hk, a:e]), f64(v[0, hk, a:e])
            dk_ref = np.zeros_like(ks)
            dv_ref = np.zeros_like(vs)
            for h in range(hk * group, (hk + 1) * group):
                qs, dos = f64(q[0, h, a:e]), f64(do[0, h, a:e])
                ref = oracle.head_backward(qs, ks, vs, dos, scale, causal, None, window)
                dk_ref += ref["dk"]
                dv_ref += ref["dv"]
                r0, r1 = f_lo - a, f_hi - a
                go = f64(o[0, h, f_lo:f_hi])
                assert np.abs(go - ref["o"][r0:r1]).max() <= BF16_O_ABS, (h, a)
                gl = lse[0, h, f_lo:f_hi].double().cpu().numpy()
                assert np.abs(gl - ref["lse"][r0:r1]).max() <= BF16_LSE_ABS, (h, a)
                err = normwise_rel(f64(dq[0, h, f_lo:f_hi]), ref["dq"][r0:r1])
                assert err <= BF16_GRAD_REL, ("dq", h, a, err)
            c0, c1 = k_lo - a, k_hi - a
            for name, got, r in (("dk", dk, dk_ref), ("dv", dv, dv_ref)):
                err = normwise_rel(f64(got[0, hk, k_lo:k_hi]), r[c0:c1])
                assert err <= BF16_GRAD_REL, (name, hk, a, err)
