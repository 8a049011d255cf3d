"""GPU parity for grouped K/V heads (grouped-query and multi-query attention):
query head h attends with K/V head h // (heads / heads_kv), and the gradient
of a shared K/V head is the sum over its group (page 1, section 九; page 4,
"FlashAttention 原理深入剖析（下篇）", section 六, name both variants).

Small cases compare the HIP path through the C ABI with the fp64 oracle,
head by head, forward and backward (dK, dV against the oracle's group sums).
At the full grouped size (B=1, H=32, H_kv=8, N=16384, d=128, causal) the
forward is compared on seeded rows, and the whole call is checked against
the ordinary multi-head call on K/V heads repeated to 32: O, LSE and dQ must
agree bit for bit (same kernels, same operands, same order), and dK, dV
against the group sums of the multi-head gradients.
"""

import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd import attention as fa
from exact_io_aware_fa_amd.inputs import WORKLOADS, custom, make_inputs
from parity_utils import check_backward_head, check_forward_head, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


GQA = [
    # (heads, heads_kv, n, d, causal, dtype, padded)
    (8, 2, 300, 128, True, "bf16", False),
    (6, 1, 257, 64, False, "bf16", True),      # multi-query
    (4, 2, 129, 256, True, "bf16", False),
    (8, 4, 1000, 64, True, "bf16", True),
    (4, 2, 1300, 64, False, "bf16", True),
    (4, 1, 383, 256, False, "bf16", True),     # multi-query, d=256
    (6, 3, 200, 64, True, "fp32", True),
    (4, 1, 150, 128, False, "fp32", False),
    (2, 1, 65, 256, True, "fp32", False),
]


@pytest.mark.parametrize("heads,heads_kv,n,d,causal,dtype,padded", GQA)
def test_grouped_heads_against_oracle(heads, heads_kv, n, d, causal, dtype, padded):
    w = custom(f"gqa_h{heads}_kv{heads_kv}_n{n}_d{d}", 2, heads, n, d, dtype, causal,
               seed=heads * 1000 + n + d, padded=padded, heads_kv=heads_kv)
    inp = make_inputs(w)
    print(f"[parity] gqa heads={heads} kv={heads_kv} n={n} d={d} causal={causal} "
          f"{dtype} padded={padded}", flush=True)
    gpu = run_gpu(w, inp)
    assert gpu["dk"].shape == inp["k"].shape and gpu["dv"].shape == inp["v"].shape
    for b, h in ((0, 0), (1, heads - 1)):
        check_forward_head(w, inp, gpu, b, h)
        check_backward_head(w, inp, gpu, b, h)


def test_grouped_equals_repeated_heads_at_full_size():
    w = WORKLOADS["gqa_causal_b1_h32_hkv8_n16384_d128"]
    grp = w.heads // w.kv_heads
    print(f"[parity] {w.name}: grouped vs repeated K/V heads", flush=True)
    inp = make_inputs(w)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = fa.flash_attn_fwd(q, k, v, True, w.softmax_scale)
    dq, dk, dv = fa.flash_attn_bwd(q, k, v, o, lse, do, True, w.softmax_scale)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(t).all(), name
    # Seeded rows of three query heads (different K/V heads) against the oracle.
    rng = np.random.default_rng(w.seed)
    gpu = {"o": o, "lse": lse}
    for h in (0, 13, 31):
        rows = np.sort(rng.choice(w.n, size=16, replace=False))
        rows[-1] = w.n - 1
        check_forward_head(w, inp, gpu, 0, h, rows=rows, peaky=True)
    # The same call with every K/V head repeated for its query heads.
    kr = k.repeat_interleave(grp, dim=1).contiguous()
    vr = v.repeat_interleave(grp, dim=1).contiguous()
    o2, lse2 = fa.flash_attn_fwd(q, kr, vr, True, w.softmax_scale)
    dq2, dk2, dv2 = fa.flash_attn_bwd(q, kr, vr, o2, lse2, do, True, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(dq, dq2)
    # Group sums of the multi-head gradients (each rounded to bf16 once per
    # head) against the grouped ones (summed in fp32, rounded once): the
    # difference is bounded by the bf16 roundings, 2^-8 relative per term.
    for g_got, g_rep in ((dk, dk2), (dv, dv2)):
        ref = g_rep.float().reshape(1, w.kv_heads, grp, w.n, w.d).sum(2)
        err = (g_got.float() - ref).abs().max().item()
        scale = g_rep.float().abs().max().item()
        assert err <= grp * 2.0 ** -8 * scale, (err, scale)
