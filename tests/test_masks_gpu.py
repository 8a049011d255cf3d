"""GPU checks of masking and indexing that must hold bit for bit.

* Hidden probabilities are exactly 0: keys hidden by the causal mask are
  given values near the bf16 maximum (2^127) and keys hidden by padding are
  given NaN/Inf; the outputs that may not depend on them stay bit-identical.
* Causal prefix invariance: changing K/V rows > t leaves O, LSE and (bf16)
  dQ rows <= t bit-identical. The fp32 path adds dQ with float atomics in
  arbitrary order, so there its rows are compared to the oracle-level
  tolerance instead.
* Padding invariance: O, LSE, (bf16) dQ and dK/dV rows < kv_len are
  bit-identical, and dK/dV rows >= kv_len are exactly 0.
* The bf16 path is bitwise deterministic: every output element is reduced by
  one wave in a fixed order, with no atomics.
"""

import pytest
import torch

from exact_io_aware_fa_amd.attention import flash_attn_bwd, flash_attn_fwd
from exact_io_aware_fa_amd.inputs import custom, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _run(q, k, v, do, causal, kv_len=None, scale=None):
    o, lse = flash_attn_fwd(q, k, v, causal, scale, kv_len)
    dq, dk, dv = flash_attn_bwd(q, k, v, o, lse, do, causal, scale, kv_len)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _gpu(w):
    inp = make_inputs(w)
    return [inp[x].cuda() for x in ("q", "k", "v", "do")], inp["kv_len"]


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "bf16"), (256, "bf16"), (64, "fp32")])
@pytest.mark.parametrize("t", [0, 37, 150, 255])
def test_causal_prefix_invariance_and_exact_zero_probabilities(d, dtype, t):
    w = custom("prefix", 2, 2, 300, d, dtype, True, seed=3 + t)
    (q, k, v, do), _ = _gpu(w)
    base = _run(q, k, v, do, True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, t + 1:] = k2[:, :, t + 1:] * 3.0 + 1.0
    # Forward: hidden values near the bf16 maximum; any nonzero hidden
    # probability (>= 2^-133 in bf16) would change O.
    v_big = v.clone()
    v_big[:, :, t + 1:] = 2.0 ** 127
    o_big, lse_big = flash_attn_fwd(q, k2, v_big, True)
    assert torch.equal(base[0][:, :, : t + 1], o_big[:, :, : t + 1])
    assert torch.equal(base[1][:, :, : t + 1], lse_big[:, :, : t + 1])
    # Backward (finite perturbation, so dP of hidden pairs stays finite).
    v2[:, :, t + 1:] = v2[:, :, t + 1:] * 3.0 - 2.0
    pert = _run(q, k2, v2, do, True)
    assert torch.equal(base[0][:, :, : t + 1], pert[0][:, :, : t + 1])
    assert torch.equal(base[1][:, :, : t + 1], pert[1][:, :, : t + 1])
    if dtype == "bf16":
        assert torch.equal(base[2][:, :, : t + 1], pert[2][:, :, : t + 1])
    else:
        torch.testing.assert_close(pert[2][:, :, : t + 1], base[2][:, :, : t + 1],
                                   atol=1e-5 * float(base[2].abs().max()), rtol=0)


@pytest.mark.parametrize("d,dtype,causal", [(64, "bf16", False), (128, "bf16", True),
                                            (256, "bf16", False), (128, "fp32", True)])
def test_padding_invariance_with_nonfinite_padded_rows(d, dtype, causal):
    w = custom("pad", 3, 2, 260, d, dtype, causal, seed=9)
    (q, k, v, do), _ = _gpu(w)
    kv_len = torch.tensor([1, 131, 260], dtype=torch.int32)
    base = _run(q, k, v, do, causal, kv_len)
    k2, v2 = k.clone(), v.clone()
    for b, L in enumerate(kv_len.tolist()):
        k2[b, :, L:] = float("nan")
        v2[b, :, L:] = float("inf")
    pert = _run(q, k2, v2, do, causal, kv_len)
    assert torch.equal(base[0], pert[0])
    assert torch.equal(base[1], pert[1])
    for b, L in enumerate(kv_len.tolist()):
        for g in (3, 4):  # dK, dV
            assert torch.equal(base[g][b, :, :L], pert[g][b, :, :L])
            assert torch.all(pert[g][b, :, L:] == 0)
    assert torch.isfinite(pert[2]).all()
    if dtype == "bf16":
        assert torch.equal(base[2], pert[2])


@pytest.mark.parametrize("d,causal", [(64, True), (128, False), (256, True)])
def test_bf16_path_bitwise_deterministic(d, causal):
    w = custom("det", 2, 3, 517, d, "bf16", causal, seed=21)
    (q, k, v, do), _ = _gpu(w)
    a = _run(q, k, v, do, causal)
    b = _run(q, k, v, do, causal)
    for i in range(5):  # O, LSE, dQ, dK, dV
        assert torch.equal(a[i], b[i])


@pytest.mark.parametrize("d", [64, 128, 256])
def test_causal_row0_returns_v_row0_bitwise(d):
    w = custom("row0", 2, 4, 200, d, "bf16", True, seed=d, qk_sigma=3.0)
    (q, k, v, do), _ = _gpu(w)
    o, lse = flash_attn_fwd(q, k, v, True)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    ref = (q[:, :, 0].float() * k[:, :, 0].float()).sum(-1) / d ** 0.5
    torch.testing.assert_close(lse[:, :, 0], ref, atol=1e-4, rtol=1e-5)
