"""Host-side argument checks of the torch wrappers (no GPU needed): every
wrong shape or dtype is rejected with ValueError before anything reaches the
library, and tensors that are not on the GPU are rejected too (the library
takes raw device pointers, so a host pointer would be read by the kernels).
The shape checks run before the device checks, which is what lets these
tests use CPU tensors."""

import pytest
import torch

from exact_io_aware_fa_amd import attention as fa


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_backward_rejects_wrong_lse_shape():
    q = _bf(2, 4, 64, 64)
    lse = torch.zeros(2, 4, 63)
    with pytest.raises(ValueError, match="lse must be float32 of shape"):
        fa.flash_attn_bwd(q, q, q, q, lse, q)


def test_backward_rejects_wrong_lse_dtype():
    q = _bf(1, 2, 32, 64)
    with pytest.raises(ValueError, match="lse must be float32"):
        fa.flash_attn_bwd(q, q, q, q, torch.zeros(1, 2, 32, dtype=torch.float64), q)
    with pytest.raises(ValueError, match="lse must be float32"):
        fa.flash_attn_bwd(q, q, q, q, torch.zeros(1, 2, 32, dtype=torch.bfloat16), q)


def test_backward_rejects_mismatched_o_and_do():
    q = _bf(1, 2, 32, 64)
    lse = torch.zeros(1, 2, 32)
    with pytest.raises(ValueError, match="o and do"):
        fa.flash_attn_bwd(q, q, q, _bf(1, 2, 31, 64), lse, q)
    with pytest.raises(ValueError, match="o and do"):
        fa.flash_attn_bwd(q, q, q, q, lse, q.float())


def test_backward_rejects_host_tensors():
    q = _bf(1, 2, 32, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flash_attn_bwd(q, q, q, q, torch.zeros(1, 2, 32), q)


def test_varlen_backward_rejects_wrong_lse():
    q = _bf(4, 100, 64)
    with pytest.raises(ValueError, match="lse must be float32 of shape"):
        fa.flash_attn_varlen_bwd(q, q, q, q, torch.zeros(4, 99), q, [0, 40, 100])
    with pytest.raises(ValueError, match="lse must be float32 of shape"):
        fa.flash_attn_varlen_bwd(q, q, q, q, torch.zeros(4, 100, 1), q, [0, 40, 100])
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flash_attn_varlen_bwd(q, q, q, q, torch.zeros(4, 100), q, [0, 40, 100])


def test_forward_shape_errors_come_first():
    with pytest.raises(ValueError, match="heads_kv"):
        fa.flash_attn_fwd(_bf(1, 4, 32, 64), _bf(1, 3, 32, 64), _bf(1, 3, 32, 64))
    with pytest.raises(ValueError, match="bfloat16 or all float32"):
        fa.flash_attn_fwd(_bf(1, 2, 32, 64), _bf(1, 2, 32, 64), torch.zeros(1, 2, 32, 64))
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flash_attn_fwd(_bf(1, 2, 32, 64), _bf(1, 2, 32, 64), _bf(1, 2, 32, 64))


def _codes(b, h, n, d):
    npad = (n + 127) // 128 * 128
    return torch.zeros(b, h, npad, d, dtype=torch.uint8)


def test_fp8_codes_reject_bad_scales_and_codes():
    b, h, hkv, n, d = 2, 4, 2, 300, 128
    q8, k8 = _codes(b, h, n, d), _codes(b, hkv, n, d)
    v8 = torch.zeros(b, hkv, 3, d, 128, dtype=torch.uint8)
    qs, ks, vs = torch.ones(b, h, 3), torch.ones(b, hkv, 3), torch.ones(b, hkv, 3)
    with pytest.raises(ValueError, match="q_scales must be float32"):
        fa.flash_attn_fp8_fwd_codes(q8, qs.double(), k8, ks, v8, vs, n)
    with pytest.raises(ValueError, match="k_scales must be float32 of shape"):
        fa.flash_attn_fp8_fwd_codes(q8, qs, k8, torch.ones(b, h, 3), v8, vs, n)
    with pytest.raises(ValueError, match="v_scales must be float32 of shape"):
        fa.flash_attn_fp8_fwd_codes(q8, qs, k8, ks, v8, torch.ones(b, hkv, 2), n)
    with pytest.raises(ValueError, match="must be uint8"):
        fa.flash_attn_fp8_fwd_codes(q8.to(torch.int8), qs, k8, ks, v8, vs, n)
    with pytest.raises(ValueError, match="layouts for this n"):
        fa.flash_attn_fp8_fwd_codes(q8, qs, k8, ks, v8, vs, 500)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flash_attn_fp8_fwd_codes(q8, qs, k8, ks, v8, vs, n)
