"""MI355X-native fused exact attention (gfx950 HIP kernels behind a C ABI).

Python surface:

* ``binding``   -- ctypes view of include/fa.h (fa_fwd, fa_fwd_gqa,
                   fa_fwd_varlen, fa_bwd, fa_bwd_gqa, fa_bwd_varlen,
                   fa_bwd_timed, fa_bwd_workspace_bytes, fa_block_index_bytes,
                   fa_block_index_build, fa_fp8_codes_bytes, fa_fp8_scales_bytes,
                   fa_fp8_quantize, fa_fwd_fp8, fa_status_str, fa_abi_version).
* ``attention`` -- torch wrappers: ``flash_attn_fwd``, ``flash_attn_bwd``
                   (grouped K/V heads when k, v have fewer heads),
                   ``flash_attn_varlen_fwd``, ``flash_attn_varlen_bwd`` and the
                   autograd-enabled ``flash_attention``,
                   ``flash_attention_varlen``; ``window`` and ``block_index``
                   arguments (``build_block_index``) for sliding windows and
                   block-sparse masks; the FP8 forward ``flash_attn_fp8_fwd``
                   (``fp8_quantize``, ``flash_attn_fp8_fwd_codes``,
                   ``hadamard_signs``).
* ``inputs``    -- seeded synthetic workloads.
* ``build``     -- hipcc build of libexact_fa.so (in-tree).
"""

from .binding import (  # noqa: F401
    FA_BF16, FA_FP32, fa_abi_version, fa_bwd, fa_bwd_workspace_bytes, fa_fwd,
    fa_status_str)


def __getattr__(name):
    # torch-facing helpers are imported on first use so that importing the
    # package (e.g. to build it) does not require torch.
    if name in ("flash_attention", "flash_attn_fwd", "flash_attn_bwd",
                "FlashAttentionFunction", "flash_attention_varlen",
                "flash_attn_varlen_fwd", "flash_attn_varlen_bwd",
                "FlashAttentionVarlenFunction", "build_block_index",
                "flash_attn_fp8_fwd", "flash_attn_fp8_fwd_codes", "fp8_quantize",
                "hadamard_signs"):
        from . import attention
        return getattr(attention, name)
    raise AttributeError(name)
