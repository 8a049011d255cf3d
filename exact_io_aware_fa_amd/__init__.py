"""MI355X-native fused exact attention (gfx950 HIP kernels behind a C ABI).

Python surface:

* ``binding``   -- ctypes view of include/fa.h (fa_fwd, fa_fwd_gqa,
                   fa_fwd_varlen, fa_bwd, fa_bwd_gqa, fa_bwd_varlen,
                   fa_bwd_timed, fa_bwd_workspace_bytes, fa_status_str,
                   fa_abi_version).
* ``attention`` -- torch wrappers: ``flash_attn_fwd``, ``flash_attn_bwd``
                   (grouped K/V heads when k, v have fewer heads),
                   ``flash_attn_varlen_fwd``, ``flash_attn_varlen_bwd`` and the
                   autograd-enabled ``flash_attention``,
                   ``flash_attention_varlen``; ``window`` and ``block_index``
                   arguments (``build_block_index``) for sliding windows and
                   block-sparse masks.
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
                "FlashAttentionVarlenFunction", "build_block_index"):
        from . import attention
        return getattr(attention, name)
    raise AttributeError(name)
