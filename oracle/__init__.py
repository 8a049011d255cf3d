"""CPU oracle for exact scaled-dot-product attention (fp64, materialised).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code, constants
or helpers with the HIP library; the two meet only through the seeded input
generators, which hold none of the method's arithmetic.

Pages this package follows (cited by title and section throughout):

* Page 1: "注意力为什么受限于显存带宽：用算术强度与分块把 FlashAttention
  推导清楚" (magicnetworld.com) -- section 五 (standard attention), section 六
  (online softmax, with the two-block worked example), section 八 (backward by
  recomputation from the saved row statistics).
* Page 2: "4. FlashAttention 深度剖析" (llm-training-tutorial.pages.dev) --
  4.2.1 three-pass safe softmax, 4.2.2 two-pass online normalizer, 4.2.3
  one-pass softmax x matmul, 4.2.4 block-state merge, 4.3.2 tiled forward with
  the stored L = m + log l, 4.3.4 backward recomputing P = exp(S - L).
* Page 3: "深入浅出 FlashAttention" (yuzheng310.github.io, a rendering of
  "ELI5: FlashAttention") -- 第八部分 (causal mask = upper-right triangle).
* Page 4: "炉案与百步之外的仓库：Flash Attention 与注意力计算的工艺极限"
  (carrie-l.github.io) -- 上篇 section 四 (worked example 7, 4, 3 then 9).

Modules:

* ``attention`` -- the definition written out: S = scale * Q K^T, mask, row
  softmax, O = P V, LSE = m + ln l, and the gradients of sum(O * dO); grouped
  K/V heads; packed variable-length batches (page 2 4.7.2, 4.7.4).
* ``online``    -- the pages' online-softmax algebra (three-, two- and
  one-pass forms, per-block update, associative block merge), used to pin
  ``attention`` and as the reading of the tiled recurrence.
* ``fp8``       -- page 2 4.5.4's FP8 recipe: the E4M3 format (rounding,
  decoding), per-block power-of-two scales and the optional random Hadamard
  rotation of Q and K are definitions; its forward on codes (probabilities
  quantised in an integer row frame, row sums of the rounded values) is a
  model of the GPU kernel's arithmetic, a secondary diagnostic. The FP8
  forward's parity gate is ``attention.head_forward`` on the dequantised
  operands (pinned by ``tests/test_oracle_fp8.py``).

Parity status: every function here is pinned by ``tests/test_oracle.py`` or
``tests/test_oracle_fp8.py``
(worked examples, closed forms, invariants, brute force, finite differences
and a library cross-check); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    visible_mask,
    head_forward,
    head_backward,
    attention_fwd,
    attention_bwd,
    varlen_fwd,
    varlen_bwd,
    default_scale,
)
from . import online  # noqa: F401
from . import fp8  # noqa: F401
