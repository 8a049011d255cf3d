"""Seeded synthetic workloads and their inputs.

This module holds no attention arithmetic: it only names the workloads
(shapes, dtypes, masks, value distributions, seeds) and draws their inputs.
Both the HIP path and the CPU oracle are fed from it, so they see identical
values. Draw order per workload: Q, K, V, dO as float32 standard normals
(Q and K multiplied by ``qk_sigma``), each rounded to the workload dtype
(bf16: round to nearest even), then the per-batch key lengths. K and V have
``heads_kv`` heads (grouped K/V heads), Q and dO ``heads``.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n: int
    d: int
    dtype: str              # "bf16" or "fp32"
    causal: bool
    seed: int
    qk_sigma: float = 1.0   # std of Q and K entries (V and dO are unit)
    padded: bool = False    # per-batch key lengths, uniform in [n/2, n]
    backward: bool = True
    scale: float | None = None  # default 1/sqrt(d)
    heads_kv: int | None = None  # K/V heads (divides heads); default heads
    window: tuple = (-1, -1)     # sliding window (left, right), -1 unbounded
    blocks: tuple | None = None  # block-sparse pattern: ("local_global", local, glob)

    @property
    def kv_heads(self) -> int:
        return self.heads if self.heads_kv is None else self.heads_kv

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d) if self.scale is None else self.scale

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def flops_fwd(self) -> float:
        """Attention FLOPs of the forward: 4 B H N^2 d, halved when causal."""
        f = 4.0 * self.batch * self.heads * self.n * self.n * self.d
        return f / 2 if self.causal else f

    def flops_bwd(self) -> float:
        """Backward FLOPs: 2.5x the forward (five N^2 d products vs two)."""
        return 2.5 * self.flops_fwd()


@dataclasses.dataclass(frozen=True)
class PackedWorkload:
    """A packed variable-length batch: sequences back to back per head,
    [heads, total, d]. Lengths are drawn uniformly from ``len_range`` until
    they reach ``total`` (the last one cut to fit), unless given."""
    name: str
    heads: int
    heads_kv: int
    total: int
    len_range: tuple
    d: int
    dtype: str
    causal: bool
    seed: int
    qk_sigma: float = 1.0
    scale: float | None = None
    lengths: tuple | None = None
    backward: bool = True

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d) if self.scale is None else self.scale

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def _draw_lengths(self, g) -> list:
        if self.lengths is not None:
            return [int(x) for x in self.lengths]
        lo, hi = self.len_range
        out, left = [], self.total
        while left > 0:
            x = int(torch.randint(lo, hi + 1, (1,), generator=g))
            out.append(min(x, left))
            left -= out[-1]
        return out

    def seqlens(self) -> list:
        return self._draw_lengths(torch.Generator(device="cpu").manual_seed(self.seed))

    def cu_seqlens(self) -> list:
        out = [0]
        for x in self.seqlens():
            out.append(out[-1] + x)
        return out

    def flops_fwd(self) -> float:
        """4 H d sum_s L_s^2, halved when causal."""
        f = 4.0 * self.heads * self.d * sum(x * x for x in self.seqlens())
        return f / 2 if self.causal else f

    def flops_bwd(self) -> float:
        return 2.5 * self.flops_fwd()


def make_packed_inputs(w: PackedWorkload, with_grad_out: bool = True) -> dict:
    """CPU tensors q [H, T, d], k, v [H_kv, T, d] (and do), and cu_seqlens
    (int32 [num_seqs + 1]). Draw order: the lengths, then Q, K, V, dO."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    lens = w._draw_lengths(g)
    total = sum(lens)
    dt = w.torch_dtype

    def draw(heads, sigma):
        x = torch.randn((heads, total, w.d), generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        return x.to(dt)

    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    out = {"q": draw(w.heads, w.qk_sigma), "k": draw(w.heads_kv, w.qk_sigma),
           "v": draw(w.heads_kv, 1.0), "cu_seqlens": cu}
    out["do"] = draw(w.heads, 1.0) if with_grad_out else None
    return out


def _sweep():
    out = []
    idx = 0
    for n in (2048, 4096, 8192):
        for d in (64, 128, 256):
            for causal in (False, True):
                out.append(Workload(
                    name=f"sweep_b2_h16_n{n}_d{d}_{'causal' if causal else 'full'}",
                    batch=2, heads=16, n=n, d=d, dtype="bf16", causal=causal,
                    seed=500 + idx))
                idx += 1
    return out


WORKLOADS = {w.name: w for w in [
    # single head, fp32, forward parity case the oracle finishes instantly
    Workload("single_head_n128_d64_fp32", 1, 1, 128, 64, "fp32", False, seed=1,
             backward=False),
    # BERT-large-shaped encoder attention with key padding
    Workload("bert_large_b8_h16_n512_d64_padded", 8, 16, 512, 64, "bf16", False,
             seed=2, padded=True),
    # GPT-2-shaped causal decoder attention
    Workload("gpt2_b8_h12_n1024_d64_causal", 8, 12, 1024, 64, "bf16", True, seed=3),
    # long-sequence causal attention with peaky rows (Q, K ~ N(0, 3^2))
    Workload("long_causal_b1_h32_n16384_d128", 1, 32, 16384, 128, "bf16", True,
             seed=4, qk_sigma=3.0),
    # sliding-window causal attention (4096-key window, Mistral style)
    Workload("window_causal_b1_h32_n16384_d128_w4096", 1, 32, 16384, 128, "bf16", True,
             seed=8, window=(4095, -1)),
    # block-sparse causal attention: 4 local blocks of 128 plus 2 global ones
    Workload("blocksparse_causal_b1_h32_n16384_d128_l4g2", 1, 32, 16384, 128, "bf16", True,
             seed=9, blocks=("local_global", 4, 2)),
    # grouped-query attention: 32 query heads sharing 8 K/V heads (groups of 4)
    Workload("gqa_causal_b1_h32_hkv8_n16384_d128", 1, 32, 16384, 128, "bf16", True,
             seed=5, qk_sigma=3.0, heads_kv=8),
    *_sweep(),
]}

# Packed variable-length batches (no padding): a causal mix of document
# lengths for long-context training and a BERT-like encoder mix.
PACKED = {w.name: w for w in [
    PackedWorkload("varlen_causal_h32_t16384_d128", 32, 32, 16384, (256, 4096), 128, "bf16",
                   True, seed=6),
    PackedWorkload("varlen_bert_h16_t32768_d64", 16, 16, 32768, (64, 512), 64, "bf16",
                   False, seed=7),
]}

HEADLINE = "long_causal_b1_h32_n16384_d128"


def block_mask(w) -> "np.ndarray | None":
    """The workload's boolean block mask over 128 x 128 blocks, or None.
    ("local_global", L, G): query block i keeps key blocks i-L+1 .. i and the
    first G blocks (a banded pattern with global tokens)."""
    if w.blocks is None:
        return None
    import numpy as np
    kind, local, glob = w.blocks
    assert kind == "local_global"
    nb = (w.n + 127) // 128
    bm = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        bm[i, max(0, i - local + 1):i + 1] = True
        bm[i, :glob] = True
    return bm


def make_inputs(w: Workload, with_grad_out: bool = True) -> dict:
    """CPU tensors q, k, v (and do), plus kv_len (int32 [batch]) or None."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    qshape = (w.batch, w.heads, w.n, w.d)
    kvshape = (w.batch, w.kv_heads, w.n, w.d)
    dt = w.torch_dtype

    def draw(shape, sigma):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        return x.to(dt)

    out = {"q": draw(qshape, w.qk_sigma), "k": draw(kvshape, w.qk_sigma),
           "v": draw(kvshape, 1.0)}
    out["do"] = draw(qshape, 1.0) if with_grad_out else None
    # Valid key lengths in [max(n/2, 1), n]: at least one key, as the torch
    # wrappers require.
    out["kv_len"] = (torch.randint(max(w.n // 2, 1), w.n + 1, (w.batch,), generator=g,
                                   dtype=torch.int32) if w.padded else None)
    return out


def custom(name, batch, heads, n, d, dtype="bf16", causal=False, seed=0,
           qk_sigma=1.0, padded=False, scale=None, heads_kv=None) -> Workload:
    """An ad-hoc workload (tests of edge cases: ragged n, tiny shapes...)."""
    return Workload(name, batch, heads, n, d, dtype, causal, seed, qk_sigma,
                    padded, True, scale, heads_kv)
