"""CPU tests of the seeded workload generator and the FLOP convention."""

import json
import os

import pytest
import torch

from exact_io_aware_fa_amd.inputs import HEADLINE, WORKLOADS, custom, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "flop_counts.json")


def test_named_workloads_have_the_stated_shapes():
    w = WORKLOADS["single_head_n128_d64_fp32"]
    assert (w.batch, w.heads, w.n, w.d, w.dtype, w.causal, w.backward) == (1, 1, 128, 64, "fp32", False, False)
    w = WORKLOADS["bert_large_b8_h16_n512_d64_padded"]
    assert (w.batch, w.heads, w.n, w.d, w.padded, w.causal) == (8, 16, 512, 64, True, False)
    w = WORKLOADS["gpt2_b8_h12_n1024_d64_causal"]
    assert (w.batch, w.heads, w.n, w.d, w.causal) == (8, 12, 1024, 64, True)
    w = WORKLOADS[HEADLINE]
    assert (w.batch, w.heads, w.n, w.d, w.causal, w.qk_sigma) == (1, 32, 16384, 128, True, 3.0)
    sweep = [x for x in WORKLOADS.values() if x.name.startswith("sweep_")]
    assert len(sweep) == 18
    assert {(x.n, x.d, x.causal) for x in sweep} == {
        (n, d, c) for n in (2048, 4096, 8192) for d in (64, 128, 256) for c in (False, True)}
    assert len({x.seed for x in WORKLOADS.values()}) == len(WORKLOADS)


def test_inputs_are_seeded_and_distributed_as_stated():
    w = custom("t", 2, 3, 256, 64, "bf16", False, seed=9, qk_sigma=3.0, padded=True)
    a, b = make_inputs(w), make_inputs(w)
    for key in ("q", "k", "v", "do", "kv_len"):
        assert torch.equal(a[key], b[key])
    assert a["q"].dtype == torch.bfloat16 and a["q"].shape == (2, 3, 256, 64)
    assert abs(a["q"].float().std().item() - 3.0) < 0.05
    assert abs(a["v"].float().std().item() - 1.0) < 0.02
    assert a["kv_len"].dtype == torch.int32
    assert int(a["kv_len"].min()) >= 128 and int(a["kv_len"].max()) <= 256
    # bf16 values are the round-to-nearest-even images of the fp32 draws.
    g = torch.Generator().manual_seed(9)
    q32 = torch.randn((2, 3, 256, 64), generator=g) * 3.0
    assert torch.equal(a["q"], q32.to(torch.bfloat16))
    c = make_inputs(custom("t", 2, 3, 256, 64, "bf16", False, seed=10))
    assert not torch.equal(a["q"], c["q"])


def test_flop_convention_matches_page_figures():
    g = json.load(open(GOLDEN))
    t = g["page5_table"]
    for n, gf in zip(t["n"], t["gflop"]):
        w = custom("p5", t["batch"], t["heads"], n, t["d"], "bf16", False)
        assert abs(w.flops_fwd() / 1e9 - gf) <= t["rel_tol"] * gf
    p1 = g["page1_per_head"]
    w = custom("p1", 1, 1, p1["n"], p1["d"], "bf16", False)
    assert abs(w.flops_fwd() - p1["flop_per_head"]) <= p1["rel_tol"] * p1["flop_per_head"]
    w = custom("p1", 1, p1["heads"], p1["n"], p1["d"], "bf16", False)
    assert abs(w.flops_fwd() - p1["flop_all_heads"]) <= p1["rel_tol"] * p1["flop_all_heads"]


def test_causal_halves_and_backward_is_two_and_a_half():
    w = WORKLOADS[HEADLINE]
    assert w.flops_fwd() == pytest.approx(2.199e12, rel=1e-3)
    assert w.flops_bwd() == pytest.approx(5.498e12, rel=1e-3)
    full = custom("f", 1, 32, 16384, 128, "bf16", False)
    assert full.flops_fwd() == 2 * w.flops_fwd()


def test_masked_flop_count_matches_brute_force():
    # bench.visible_pairs counts the (query, key) pairs a masked workload
    # computes; brute force over the oracle's element mask must agree.
    import bench
    import oracle
    from exact_io_aware_fa_amd.inputs import Workload, block_mask
    for window, blocks, causal in (((37, 5), None, False), ((100, -1), None, True),
                                   ((-1, -1), ("local_global", 2, 1), True),
                                   ((150, 20), ("local_global", 3, 1), False)):
        w = Workload("t", 1, 1, 700, 64, "bf16", causal, 0, window=window, blocks=blocks)
        vis = oracle.visible_mask(w.n, causal, None, None, window, block_mask(w))
        assert bench.visible_pairs(w) == float(vis.sum())
