"""Pins for the fp64 CPU oracle (runs without a GPU).

The oracle is checked against things other than itself:

* the worked examples the pages print (tests/golden/worked_examples.json);
* brute-force agreement of the pages' three-, two- and one-pass softmax forms
  and of the tiled Q-outer/KV-inner recurrence with the materialised
  definition, including peaky rows;
* the monoid laws of the block-state merge (associativity, identity);
* closed forms: zero scale gives the mean of the visible values, a single
  visible key returns its value, equal keys give uniform weights;
* invariants: rows of P sum to 1, hidden probabilities are exactly 0, padded
  keys get exactly zero gradients, causal prefix invariance, the identity
  D_i = sum_j P_ij dP_ij = <dO_i, O_i>;
* central finite differences of f = sum(O * dO) for every input entry;
* a library cross-check against torch's CPU float64
  scaled_dot_product_attention and its autograd, also with grouped K/V heads
  (enable_gqa), where finite differences pin the summed K/V gradients too.

The last test plants plausible mistakes in copies of the oracle and checks
that at least one pin rejects each of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import online
from oracle.attention import head_backward, head_forward, visible_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------

def test_page4_worked_example_three_scores_then_nine():
    g = _golden()["page4_scores_7_4_3_then_9"]
    pp, tol = g["page_printed"], g["page_tol"]
    x = g["scores"]

    m, s1, _ = online.normalizer_two_pass(x)
    assert m == 7.0
    assert abs(s1 - pp["s1"]) <= tol
    assert abs(s1 - (1.0 + math.exp(-3.0) + math.exp(-4.0))) <= 1e-14
    w = online.normalised(x, m, s1)
    np.testing.assert_allclose(w, pp["weights"], atol=tol, rtol=0)
    np.testing.assert_allclose(online.softmax_three_pass(x), w, rtol=1e-15)

    # Adding the score 9: the correction rule s = s1 * exp(7 - 9) + exp(9 - 9).
    m2, s, hist = online.normalizer_two_pass(x + [g["added_score"]])
    assert m2 == 9.0
    assert abs(s - pp["s"]) <= tol
    assert abs(hist[2][1] - s1) <= 1e-15
    assert abs(s - (s1 * math.exp(7.0 - 9.0) + 1.0)) <= 1e-14
    assert abs(math.exp(7.0 - 9.0) - pp["rescale_factor"]) <= tol
    terms = [math.exp(t - 9.0) for t in x + [9.0]]
    np.testing.assert_allclose(terms, pp["terms_after_added"], atol=tol, rtol=0)

    # The same step as a merge of two block states.
    merged = online.merge(online.block_state(x, np.ones((3, 1))),
                          online.block_state([9.0], np.ones((1, 1))))
    assert merged[0] == 9.0 and abs(merged[1] - s) <= 1e-14


def test_page1_worked_example_two_blocks():
    g = _golden()["page1_blocks_3_1_then_5_2"]
    pp, tol = g["page_printed"], g["page_tol"]
    b1, b2 = (np.array([blk]) for blk in g["blocks"])
    v1 = np.ones((2, 1))
    st = (np.array([-math.inf]), np.zeros(1), np.zeros((1, 1)))
    st = online.block_update(st, b1, v1)
    assert st[0][0] == pp["m_after_block1"]
    assert abs(st[1][0] - pp["l_after_block1"]) <= tol
    l1 = st[1][0]
    st = online.block_update(st, b2, v1)
    assert st[0][0] == pp["m_after_block2"]
    assert abs(l1 * math.exp(3.0 - 5.0) - pp["l_rescaled"]) <= tol
    assert abs(math.exp(0.0) + math.exp(-3.0) - pp["block2_sum"]) <= tol
    assert abs(st[1][0] - pp["l_final"]) <= tol
    direct = sum(math.exp(t - 5.0) for t in [3.0, 1.0, 5.0, 2.0])
    assert abs(st[1][0] - direct) <= 1e-14
    np.testing.assert_allclose([math.exp(t - 5.0) for t in [3.0, 1.0, 5.0, 2.0]],
                               pp["direct_terms"], atol=tol, rtol=0)


# --------------------------------------------------------------------------
# Softmax forms agree (brute force on tiny inputs)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("sigma", [1.0, 3.0, 30.0])
@pytest.mark.parametrize("n", [1, 2, 5, 16])
def test_one_two_three_pass_and_definition_agree(sigma, n):
    rng = np.random.default_rng(1000 + n + int(sigma))
    x = rng.normal(0.0, sigma, size=n)
    y3 = online.softmax_three_pass(x)
    m, d, _ = online.normalizer_two_pass(x)
    y2 = online.normalised(x, m, d)
    m1, l1, o1 = online.softmax_matmul_one_pass(x, np.eye(n))
    y1 = o1 / l1
    # The oracle's definition with q = [1], k = x, scale 1 gives S = x.
    p = head_forward(np.ones((1, 1)), x[:, None], np.eye(n), 1.0, False,
                     want_p=True)["p"][0]
    for y in (y2, y1, p):
        np.testing.assert_allclose(y, y3, rtol=1e-13, atol=1e-300)
    assert m1 == m == x.max()
    assert abs(l1 - d) <= 1e-13 * d


def test_two_pass_induction_invariant():
    # After element i, d^(i) equals sum_{j<=i} e^(x_j - m^(i)) (page 2, 4.2.2).
    rng = np.random.default_rng(7)
    x = rng.normal(0.0, 5.0, size=12)
    _, _, hist = online.normalizer_two_pass(x)
    for i, (mi, di) in enumerate(hist):
        assert mi == x[: i + 1].max()
        ref = sum(math.exp(t - mi) for t in x[: i + 1])
        assert abs(di - ref) <= 1e-13 * ref


# --------------------------------------------------------------------------
# Merge monoid
# --------------------------------------------------------------------------

def _random_partition(rng, n):
    cuts = sorted(rng.choice(np.arange(1, n), size=rng.integers(0, n - 1),
                             replace=False).tolist()) if n > 1 else []
    edges = [0] + cuts + [n]
    return [(a, b) for a, b in zip(edges[:-1], edges[1:])]


def _tree_merge(rng, states):
    states = list(states)
    while len(states) > 1:
        i = int(rng.integers(0, len(states) - 1))
        states[i:i + 2] = [online.merge(states[i], states[i + 1])]
    return states[0]


@pytest.mark.parametrize("trial", range(8))
def test_merge_is_associative_over_partitions_and_trees(trial):
    rng = np.random.default_rng(trial)
    n, dv = int(rng.integers(2, 40)), 3
    x = rng.normal(0.0, [1.0, 3.0, 30.0][trial % 3], size=n)
    v = rng.normal(size=(n, dv))
    whole = online.block_state(x, v)
    parts = [online.block_state(x[a:b], v[a:b]) for a, b in _random_partition(rng, n)]
    left = parts[0]
    for s in parts[1:]:
        left = online.merge(left, s)
    right = parts[-1]
    for s in reversed(parts[:-1]):
        right = online.merge(s, right)
    tree = _tree_merge(rng, parts)
    flat = online.merge(*parts)  # every block state at once
    for st in (left, right, tree, flat):
        assert st[0] == whole[0]
        assert abs(st[1] - whole[1]) <= 1e-12 * whole[1]
        np.testing.assert_allclose(st[2], whole[2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(left[2] / left[1], v.T @ online.softmax_three_pass(x),
                               rtol=1e-12, atol=1e-14)


def test_merge_identity_is_the_empty_state():
    st = online.block_state([1.0, -2.0], np.array([[1.0, 2.0], [3.0, 4.0]]))
    for merged in (online.merge(online.empty_state(2), st),
                   online.merge(st, online.empty_state(2))):
        assert merged[0] == st[0] and merged[1] == st[1]
        np.testing.assert_array_equal(merged[2], st[2])
    e = online.merge(online.empty_state(2), online.empty_state(2))
    assert e[0] == -math.inf and e[1] == 0.0 and not np.isnan(e[2]).any()


# --------------------------------------------------------------------------
# Tiled recurrence == definition ("exact, not approximate")
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,br,bc,causal,kvl", [
    (16, 4, 4, False, None), (16, 4, 8, True, None), (37, 8, 5, True, None),
    (37, 16, 16, False, 20), (37, 8, 16, True, 29), (1, 16, 16, True, None),
    (50, 7, 3, False, 1)])
def test_tiled_forward_equals_definition(n, br, bc, causal, kvl):
    rng = np.random.default_rng(n * 31 + br)
    q, k, v = (rng.normal(0.0, 3.0, size=(n, 6)) for _ in range(3))
    scale = 0.37
    ref = head_forward(q, k, v, scale, causal, kvl)
    o, lse = online.tiled_forward(q, k, v, scale, causal, kvl, br, bc)
    np.testing.assert_allclose(o, ref["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Closed forms and invariants of the definition
# --------------------------------------------------------------------------

def _rand(rng, *shape, sigma=1.0):
    return rng.normal(0.0, sigma, size=shape)


@pytest.mark.parametrize("causal,kvl", [(False, None), (True, None), (False, 9), (True, 9)])
def test_rows_sum_to_one_and_hidden_probabilities_are_zero(causal, kvl):
    rng = np.random.default_rng(3)
    n = 17
    q, k = _rand(rng, n, 8, sigma=3.0), _rand(rng, n, 8, sigma=3.0)
    r = head_forward(q, k, _rand(rng, n, 8), 0.5, causal, kvl, want_p=True)
    p = r["p"]
    vis = visible_mask(n, causal, kvl)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[~vis] == 0.0)
    assert np.all(p[vis] > 0.0)
    # sum_j exp(S_ij - LSE_i) = 1, the recompute identity of page 2, 4.3.4.
    s = 0.5 * (q @ k.T)
    np.testing.assert_allclose(np.where(vis, np.exp(s - r["lse"][:, None]), 0.0).sum(1),
                               1.0, atol=1e-12)


@pytest.mark.parametrize("causal,kvl", [(False, None), (True, None), (False, 5), (True, 7)])
def test_zero_scale_gives_mean_of_visible_values(causal, kvl):
    rng = np.random.default_rng(4)
    n = 12
    q, k, v = _rand(rng, n, 4), _rand(rng, n, 4), _rand(rng, n, 4)
    r = head_forward(q, k, v, 0.0, causal, kvl)
    vis = visible_mask(n, causal, kvl)
    for i in range(n):
        np.testing.assert_allclose(r["o"][i], v[vis[i]].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert abs(r["lse"][i] - math.log(vis[i].sum())) <= 1e-13


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(5)
    n = 9
    q, k, v = _rand(rng, n, 5), _rand(rng, n, 5), _rand(rng, n, 5)
    r = head_forward(q, k, v, 0.3, True, None)
    np.testing.assert_array_equal(r["o"][0], v[0])
    assert abs(r["lse"][0] - 0.3 * float(q[0] @ k[0])) <= 1e-14
    r1 = head_forward(q, k, v, 0.3, False, 1)        # kv_len = 1
    np.testing.assert_array_equal(r1["o"], np.broadcast_to(v[0], (n, 5)))
    one = head_forward(q[:1], k[:1], v[:1], 0.3, False)  # N = 1
    np.testing.assert_array_equal(one["o"][0], v[0])


def test_equal_keys_give_uniform_weights_and_peaky_rows_pick_one_value():
    rng = np.random.default_rng(6)
    n = 10
    q, v = _rand(rng, n, 4), _rand(rng, n, 4)
    k = np.broadcast_to(_rand(rng, 1, 4), (n, 4))
    r = head_forward(q, k, v, 1.0, False, want_p=True)
    np.testing.assert_allclose(r["p"], 1.0 / n, rtol=1e-13)
    # One key aligned with q and scaled far above the rest: weight -> 1.
    k2 = _rand(rng, n, 4) * 0.01
    k2[6] = q[2] * 1e3
    r2 = head_forward(q, k2, v, 1.0, False)
    np.testing.assert_allclose(r2["o"][2], v[6], rtol=1e-12, atol=1e-12)


def test_causal_prefix_invariance_in_fp64():
    rng = np.random.default_rng(8)
    n, t = 20, 11
    q, k, v = _rand(rng, n, 6), _rand(rng, n, 6), _rand(rng, n, 6)
    k2, v2 = k.copy(), v.copy()
    k2[t + 1:] += 5.0
    v2[t + 1:] -= 7.0
    a = head_forward(q, k, v, 0.4, True)
    b = head_forward(q, k2, v2, 0.4, True)
    np.testing.assert_allclose(b["o"][: t + 1], a["o"][: t + 1], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(b["lse"][: t + 1], a["lse"][: t + 1], rtol=1e-15)


def test_padded_keys_get_exactly_zero_gradients_and_d_identity():
    rng = np.random.default_rng(9)
    n, kvl = 14, 9
    q, k, v, do = (_rand(rng, n, 5) for _ in range(4))
    for causal in (False, True):
        g = head_backward(q, k, v, do, 0.45, causal, kvl)
        assert np.all(g["dk"][kvl:] == 0.0) and np.all(g["dv"][kvl:] == 0.0)
        np.testing.assert_allclose(g["d"], (do * g["o"]).sum(axis=1), rtol=1e-12, atol=1e-14)


def test_fully_hidden_row_gives_zero_output_and_minus_inf_lse():
    rng = np.random.default_rng(10)
    q, k, v, do = (_rand(rng, 4, 3) for _ in range(4))
    r = head_forward(q, k, v, 1.0, False, 0)
    assert np.all(r["o"] == 0.0) and np.all(r["lse"] == -np.inf)
    g = head_backward(q, k, v, do, 1.0, False, 0)
    for key in ("dq", "dk", "dv"):
        assert np.all(g[key] == 0.0)


# --------------------------------------------------------------------------
# Finite differences of f = sum(O * dO)
# --------------------------------------------------------------------------

def _fd_check(fwd, bwd, causal, kvl, n=9, d=4, seed=11, h=1e-6):
    rng = np.random.default_rng(seed)
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    scale = 0.7
    g = bwd(q, k, v, do, scale, causal, kvl)

    def f(qq, kk, vv):
        return float((fwd(qq, kk, vv, scale, causal, kvl)["o"] * do).sum())

    worst = 0.0
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = {"dq": 0, "dk": 1, "dv": 2}[name]
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        err = np.abs(num - g[name]).max() / max(np.abs(num).max(), 1e-30)
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("causal,kvl", [(False, None), (True, None), (False, 6), (True, 5)])
def test_backward_matches_central_finite_differences(causal, kvl):
    assert _fd_check(head_forward, head_backward, causal, kvl) <= 1e-6


# --------------------------------------------------------------------------
# Library cross-check: torch CPU float64 SDPA and autograd
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (False, True), (True, True)])
def test_cross_check_against_torch_cpu_float64_sdpa(causal, padded):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(12)
    b, hh, n, d = 2, 3, 19, 8
    q, k, v, do = (torch.randn(b, hh, n, d, generator=g, dtype=torch.float64) for _ in range(4))
    kv_len = np.array([13, 19]) if padded else None
    scale = 0.29
    mask = None
    if padded or causal:
        vis = np.stack([visible_mask(n, causal, None if kv_len is None else kv_len[i])
                        for i in range(b)])[:, None]
        mask = torch.from_numpy(vis)
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    ref.backward(do)
    o, lse = oracle.attention_fwd(q.numpy(), k.numpy(), v.numpy(), causal, scale, kv_len)
    dq, dk, dv = oracle.attention_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(),
                                      causal, scale, kv_len)
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=1e-12, atol=1e-13)
    for mine, theirs in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(mine, theirs.numpy(), rtol=1e-11, atol=1e-12)
    s = scale * (q @ k.transpose(-1, -2))
    if mask is not None:
        s = s.masked_fill(~mask, -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Grouped K/V heads (GQA / MQA)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("heads_kv", [1, 2, 3])
@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (True, True)])
def test_grouped_heads_cross_check_against_torch_sdpa_enable_gqa(heads_kv, causal, padded):
    """torch's CPU float64 SDPA with enable_gqa (query head h uses K/V head
    h // (H // H_kv)) and its autograd, which sums the gradients of a shared
    K/V head over its group."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(31 + heads_kv)
    b, hh, n, d = 2, 6, 17, 8
    q, do = (torch.randn(b, hh, n, d, generator=g, dtype=torch.float64) for _ in range(2))
    k, v = (torch.randn(b, heads_kv, n, d, generator=g, dtype=torch.float64) for _ in range(2))
    kv_len = np.array([11, 17]) if padded else None
    scale = 0.37
    mask = None
    if padded or causal:
        vis = np.stack([visible_mask(n, causal, None if kv_len is None else kv_len[i])
                        for i in range(b)])[:, None]
        mask = torch.from_numpy(vis)
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    ref.backward(do)
    o, _ = oracle.attention_fwd(q.numpy(), k.numpy(), v.numpy(), causal, scale, kv_len)
    dq, dk, dv = oracle.attention_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(),
                                      causal, scale, kv_len)
    assert dk.shape == (b, heads_kv, n, d)
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=1e-12, atol=1e-13)
    for mine, theirs in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(mine, theirs.numpy(), rtol=1e-11, atol=1e-12)


def _fd_grouped(fwd, bwd, causal, h=1e-6):
    """Central differences of f = sum(O * dO) over every entry of q, k, v for a
    tiny grouped problem (4 query heads, 2 K/V heads)."""
    rng = np.random.default_rng(17)
    q, do = rng.standard_normal((1, 4, 6, 3)), rng.standard_normal((1, 4, 6, 3))
    k, v = rng.standard_normal((1, 2, 6, 3)), rng.standard_normal((1, 2, 6, 3))
    scale = 0.8
    grads = bwd(q, k, v, do, causal, scale)

    def f(args):
        return float((fwd(*args, causal, scale)[0] * do).sum())

    worst = 0.0
    for pos, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            ap, am = [q, k, v], [q, k, v]
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap[pos], am[pos] = xp, xm
            num[idx] = (f(ap) - f(am)) / (2 * h)
        worst = max(worst, np.abs(num - grads[pos]).max() / np.abs(num).max())
    return worst


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_backward_matches_finite_differences(causal):
    assert _fd_grouped(oracle.attention_fwd, oracle.attention_bwd, causal) <= 1e-6


def test_grouped_heads_planted_mistakes_are_rejected():
    """Two plausible slips: interleaved head mapping (h % H_kv) and dK/dV
    taken from the first head of a group instead of summed over it."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    def fwd_interleaved(q, k, v, causal, scale, kv_len=None):
        hkv = k.shape[1]
        o = np.empty_like(q)
        for h in range(q.shape[1]):
            o[0, h] = head_forward(q[0, h], k[0, h % hkv], v[0, h % hkv], scale, causal)["o"]
        return o, None

    def bwd_first_only(q, k, v, do, causal, scale, kv_len=None):
        grp = q.shape[1] // k.shape[1]
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)
        for g in range(k.shape[1]):
            r = head_backward(q[0, g * grp], k[0, g], v[0, g], do[0, g * grp], scale, causal)
            dk[0, g], dv[0, g] = r["dk"], r["dv"]
        return dq, dk, dv

    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((1, 4, 7, 3)), rng.standard_normal((1, 2, 7, 3)), rng.standard_normal((1, 2, 7, 3))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                         scale=0.5, enable_gqa=True).numpy()
    assert not np.allclose(fwd_interleaved(q, k, v, False, 0.5)[0], ref, atol=1e-6)
    assert np.allclose(oracle.attention_fwd(q, k, v, False, 0.5)[0], ref, atol=1e-12)
    assert _fd_grouped(oracle.attention_fwd, bwd_first_only, False) > 1e-3


# --------------------------------------------------------------------------
# Packed variable-length batches (page 2 4.7.2 / 4.7.4). The pins build the
# block-diagonal mask from a segment id per row -- independently of the
# oracle's span loop -- and hand the whole packed batch to torch's CPU float64
# SDPA (and its autograd, and torch.logsumexp for the LSE).

VARLEN_CU = [0, 5, 6, 6, 19, 27]   # lengths 5, 1, 0 (empty), 13, 8


def _varlen_inputs(heads, heads_kv, d, seed):
    rng = np.random.default_rng(seed)
    t = VARLEN_CU[-1]
    q, do = rng.standard_normal((heads, t, d)), rng.standard_normal((heads, t, d))
    k, v = rng.standard_normal((heads_kv, t, d)), rng.standard_normal((heads_kv, t, d))
    return q, k, v, do


def _block_diagonal(cu, causal):
    t = cu[-1]
    seg = np.zeros(t, dtype=np.int64)
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        seg[a:e] = s
    i, j = np.arange(t)[:, None], np.arange(t)[None, :]
    vis = seg[:, None] == seg[None, :]
    if causal:
        vis &= j <= i
    return vis


def _torch_varlen(q, k, v, do, cu, causal, scale):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    mask = torch.from_numpy(_block_diagonal(cu, causal))
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=mask,
                                       scale=scale, enable_gqa=True)[0]
    o.backward(torch.from_numpy(do))
    grp = q.shape[0] // k.shape[0]
    s = scale * torch.matmul(torch.from_numpy(q), torch.from_numpy(np.repeat(k, grp, 0)).transpose(1, 2))
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return (o.detach().numpy(), lse.numpy(), qt.grad.numpy(), kt.grad.numpy(),
            vt.grad.numpy())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads_kv", [1, 2, 4])
def test_varlen_matches_block_diagonal_sdpa(causal, heads_kv):
    q, k, v, do = _varlen_inputs(4, heads_kv, 8, seed=40 + heads_kv)
    scale = 0.41
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = _torch_varlen(q, k, v, do, VARLEN_CU, causal, scale)
    o, lse = oracle.varlen_fwd(q, k, v, VARLEN_CU, causal, scale)
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, VARLEN_CU, causal, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
    for mine, theirs in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(mine, theirs, rtol=1e-11, atol=1e-12)


def test_varlen_single_row_sequence_returns_its_value_row():
    # A sequence of one row sees only itself: O = V row, LSE = scale q.k.
    q, k, v, _ = _varlen_inputs(2, 2, 4, seed=3)
    o, lse = oracle.varlen_fwd(q, k, v, VARLEN_CU, False, 0.7)
    np.testing.assert_array_equal(o[:, 5], v[:, 5])
    np.testing.assert_allclose(lse[:, 5], 0.7 * (q[:, 5] * k[:, 5]).sum(-1), rtol=1e-14)


def test_varlen_sequence_order_is_irrelevant():
    # Permuting whole sequences permutes the outputs the same way.
    q, k, v, do = _varlen_inputs(2, 1, 4, seed=9)
    spans = list(zip(VARLEN_CU[:-1], VARLEN_CU[1:]))
    order = [3, 0, 4, 1, 2]
    rows = np.concatenate([np.arange(*spans[s]) for s in order]).astype(np.int64)
    cu2 = np.cumsum([0] + [spans[s][1] - spans[s][0] for s in order])
    o, _ = oracle.varlen_fwd(q, k, v, VARLEN_CU, True, 0.5)
    o2, _ = oracle.varlen_fwd(q[:, rows], k[:, rows], v[:, rows], cu2, True, 0.5)
    np.testing.assert_allclose(o2, o[:, rows], rtol=0, atol=1e-15)
    dq, dk, _ = oracle.varlen_bwd(q, k, v, do, VARLEN_CU, True, 0.5)
    dq2, dk2, _ = oracle.varlen_bwd(q[:, rows], k[:, rows], v[:, rows], do[:, rows], cu2, True, 0.5)
    np.testing.assert_allclose(dq2, dq[:, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk2, dk[:, rows], rtol=0, atol=1e-14)


def test_varlen_planted_mistakes_are_rejected(monkeypatch):
    """Sequence spans that start one row early (the previous sequence's last
    key leaks in, visible even under the causal mask) and the packed batch
    treated as one sequence are both caught by the block-diagonal SDPA pin."""
    import oracle.attention as oa
    q, k, v, do = _varlen_inputs(2, 2, 4, seed=12)
    o_ref = _torch_varlen(q, k, v, do, VARLEN_CU, True, 0.6)[0]
    good = oa._spans
    monkeypatch.setattr(oa, "_spans", lambda cu: [(max(a - 1, 0), e) for a, e in good(cu)])
    assert not np.allclose(oracle.varlen_fwd(q, k, v, VARLEN_CU, True, 0.6)[0], o_ref, atol=1e-6)
    monkeypatch.setattr(oa, "_spans", lambda cu: [(0, VARLEN_CU[-1])])
    assert not np.allclose(oracle.varlen_fwd(q, k, v, VARLEN_CU, True, 0.6)[0], o_ref, atol=1e-6)
    monkeypatch.setattr(oa, "_spans", good)
    np.testing.assert_allclose(oracle.varlen_fwd(q, k, v, VARLEN_CU, True, 0.6)[0], o_ref,
                               rtol=1e-12, atol=1e-13)


def test_varlen_rejects_bad_offsets():
    q, k, v, _ = _varlen_inputs(1, 1, 4, seed=1)
    with pytest.raises(ValueError):
        oracle.varlen_fwd(q, k, v, [1, 27], False)
    with pytest.raises(ValueError):
        oracle.varlen_fwd(q, k, v, [0, 9, 5, 27], False)


# --------------------------------------------------------------------------
# Planted mistakes: each must be rejected by at least one pin
# --------------------------------------------------------------------------

def _fwd_pins_reject(fwd):
    """Run the forward pins against ``fwd``; True if any of them fails."""
    rng = np.random.default_rng(21)
    n = 10
    q, k, v = _rand(rng, n, 4), _rand(rng, n, 4), _rand(rng, n, 4)
    checks = []
    for causal, kvl in ((False, None), (True, None), (False, 6), (True, 6)):
        for scale in (0.0, 0.6):
            r = fwd(q, k, v, scale, causal, kvl)
            vis = visible_mask(n, causal, kvl)
            # closed form at scale 0 / the exact definition via torch
            if scale == 0.0:
                mean = np.stack([v[vis[i]].mean(0) for i in range(n)])
                checks.append(np.allclose(r["o"], mean, atol=1e-12))
                checks.append(np.allclose(r["lse"], np.log(vis.sum(1)), atol=1e-12))
            else:
                torch = pytest.importorskip("torch")
                import torch.nn.functional as F
                t = [torch.from_numpy(x)[None, None] for x in (q, k, v)]
                ref = F.scaled_dot_product_attention(*t, attn_mask=torch.from_numpy(vis),
                                                     scale=scale)[0, 0].numpy()
                checks.append(np.allclose(r["o"], ref, rtol=1e-10, atol=1e-12))
                s = np.where(vis, scale * q @ k.T, -np.inf)
                lse_ref = np.log(np.where(vis, np.exp(s), 0.0).sum(1))
                checks.append(np.allclose(r["lse"], lse_ref, rtol=1e-10, atol=1e-12))
    return not all(checks)


def test_planted_mistakes_are_rejected():
    # The correct oracle passes its pins...
    assert not _fwd_pins_reject(head_forward)
    assert _fd_check(head_forward, head_backward, True, 6) <= 1e-6

    def mutate_forward(kind):
        def fwd(q, k, v, scale, causal, kvl=None, rows=None, want_p=False):
            if kind == "dropped_scale":
                scale = 1.0
            if kind == "transposed_operand":
                q, k = k, q
            r = head_forward(q, k, v, scale, causal if kind != "causal_off_by_one" else False,
                             kvl, want_p=True)
            if kind == "causal_off_by_one" and causal:
                n = k.shape[0]
                vis = visible_mask(n, False, kvl) & (np.arange(n)[None, :] < np.arange(n)[:, None] + 2)
                s = np.where(vis, scale * (np.asarray(q) @ np.asarray(k).T), -np.inf)
                m = s.max(1, keepdims=True)
                e = np.where(vis, np.exp(s - m), 0.0)
                r = {"o": (e / e.sum(1, keepdims=True)) @ v, "lse": m[:, 0] + np.log(e.sum(1))}
            if kind == "lse_without_max":
                r["lse"] = r["lse"] - np.where(np.isfinite(r["lse"]), 0.0, 0.0) - 1.0
            if kind == "mask_padding_ignored" and kvl is not None:
                r = head_forward(q, k, v, scale, causal, None)
            return r
        return fwd

    for kind in ("dropped_scale", "transposed_operand", "causal_off_by_one",
                 "lse_without_max", "mask_padding_ignored"):
        assert _fwd_pins_reject(mutate_forward(kind)), kind

    def mutate_backward(kind):
        def bwd(q, k, v, do, scale, causal, kvl=None):
            g = head_backward(q, k, v, do, scale, causal, kvl)
            p = head_forward(q, k, v, scale, causal, kvl, want_p=True)["p"]
            dp = do @ v.T
            if kind == "dropped_d_term":
                ds = p * dp
                g["dq"], g["dk"] = scale * ds @ k, scale * ds.T @ q
            if kind == "transposed_ds_in_dk":
                ds = p * (dp - g["d"][:, None])
                g["dk"] = scale * ds @ q
            if kind == "dropped_scale_in_dq":
                g["dq"] = g["dq"] / scale
            if kind == "dv_not_transposed":
                g["dv"] = p @ do
            return g
        return bwd

    for kind in ("dropped_d_term", "transposed_ds_in_dk", "dropped_scale_in_dq",
                 "dv_not_transposed"):
        assert _fd_check(head_forward, mutate_backward(kind), True, 6) > 1e-3, kind


# --------------------------------------------------------------------------
# Sliding windows and block-sparse masks (page 4 下篇 section 六's
# window_size; page 3 第八部分's block-level mask). The pins build the mask
# element by element in plain Python loops -- independently of the oracle's
# vectorised visible_mask -- and hand it to torch's CPU float64 SDPA.

def _brute_visible(n, causal, kv_len, window, block_mask, block=128):
    vis = np.zeros((n, n), dtype=bool)
    left, right = window
    for i in range(n):
        for j in range(n):
            ok = True
            if causal and j > i:
                ok = False
            if kv_len is not None and j >= kv_len:
                ok = False
            if left >= 0 and j < i - left:
                ok = False
            if right >= 0 and j > i + right:
                ok = False
            if block_mask is not None and not block_mask[i // block][j // block]:
                ok = False
            vis[i, j] = ok
    return vis


def _asym_block_mask(n, seed):
    nb = (n + 127) // 128
    rng = np.random.default_rng(seed)
    bm = rng.random((nb, nb)) < 0.6
    bm[0, 1], bm[1, 0] = True, False  # not symmetric: a transposed mask differs
    return bm


MASK_CASES = [
    # (causal, kv_len, window, use_block_mask)
    (False, None, (37, 5), False),
    (True, None, (100, -1), False),
    (False, 250, (-1, 60), False),
    (False, None, (-1, -1), True),
    (True, 280, (-1, -1), True),
    (False, None, (150, 150), True),
]


@pytest.mark.parametrize("causal,kv_len,window,use_bm", MASK_CASES)
def test_window_and_block_masks_match_brute_force_sdpa(causal, kv_len, window, use_bm):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    n, d, scale = 300, 8, 0.3
    bm = _asym_block_mask(n, 7) if use_bm else None
    vis = _brute_visible(n, causal, kv_len, window, bm)
    np.testing.assert_array_equal(visible_mask(n, causal, kv_len, None, window, bm), vis)
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    keep = vis.any(axis=1)  # SDPA gives NaN on rows with no visible key
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    o_ref = F.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                           attn_mask=torch.from_numpy(vis), scale=scale)[0]
    o_ref = torch.where(torch.from_numpy(keep)[:, None], o_ref, torch.zeros_like(o_ref))
    o_ref.backward(torch.from_numpy(do))
    r = head_backward(q, k, v, do, scale, causal, kv_len, window, bm)
    np.testing.assert_allclose(r["o"], o_ref.detach().numpy(), rtol=1e-12, atol=1e-13)
    for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
        g = np.nan_to_num(t.grad.numpy())
        np.testing.assert_allclose(r[name], g, rtol=1e-11, atol=1e-12)
    assert np.all(r["lse"][~keep] == -np.inf) and np.all(r["o"][~keep] == 0.0)


def test_zero_window_returns_each_rows_own_value():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((50, 4)) for _ in range(3))
    r = head_forward(q, k, v, 0.9, False, window=(0, 0))
    np.testing.assert_array_equal(r["o"], v)
    np.testing.assert_allclose(r["lse"], 0.9 * (q * k).sum(1), rtol=1e-14)


def test_diagonal_block_mask_equals_packed_sequences_of_one_block():
    # Only the diagonal blocks kept = independent sequences of 128 rows: the
    # packed-batch oracle (slices, no block mask) must agree.
    rng = np.random.default_rng(4)
    n, d = 384, 8
    q, k, v, do = (rng.standard_normal((1, n, d)) for _ in range(4))
    bm = np.eye(3, dtype=bool)
    o, lse = oracle.attention_fwd(q[None], k[None], v[None], True, 0.4, block_mask=bm)
    o2, lse2 = oracle.varlen_fwd(q, k, v, [0, 128, 256, 384], True, 0.4)
    np.testing.assert_allclose(o[0], o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[0], lse2, rtol=1e-13)
    g = oracle.attention_bwd(q[None], k[None], v[None], do[None], True, 0.4, block_mask=bm)
    g2 = oracle.varlen_bwd(q, k, v, do, [0, 128, 256, 384], True, 0.4)
    for a, b in zip(g, g2):
        np.testing.assert_allclose(a[0], b, rtol=1e-12, atol=1e-13)


def test_window_and_block_planted_mistakes_are_rejected():
    n = 300
    bm = _asym_block_mask(n, 7)
    ref = _brute_visible(n, False, None, (37, 5), None)
    # window lower edge off by one (j > i - left instead of j >= i - left)
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    wrong = (j > i - 37) & (j <= i + 5)
    assert not np.array_equal(wrong, ref)
    assert np.array_equal(visible_mask(n, False, None, None, (37, 5)), ref)
    # block mask read transposed
    ref_b = _brute_visible(n, False, None, (-1, -1), bm)
    wrong_b = visible_mask(n, False, None, None, (-1, -1), bm.T)
    assert not np.array_equal(wrong_b, ref_b)
    assert np.array_equal(visible_mask(n, False, None, None, (-1, -1), bm), ref_b)


@pytest.mark.parametrize("causal,window", [(True, (50, -1)), (False, (40, 30))])
def test_window_locality_of_slices(causal, window):
    """The property the maximum-size GPU test rests on: with a window, the
    oracle on a slice [a, e) of the sequence gives the full problem's O, LSE
    and dQ for rows whose window lies inside the slice, and its dK, dV for
    keys whose queries do (the masks depend on i - j only)."""
    from test_max_size_gpu import _segments, _valid
    n, d = 900, 16
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    full = head_backward(q, k, v, do, 0.3, causal, None, window)
    left, right = window[0], 0 if causal else window[1]
    for a, e in _segments(n, left, right):
        (f_lo, f_hi), (k_lo, k_hi) = _valid(n, a, e, left, right)
        assert f_hi - f_lo > 0 and k_hi - k_lo > 0
        part = head_backward(q[a:e], k[a:e], v[a:e], do[a:e], 0.3, causal, None, window)
        for name, lo, hi in (("o", f_lo, f_hi), ("lse", f_lo, f_hi), ("dq", f_lo, f_hi),
                             ("dk", k_lo, k_hi), ("dv", k_lo, k_hi)):
            np.testing.assert_allclose(part[name][lo - a:hi - a], full[name][lo:hi],
                                       rtol=1e-10, atol=1e-12, err_msg=name)
        # One row or key more on either side would reach outside the slice.
        if a > 0:
            lo = f_lo - 1 - a
            assert not np.allclose(part["dq"][lo], full["dq"][f_lo - 1], rtol=1e-10, atol=1e-12)
            lo = k_lo - 1 - a
            assert not np.allclose(part["dk"][lo], full["dk"][k_lo - 1], rtol=1e-10, atol=1e-12)
