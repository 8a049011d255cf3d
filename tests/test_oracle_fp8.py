"""Pins for the FP8 (E4M3) forward oracle, oracle/fp8.py (runs without a GPU).

The oracle is checked against things other than itself:

* the format figures page 2 prints (exercise 3: largest magnitude 448,
  smallest normal 2^-6; tests/golden/fp8_format.json);
* a library cross-check of the E4M3 rounding against torch's float8_e4m3fn
  cast, and the round trip of every finite code;
* scipy's Hadamard matrix, orthogonality, and the page's identity
  (Q H)(K H)^T = Q K^T;
* brute force for the block exponent (smallest e with amax <= 448 * 2^e);
* closed forms: two groups of equal keys give the library-rounded weights'
  average of the two groups' mean value rows; constant V gives exactly that
  constant; the LSE lies within ln(1 + 2^-4) of scipy's logsumexp of the
  dequantised scores;
* the tiled online forward with running integer frames, written here
  independently (library E4M3 rounding, any tile width, either tile order),
  agrees with the one-shot definition, exactly when every probability is in
  E4M3's normal range and within the subnormal bound otherwise;
* the error against exact attention stays inside E4M3's relative rounding
  bound, and the rotation lowers the score error on inputs with outlier
  channels (the page's reason for it);
* planted mistakes in the oracle are each rejected by one of the pins.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
from oracle import fp8 as of

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_format.json")
LOG2E = 1.0 / math.log(2.0)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _torch_e4m3(x):
    """Library E4M3 rounding: torch's float8_e4m3fn cast (in range)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy())
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _inputs(seed, b=1, h=2, n=300, d=64, hkv=None, outliers=0):
    rng = np.random.default_rng(seed)
    hkv = h if hkv is None else hkv
    q = rng.standard_normal((b, h, n, d))
    k = rng.standard_normal((b, hkv, n, d))
    v = rng.standard_normal((b, hkv, n, d))
    if outliers:
        ch = rng.choice(d, outliers, replace=False)
        q[..., ch] *= 30.0
        k[..., ch] *= 30.0
    return q, k, v


# --------------------------------------------------------------------------
# The E4M3 format
# --------------------------------------------------------------------------

def test_page2_format_figures():
    g = _golden()["e4m3_range"]
    vals = of.e4m3_decode(np.arange(256))
    finite = vals[np.isfinite(vals)]
    assert np.max(np.abs(finite)) == g["max_magnitude"] == of.E4M3_MAX
    normals = np.abs(finite)[np.abs(finite) >= g["min_normal"]]
    assert np.min(normals) == g["min_normal"] == 2.0 ** g["min_normal_as_power_of_two"]
    assert of.e4m3_encode(448.0) == 0x7E and of.e4m3_encode(-448.0) == 0xFE
    assert of.e4m3_encode(2.0 ** -6) == 0x08
    assert of.e4m3_encode(2.0 ** -9) == 0x01
    assert of.e4m3_encode(1.0) == 0x38
    # Only S.1111.111 is NaN: 254 finite codes, no infinities.
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and finite.size == 254


def test_e4m3_round_matches_library_cast():
    rng = np.random.default_rng(1)
    mags = 2.0 ** rng.uniform(-13, math.log2(448.0), 200_000)
    x = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32).astype(np.float64)
    grid = np.unique(np.abs(of.e4m3_decode(np.arange(127))))
    mids = (grid[1:] + grid[:-1]) / 2  # exact ties: the even neighbour wins
    x = np.concatenate([x, mids, -mids, grid, [0.0, 448.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    np.testing.assert_array_equal(of.e4m3_round(x), _torch_e4m3(x))
    # Ties to even: 1 + 2^-4 lies halfway between 1 (mantissa 0) and 1.125.
    assert of.e4m3_round(1.0625) == 1.0 and of.e4m3_round(1.1875) == 1.25
    # Saturation past the largest value.
    assert of.e4m3_round(1000.0) == 448.0 and of.e4m3_round(-460.0) == -448.0


def test_e4m3_encode_decode_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    np.testing.assert_array_equal(of.e4m3_encode(of.e4m3_decode(codes)), codes)
    torch_codes = torch.from_numpy(of.e4m3_decode(codes).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(torch_codes, codes)
    # Rounding is monotone and idempotent.
    x = np.sort(np.random.default_rng(2).uniform(-448, 448, 10_000))
    r = of.e4m3_round(x)
    assert np.all(np.diff(r) >= 0)
    np.testing.assert_array_equal(of.e4m3_round(r), r)


# --------------------------------------------------------------------------
# Hadamard rotation and block scales
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [1, 2, 8, 64, 128, 256])
def test_hadamard_is_sylvester_and_orthogonal(d):
    h = of.hadamard(d)
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(d))
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


def test_rotation_keeps_scores():
    rng = np.random.default_rng(3)
    d = 128
    s = rng.choice([-1.0, 1.0], d)
    r = of.rotation(s)
    np.testing.assert_array_equal(r, np.diag(s) @ scipy.linalg.hadamard(d))
    hm = r / math.sqrt(d)  # the page's H: entries +-1/sqrt(d), H H^T = I
    np.testing.assert_allclose(hm @ hm.T, np.eye(d), atol=1e-15)
    q, k = rng.standard_normal((50, d)), rng.standard_normal((60, d))
    np.testing.assert_allclose((q @ hm) @ (k @ hm).T, q @ k.T, atol=1e-12)
    with pytest.raises(ValueError):
        of.rotation(np.full(d, 0.5))
    with pytest.raises(ValueError):
        of.hadamard(96)


def test_block_exponent_is_the_smallest():
    rng = np.random.default_rng(4)
    amax = np.concatenate([2.0 ** rng.uniform(-30, 30, 5000),
                           448.0 * 2.0 ** np.arange(-20, 20),
                           np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), np.inf)])
    e = of.block_exponent(amax)
    for a, ei in zip(amax, e):
        assert a <= 448.0 * 2.0 ** ei
        assert a > 448.0 * 2.0 ** (ei - 1)
    assert of.block_exponent(0.0) == 0


def test_quantize_blocks_and_bounds():
    q, _, _ = _inputs(5, b=2, h=3, n=300, d=64)
    q[1, 2, 128:256] *= 1e-3  # a block with its own, much smaller scale
    codes, scales = of.quantize(q)
    assert codes.shape == (2, 3, 384, 64) and scales.shape == (2, 3, 3)
    assert np.all(codes[:, :, 300:] == 0)  # padding rows
    e = np.log2(scales)
    np.testing.assert_array_equal(e, np.round(e))  # powers of two
    for b in range(2):
        for h in range(3):
            x = q[b, h]
            xd = of.dequantize(codes[b, h], scales[b, h], 300)
            sc = scales[b, h][np.arange(300) // 128][:, None]
            # Block maxima land in (224, 448] once scaled (tight scaling).
            for blk in range(3):
                seg = np.abs(x[blk * 128:(blk + 1) * 128]) / scales[b, h, blk]
                assert 224.0 < seg.max() <= 448.0
            # Half an E4M3 step: 2^-4 relative in the normal range, 2^-10
            # absolute (in scaled units) below it.
            err = np.abs(xd - x)
            bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sc)
            assert np.all(err <= bound * (1 + 1e-12))


def test_rotated_quantize_represents_x_times_h():
    rng = np.random.default_rng(6)
    d = 64
    s = rng.choice([-1.0, 1.0], d)
    x, _, _ = _inputs(7, n=200, d=d)
    codes, scales = of.quantize(x, s)
    xh = x[0, 0] @ (np.diag(s) @ scipy.linalg.hadamard(d)) / math.sqrt(d)
    xd = of.dequantize(codes[0, 0], scales[0, 0], 200)
    sc = scales[0, 0][np.arange(200) // 128][:, None]
    assert np.all(np.abs(xd - xh) <= np.maximum(2.0 ** -4 * np.abs(xh), 2.0 ** -10 * sc) + 1e-15)
    # The scale carries the 1/sqrt(d): scale * sqrt(d) is a power of two.
    e = np.log2(scales * math.sqrt(d))
    np.testing.assert_allclose(e, np.round(e), atol=1e-12)


def test_rotation_flattens_outlier_channels():
    """Page 2 4.5.4: the rotation spreads outliers and lowers the FP8 error."""
    d = 128
    q, k, _ = _inputs(8, n=256, d=d, outliers=3)
    s = np.random.default_rng(9).choice([-1.0, 1.0], d)
    exact = q[0, 0] @ k[0, 0].T

    def score_err(signs):
        qc, qs = of.quantize(q, signs)
        kc, ks = of.quantize(k, signs)
        sq = of.dequantize(qc[0, 0], qs[0, 0], 256) @ of.dequantize(kc[0, 0], ks[0, 0], 256).T
        return np.linalg.norm(sq - exact) / np.linalg.norm(exact)

    plain, rotated = score_err(None), score_err(s)
    assert rotated < 0.5 * plain
    # The rotated tensor's peak-to-rms ratio drops.
    qr = q[0, 0] @ of.rotation(s)
    ratio = lambda a: np.abs(a).max() / np.sqrt((a ** 2).mean())  # noqa: E731
    assert ratio(qr) < 0.5 * ratio(q[0, 0])


# --------------------------------------------------------------------------
# The forward
# --------------------------------------------------------------------------

def _head(qc, qs, kc, ks, vc, vs, n, scale, causal=False, kvb=None):
    return of.fp8_head_forward(qc[0, 0], qs[0, 0], kc[0, 0], ks[0, 0], vc[0, 0], vs[0, 0],
                               n, scale, causal, kvb, parts=True)


def test_two_key_groups_closed_form():
    """Keys equal within each of two groups: a row's scores take two values
    t_A, t_B, so with f = ceil(max(t_A, t_B)), u = 2^(t - f + 8) and
    P^ = E4M3(u) (library rounding) the output is
    (n_A P^_A vbar_A + n_B P^_B vbar_B) / (n_A P^_A + n_B P^_B)."""
    rng = np.random.default_rng(10)
    n, d, na = 200, 64, 77
    q = rng.standard_normal((1, 1, n, d))
    k = np.empty((1, 1, n, d))
    k[0, 0, :na] = rng.standard_normal(d)
    k[0, 0, na:] = rng.standard_normal(d)
    v = rng.standard_normal((1, 1, n, d))
    qc, qs = of.quantize(q)
    kc, ks = of.quantize(k)
    vc, vs = of.quantize(v)
    scale = 0.61
    r = _head(qc, qs, kc, ks, vc, vs, n, scale)
    qd = of.dequantize(qc[0, 0], qs[0, 0], n)
    kd = of.dequantize(kc[0, 0], ks[0, 0], n)
    vd = of.dequantize(vc[0, 0], vs[0, 0], n)
    ta = scale * (qd @ kd[0]) * LOG2E
    tb = scale * (qd @ kd[na]) * LOG2E
    f = np.ceil(np.maximum(ta, tb))
    pa, pb = _torch_e4m3(2.0 ** (ta - f + 8)), _torch_e4m3(2.0 ** (tb - f + 8))
    va, vb = vd[:na].mean(axis=0), vd[na:].mean(axis=0)
    want = (na * pa[:, None] * va + (n - na) * pb[:, None] * vb) / (na * pa + (n - na) * pb)[:, None]
    np.testing.assert_allclose(r["o"], want, rtol=1e-12, atol=1e-14)
    # The rounding of P is visible: unrounded weights give another result.
    ua, ub = 2.0 ** (ta - f + 8), 2.0 ** (tb - f + 8)
    plain = (na * ua[:, None] * va + (n - na) * ub[:, None] * vb) / (na * ua + (n - na) * ub)[:, None]
    assert np.abs(plain - want).max() > 1e-3
    # The larger group's u lies in (128, 256]: the frame is the ceiling.
    top = np.maximum(2.0 ** (ta - f + 8), 2.0 ** (tb - f + 8))
    assert np.all((top > 128) & (top <= 256))


def test_constant_values_give_exactly_that_value():
    """O is a convex combination of V rows (the weights are the rounded
    probabilities over their own sum): V = 1 everywhere gives O = 1 exactly,
    for any scores and masks."""
    q, k, _ = _inputs(21, n=300, d=64)
    v = np.ones((1, 2, 300, 64))
    for causal, kvl in ((False, None), (True, [250])):
        o, _ = of.fp8_attention_fwd(q * 2.5, k, v, causal=causal, kv_len=kvl)
        np.testing.assert_array_equal(o, np.ones_like(o))


def test_lse_is_near_logsumexp_of_quantised_scores():
    q, k, v = _inputs(11, n=300, d=64)
    qc, qs = of.quantize(q)
    kc, ks = of.quantize(k)
    vc, vs = of.quantize(v)
    for causal, kvb in [(False, None), (True, None), (False, 170), (True, 170)]:
        r = _head(qc, qs, kc, ks, vc, vs, 300, 0.125, causal, kvb)
        qd = of.dequantize(qc[0, 0], qs[0, 0], 300)
        kd = of.dequantize(kc[0, 0], ks[0, 0], 300)
        s = 0.125 * qd @ kd.T
        vis = oracle.visible_mask(300, causal, kvb)
        ref = scipy.special.logsumexp(np.where(vis, s, -np.inf), axis=1)
        # The rounded probabilities are each within 2^-4 of the exact ones,
        # so their sum is too: |LSE - logsumexp| <= ln(1 + 2^-4).
        err = np.abs(r["lse"] - ref)
        assert np.all(err <= math.log1p(2.0 ** -4) + 1e-12)
        assert err.max() > 1e-6


def _tiled_forward(qd, kd, vd, scale, bc, causal, kvb, reverse=False):
    """The online forward tile by tile with running integer frames (page 1
    section 六 / page 2 4.3.2 update, with the frame ceil of the running
    max), E4M3 rounding from the library."""
    n = qd.shape[0]
    f = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros_like(qd[:, :1] * vd[:1, :])
    starts = list(range(0, n, bc))
    if reverse:
        starts = starts[::-1]
    vis_all = oracle.visible_mask(n, causal, kvb)
    for j0 in starts:
        j1 = min(j0 + bc, n)
        vis = vis_all[:, j0:j1]
        t = np.where(vis, scale * (qd @ kd[j0:j1].T) * LOG2E, -np.inf)
        tmax = t.max(axis=1)
        fnew = np.where(np.isfinite(tmax), np.maximum(f, np.ceil(np.where(np.isfinite(tmax), tmax, 0))), f)
        alpha = np.where(np.isfinite(f), np.exp2(f - np.where(np.isfinite(fnew), fnew, 0)), 0.0)
        fr = np.where(np.isfinite(fnew), fnew, 0.0)
        u = np.where(vis, np.exp2(t - fr[:, None] + 8), 0.0)
        pq = _torch_e4m3(u)
        acc = acc * alpha[:, None] + pq @ vd[j0:j1]
        l = l * alpha + pq.sum(axis=1)
        f = fnew
    has = np.isfinite(f)
    o = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
    return o


@pytest.mark.parametrize("causal,kvb", [(False, None), (True, None), (True, 333)])
def test_tiled_online_forward_agrees(causal, kvb):
    q, k, v = _inputs(12, n=400, d=64)
    # Small scores: every u is in E4M3's normal range, so any tiling and any
    # tile order must reproduce the one-shot result exactly (up to fp64 sums).
    q *= 0.1
    qc, qs = of.quantize(q)
    kc, ks = of.quantize(k)
    vc, vs = of.quantize(v)
    r = _head(qc, qs, kc, ks, vc, vs, 400, 0.3, causal, kvb)
    assert np.all((r["u"] >= 2.0 ** -6) | ~r["vis"])
    qd, kd = of.dequantize(qc[0, 0], qs[0, 0], 400), of.dequantize(kc[0, 0], ks[0, 0], 400)
    vd = of.dequantize(vc[0, 0], vs[0, 0], 400)
    for bc in (64, 128, 37):
        for rev in (False, True):
            o = _tiled_forward(qd, kd, vd, 0.3, bc, causal, kvb, rev)
            np.testing.assert_allclose(o, r["o"], rtol=0, atol=1e-12)


def test_tiled_online_forward_subnormal_bound():
    """With peaky rows some u fall below 2^-6 in the final frame; a tiled run
    may round them in a finer running frame. Each such P^ moves by at most
    2^-9 (half a subnormal step on either side), in the numerator and in l
    alike, so |dO| <= 2^-9 (sum|v| + m |O|) / (l - 2^-9 m) over the m small
    entries of the row."""
    q, k, v = _inputs(13, n=384, d=64)
    qc, qs = of.quantize(q * 3.0)
    kc, ks = of.quantize(k)
    vc, vs = of.quantize(v)
    r = _head(qc, qs, kc, ks, vc, vs, 384, 0.25, True)
    small = (r["u"] < 2.0 ** -6) & r["vis"]
    assert small.sum() > 1000
    qd, kd = of.dequantize(qc[0, 0], qs[0, 0], 384), of.dequantize(kc[0, 0], ks[0, 0], 384)
    vd = of.dequantize(vc[0, 0], vs[0, 0], 384)
    m = small.sum(axis=1)[:, None]
    bound = 2.0 ** -9 * ((small.astype(float) @ np.abs(vd)) + m * np.abs(r["o"])) / (
        r["l"][:, None] - 2.0 ** -9 * m) + 1e-12
    for bc in (64, 128):
        o = _tiled_forward(qd, kd, vd, 0.25, bc, True, None, reverse=True)
        assert np.all(np.abs(o - r["o"]) <= bound)


@pytest.mark.parametrize("rotate", [False, True])
def test_close_to_exact_attention(rotate):
    """Against exact attention on the unquantised inputs. Each of the three
    roundings (Q and K through the scores, V, and P) has a relative error
    of at most half an E4M3 step, 2^-4, and about 2^-4 / sqrt(3) in RMS;
    three independent ones add to about 6% in RMS, so the normwise error of
    O stays below 2^-3. It is far from zero because P is rounded too."""
    q, k, v = _inputs(14, b=2, h=4, n=260, d=64, hkv=2)
    s = np.random.default_rng(15).choice([-1.0, 1.0], 64) if rotate else None
    for causal in (False, True):
        got_o, got_lse = of.fp8_attention_fwd(q, k, v, causal=causal, signs=s, kv_len=[260, 201])
        ref_o, ref_lse = oracle.attention_fwd(q, k, v, causal=causal, kv_len=[260, 201])
        err = np.linalg.norm(got_o - ref_o) / np.linalg.norm(ref_o)
        assert 1e-4 < err < 2.0 ** -3
        # logsumexp is 1-Lipschitz in the scores: |dLSE_i| <= max_j |dS_ij|
        # + ln(1 + 2^-4) (the rounding of P inside the sum). Every encoded
        # entry x (of Q H and K H, or Q and K) is within 2^-4 |x| + 2^-10 s
        # of its value (s its block scale), which bounds dS_ij.
        rot = np.eye(64) if s is None else of.rotation(s) / 8.0
        for b in range(2):
            for h in range(4):
                qr, kr = q[b, h] @ rot, k[b, h // 2] @ rot
                _, qs_ = of.quantize(q[b:b + 1, h:h + 1], s)
                _, ks_ = of.quantize(k[b:b + 1, h // 2:h // 2 + 1], s)
                rows = np.arange(260) // 128
                eq = 2.0 ** -4 * np.abs(qr) + 2.0 ** -10 * qs_[0, 0][rows][:, None]
                ek = 2.0 ** -4 * np.abs(kr) + 2.0 ** -10 * ks_[0, 0][rows][:, None]
                ds = (eq @ np.abs(kr).T + np.abs(qr) @ ek.T + eq @ ek.T) / 8.0
                vis = oracle.visible_mask(260, causal, [260, 201][b])
                bound = np.where(vis, ds, 0.0).max(axis=1) + math.log1p(2.0 ** -4) + 1e-9
                assert np.all(np.abs(got_lse[b, h] - ref_lse[b, h]) <= bound)


def test_padded_keys_do_not_matter():
    """Hidden keys enter only through their block's scale: new values of the
    same magnitudes (here, the negated ones) leave the result unchanged."""
    q, k, v = _inputs(16, n=300, d=64)
    a = of.fp8_attention_fwd(q, k, v, causal=False, kv_len=[230])
    k2, v2 = k.copy(), v.copy()
    k2[..., 230:, :] *= -1.0
    v2[..., 230:, :] *= -1.0
    b = of.fp8_attention_fwd(q, k2, v2, causal=False, kv_len=[230])
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # ... whereas a larger hidden value changes the block's scale.
    k2[0, 0, 240, 0] = 1e3  # hidden, but in the block of visible keys 128..229
    c = of.fp8_attention_fwd(q, k2, v2, causal=False, kv_len=[230])
    assert not np.array_equal(a[0], c[0])


def test_row_subsets_are_the_same_rows():
    """Each output row depends on its own query row and the keys only, so the
    rows= evaluation is the same definition on fewer rows."""
    q, k, v = _inputs(20, n=400, d=64)
    qc, qs = of.quantize(q)
    kc, ks = of.quantize(k)
    vc, vs = of.quantize(v)
    full = _head(qc, qs, kc, ks, vc, vs, 400, 0.2, True, 350)
    rows = np.array([0, 1, 127, 128, 255, 399])
    part = of.fp8_head_forward(qc[0, 0], qs[0, 0], kc[0, 0], ks[0, 0], vc[0, 0], vs[0, 0], 400,
                               0.2, True, 350, parts=True, rows=rows)
    np.testing.assert_array_equal(part["o"], full["o"][rows])
    np.testing.assert_array_equal(part["lse"], full["lse"][rows])
    np.testing.assert_array_equal(part["u"], full["u"][rows])


def test_grouped_heads_use_their_kv_head():
    q, k, v = _inputs(18, b=1, h=4, n=140, d=64, hkv=2)
    full = of.fp8_attention_fwd(q, k, v, causal=True)
    for h in range(4):
        one = of.fp8_attention_fwd(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1],
                                   causal=True)
        np.testing.assert_array_equal(full[0][:, h], one[0][:, 0])
    with pytest.raises(ValueError):
        of.fp8_attention_fwd(q[:, :3], k, v)


def test_empty_rows_and_negative_scale():
    q, k, v = _inputs(19, n=130, d=64)
    o, lse = of.fp8_attention_fwd(q, k, v, kv_len=[0])
    assert np.all(o == 0) and np.all(lse == -np.inf)
    # A negative scale is the same as negating Q (exact in E4M3).
    a = of.fp8_attention_fwd(q, k, v, scale=-0.125)
    b = of.fp8_attention_fwd(-q, k, v, scale=0.125)
    np.testing.assert_array_equal(a[0], b[0])


# --------------------------------------------------------------------------
# Planted mistakes
# --------------------------------------------------------------------------

def _runs_clean(tests):
    for t in tests:
        try:
            t()
        except AssertionError:
            return False
    return True


def test_fp8_planted_mistakes_are_rejected(monkeypatch):
    pins = [test_two_key_groups_closed_form,
            lambda: test_close_to_exact_attention(True),
            lambda: test_close_to_exact_attention(False),
            test_quantize_blocks_and_bounds,
            test_rotated_quantize_represents_x_times_h,
            test_rotation_keeps_scores,
            lambda: test_tiled_online_forward_agrees(True, None),
            test_lse_is_near_logsumexp_of_quantised_scores,
            test_constant_values_give_exactly_that_value,
            test_e4m3_round_matches_library_cast]
    assert _runs_clean(pins)
    good_round, good_exp = of.e4m3_round, of.block_exponent
    good_frame, good_rot, good_deq = of._frame, of.rotation, of.dequantize
    good_sum = of._row_sum
    mistakes = {
        "P not rounded": ("_quantize_p", lambda u: u),
        "row sum of the unrounded u": ("_row_sum", lambda u, pq: u.sum(axis=1)),
        "floor frame (u up to 512 saturates)": ("_frame", np.floor),
        "frame one too low": ("_frame", lambda t: good_frame(t) - 1),
        "block exponent one too high": ("block_exponent", lambda a: good_exp(a) + 1),
        "block exponent one too low": ("block_exponent", lambda a: good_exp(a) - 1),
        "ties away from zero": ("e4m3_round", lambda x: np.copysign(
            np.minimum(np.floor(np.abs(np.asarray(x, float)) / np.ldexp(1.0, np.maximum(
                np.frexp(np.abs(np.asarray(x, float)))[1] - 1, -6) - 3) + 0.5) * np.ldexp(
                1.0, np.maximum(np.frexp(np.abs(np.asarray(x, float)))[1] - 1, -6) - 3), 448.0), x)),
        "rotation without signs": ("rotation", lambda s: of.hadamard(np.asarray(s).size)),
        "scales ignored": ("dequantize", lambda c, s, n: of.e4m3_decode(np.asarray(c)[:n])),
        "block scale of the wrong block": ("dequantize", lambda c, s, n: of.e4m3_decode(
            np.asarray(c)[:n]) * np.asarray(s, float)[::-1][np.arange(n) // 128][:, None]),
    }
    for name, (attr, fn) in mistakes.items():
        monkeypatch.setattr(of, attr, fn)
        assert not _runs_clean(pins), name
        monkeypatch.setattr(of, "_quantize_p", lambda u: good_round(u))
        monkeypatch.setattr(of, "_frame", good_frame)
        monkeypatch.setattr(of, "block_exponent", good_exp)
        monkeypatch.setattr(of, "e4m3_round", good_round)
        monkeypatch.setattr(of, "rotation", good_rot)
        monkeypatch.setattr(of, "dequantize", good_deq)
        monkeypatch.setattr(of, "_row_sum", good_sum)
    assert _runs_clean(pins)
