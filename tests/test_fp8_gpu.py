"""GPU parity of the FP8 (E4M3) forward (page 2, "4. FlashAttention 深度剖析",
4.5.4), through the C ABI.

Primary gate -- exact attention on the operands the kernel sees. The codes
the GPU encoder wrote are read back and decoded with torch's own E4M3 type
(float8_e4m3fn), multiplied by their block scales, and the plain fp64
definition of attention (oracle.head_forward, the same oracle as the bf16
path) runs on those dequantised (and, with the Hadamard rotation, rotated)
Q, K, V. The GPU output must lie within a bound derived only from what the
page fixes for the FP8 forward:

* The probabilities enter the P V product as E4M3 values, so each weight
  carries at most half an E4M3 step of error: 2^-4 relative in the normal
  range. The weights of a row are scaled so that its largest lies in the
  top binade below the format's maximum, (128, 256]; weights that end up
  below the smallest normal (2^-6) are off by at most half a subnormal
  step, 2^-10, doubled here to 2^-9 because the kernel's own rounded
  maximum may put the row's scaling one binade higher.
* The products accumulate in fp32 (page 2 4.5.4) on the matrix cores,
  which sum E4M3 products with a truncation of up to 2^-12.5 of the summed
  magnitudes (measured; bound here by EPS_MMA = 2^-10): a score moves by
  at most EPS_MMA times its summed magnitudes, which scales its weight by
  at most ln 2 times that (plus 2^-20 for exp2 and fp32 rounding); the row
  sum and the P V product move by EPS_MMA of their summed magnitudes.
* O is rounded to bf16 (2^-9 relative; 2^-8 allowed).

With u_j the exact weights in that scaling, delta_j their allowance,
numerator error a_c and row-sum error b:
    |O_gpu - O|_c <= (sum_j delta_j |v_jc - O_c| + a_c + |O_c| b) / (sum_j u_j - b')
    |LSE_gpu - LSE| <= -ln(1 - b' / sum_j u_j)
(b' = sum_j delta_j + b). The LSE bound is at most ln(1 + 2^-4)-ish when
every weight of a row rounds the same way by a full half step; typical
errors are far smaller and are printed.

Diagnostic -- the kernel against a model of its own arithmetic
(oracle/fp8.py: probabilities rounded in an integer row frame, row sums of
the rounded values). With identical codes on both sides the GPU must follow
that model up to the neighbouring-code roundings its fp32 scores allow:
* Quantiser: codes and scales of fa_fp8_quantize equal the oracle's bit for
  bit without a rotation (the scaling is exact and both round to nearest
  even); with the Hadamard rotation (fp32 butterflies on the GPU, fp64 in
  the oracle) a code may differ only by one step, and only where the
  oracle's exact value lies within fp32 rounding of a rounding boundary.
* Forward on identical codes: element by element, within the envelope
  below, and normwise within 1e-2 (the bf16 path's bar for O).

Envelope of the model check. With the same EPS_MMA, a score's base-2 value
t deviates by at most dt = eps * sum_k |q^_k k^_k| * c + 2^-22 |t|, and a
probability u = 2^(t - f + 8) by a relative delta = ln 2 * dt + 2^-20.
Where E4M3(u (1 - delta)) != E4M3(u (1 + delta)) the GPU may legitimately
round u to the neighbouring code: that element may move O_i by the code
step times |v_j| / l_i. Probabilities below 2^-5 of the row frame may be
rounded in a finer running frame (or the frame itself may differ by one):
at most 2^-9 each. The row sum l is the sum of the same rounded values
(taken on the matrix cores): it moves by those steps and by eps * l, and the
O product by eps * sum_j P^_ij |v_j|; with numerator error a and row-sum
error b, |dO_i| <= (a + |O_i| b) / (l_i - b). On top: the bf16 rounding of
O (2^-9 relative; 2^-8 is allowed) and 1e-5 absolute.
"""

import math

import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd import attention as fa
from exact_io_aware_fa_amd import binding as B
from exact_io_aware_fa_amd.inputs import WORKLOADS, custom, make_inputs
from oracle import fp8 as of

pytestmark = pytest.mark.gpu

EPS_MMA = 2.0 ** -10
NORMWISE_TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _signs(d, seed):
    return np.random.default_rng(seed).choice([-1, 1], d).astype(np.int8)


def _oracle_codes(x, signs=None):
    """Oracle codes [B, H, np, d] (uint8) and fp32 scales of a bf16 CPU tensor."""
    codes, scales = of.quantize(x.float().numpy().astype(np.float64),
                                None if signs is None else signs.astype(np.float64))
    return codes, scales.astype(np.float32)


def _vt(codes):
    """Rows layout [B, H, np, d] -> V layout [B, H, nb, d, 128]."""
    b, h, np_, d = codes.shape
    return np.ascontiguousarray(codes.reshape(b, h, np_ // 128, 128, d).transpose(0, 1, 2, 4, 3))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _allowance(parts):
    """Per-element bound on |O_gpu - O_oracle| beyond bf16 rounding (see the
    module docstring): the numerator's error over l, and the row sum's
    relative error."""
    vis, u, l, vv = parts["vis"], parts["u"], parts["l"], parts["vv"]
    t = np.where(vis, parts["t"], 0.0)
    dt = EPS_MMA * parts["tabs"] + 2.0 ** -22 * np.abs(t)
    delta = math.log(2.0) * dt + 2.0 ** -20
    lo = of.e4m3_round(u * (1 - delta))
    hi = of.e4m3_round(u * (1 + delta))
    band = np.where(vis, hi - lo, 0.0) + np.where(vis & (u < 2.0 ** -5), 2.0 ** -9, 0.0)
    has = l > 0
    ls = np.where(has, l, 1.0)
    av = np.abs(vv)
    num = (band @ av + EPS_MMA * (parts["pq"] @ av)) / ls[:, None]
    l_rel = np.where(has, band.sum(axis=1) / ls + EPS_MMA, 0.0)
    return num, l_rel


def _check_head(o_gpu, lse_gpu, qc, qs, kc, ks, vc, vs, n, scale, causal, kvb, rows=None):
    r = of.fp8_head_forward(qc, qs.astype(np.float64), kc, ks.astype(np.float64), vc,
                            vs.astype(np.float64), n, scale, causal, kvb, parts=True, rows=rows)
    num, l_rel = _allowance(r)
    ref = r["o"]
    got = o_gpu.astype(np.float64)
    lr = np.minimum(l_rel, 0.5)[:, None]
    tol = 2.0 ** -8 * np.abs(ref) + (num + np.abs(ref) * lr) / (1 - lr) + 1e-5
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} elements out of tolerance; worst excess "
                           f"{(err - tol).max():.3g} at {np.unravel_index((err - tol).argmax(), err.shape)}")
    lref = r["lse"]
    fin = np.isfinite(lref)
    assert np.array_equal(np.isfinite(lse_gpu), fin)
    ltol = l_rel + 2.0 ** -21 * np.abs(np.where(fin, lref, 0.0)) + 1e-6
    assert np.all(np.abs(lse_gpu[fin] - lref[fin]) <= ltol[fin])
    nw = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    lmax = float(np.abs(lse_gpu[fin] - lref[fin]).max()) if fin.any() else 0.0
    print(f"[fp8] normwise O err {nw:.3e}, max LSE err {lmax:.3e}, "
          f"median tol/|o| {np.median(tol / np.maximum(np.abs(ref), 1e-30)):.3e}", flush=True)
    assert nw <= NORMWISE_TOL, nw
    return nw


# --------------------------------------------------------------------------
# Primary gate: exact attention on the dequantised operands
# --------------------------------------------------------------------------

LOG2E = 1.0 / math.log(2.0)
SUB_ABS = 2.0 ** -9       # subnormal weights: half a step, x2 for a frame one higher
HALF_STEP_REL = 2.0 ** -4  # normal weights: half an E4M3 step (3 mantissa bits)


def _decode(codes, scales):
    """scale * value of each code of one head: codes [np, d] (uint8, rows
    layout), scales [nb] -- decoded with torch's float8_e4m3fn type."""
    c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    vals = c.to(torch.float64).numpy()
    rows = np.arange(vals.shape[0]) // 128
    return vals * np.asarray(scales, dtype=np.float64)[rows][:, None]


def _gpu_codes(x, signs=None, layout="rows"):
    """GPU encoder output for a bf16 CPU tensor, read back to the host, in
    the rows layout [B, H, np, d] (V blocks transposed back)."""
    codes, scales = fa.fp8_quantize(x.cuda(), None if signs is None else _dev(signs),
                                    layout=layout)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    if layout == "vt":
        b, h, nb, d, blk = c.shape
        c = np.ascontiguousarray(c.transpose(0, 1, 2, 4, 3).reshape(b, h, nb * blk, d))
    return c, scales.cpu().numpy()


def _check_exact(o_gpu, lse_gpu, qd, kd, vd, scale, causal, kvb, rows=None):
    """O and LSE of one head (optionally only query ``rows``) against the
    fp64 definition of attention on dequantised operands qd, kd, vd [n, d],
    within the E4M3-derived bound of the module docstring."""
    import oracle
    from oracle.attention import visible_mask

    n = kd.shape[0]
    ref = oracle.head_forward(qd, kd, vd, scale, causal, kvb, rows=rows)
    qr = qd if rows is None else qd[np.asarray(rows, dtype=np.int64)]
    vis = visible_mask(n, causal, kvb, rows)
    t = np.where(vis, scale * (qr @ kd.T) * LOG2E, -np.inf)
    tmax = t.max(axis=1)
    has = np.isfinite(tmax)
    frame = np.where(has, np.ceil(np.where(has, tmax, 0.0)), 0.0)
    u = np.where(vis, np.exp2(t - frame[:, None] + 8.0), 0.0)   # row max in (128, 256]
    tabs = abs(scale) * LOG2E * (np.abs(qr) @ np.abs(kd).T)
    rho = math.log(2.0) * (EPS_MMA * tabs + 2.0 ** -22 * np.abs(np.where(vis, t, 0.0))) + 2.0 ** -20
    delta = np.where(vis, (HALF_STEP_REL * (1 + rho) + rho) * u + SUB_ABS, 0.0)
    lsum = u.sum(axis=1)
    pmax = u + delta
    o = ref["o"]
    av = np.abs(vd)
    # numerator: rounded weights, then the P V product's accumulation
    num = EPS_MMA * (pmax @ av)
    step = max(1, (1 << 23) // (n * vd.shape[1]))            # rows per chunk (64 MB)
    for r0 in range(0, o.shape[0], step):
        r1 = min(r0 + step, o.shape[0])
        dev = np.abs(vd[None, :, :] - o[r0:r1, None, :])
        num[r0:r1] += np.einsum("rj,rjc->rc", delta[r0:r1], dev)
    b_sum = EPS_MMA * pmax.sum(axis=1)                      # row-sum accumulation
    b_all = delta.sum(axis=1) + b_sum
    den = np.where(has, lsum - b_all, 1.0)
    assert np.all(den[has] > 0.5 * lsum[has])
    tol = (num + np.abs(o) * b_sum[:, None]) / den[:, None]
    tol = tol + 2.0 ** -8 * (np.abs(o) + tol) + 1e-6          # bf16 rounding of O
    got = o_gpu.astype(np.float64)
    err = np.abs(got - o)
    bad = (err > tol) & has[:, None]
    assert not bad.any(), (f"{bad.sum()} elements out of the E4M3 bound; worst excess "
                           f"{(err - tol).max():.3g}")
    assert np.all(got[~has] == 0.0)
    lref = ref["lse"]
    assert np.array_equal(np.isfinite(lse_gpu), has)
    ltol = -np.log1p(-np.where(has, b_all / np.where(has, lsum, 1.0), 0.0)) \
        + 2.0 ** -20 * np.abs(np.where(has, lref, 0.0)) + 1e-6
    lerr = np.abs(np.where(has, lse_gpu - lref, 0.0))
    assert np.all(lerr <= ltol), float((lerr - ltol).max())
    nw = float(np.linalg.norm(got - o) / max(np.linalg.norm(o), 1e-30))
    print(f"[fp8 exact] normwise O err {nw:.3e} (max elem {err.max():.3e}, median bound "
          f"{np.median(tol[has]):.3e}); LSE err max {lerr.max():.3e} mean "
          f"{lerr[has].mean() if has.any() else 0.0:.3e}, bound median "
          f"{np.median(ltol[has]) if has.any() else 0.0:.3e}", flush=True)
    return nw, float(lerr.max())


EXACT = [
    # (batch, heads, heads_kv, n, d, causal, padded, qk_sigma, scale, rotate)
    (2, 4, 2, 300, 128, True, False, 1.0, None, False),
    (2, 4, 2, 300, 128, False, True, 1.0, None, True),
    (1, 2, 2, 1000, 128, True, False, 3.0, None, True),    # peaky rows: the row max moves
    (1, 2, 1, 777, 128, False, False, 1.0, None, False),   # multi-query
    (2, 2, 2, 257, 128, True, True, 1.0, -0.07, False),    # negative scale
    (1, 2, 2, 200, 128, False, False, 1.0, 0.0, False),    # zero scale: uniform weights
    (1, 1, 1, 1, 128, True, False, 1.0, None, False),
    (2, 4, 2, 300, 64, True, True, 1.0, None, True),
    (1, 2, 1, 1000, 64, False, False, 3.0, None, False),   # peaky, multi-query
    (1, 2, 2, 129, 64, True, False, 1.0, -0.2, True),
    (2, 4, 2, 300, 256, True, True, 1.0, None, True),    # d = 256: 4-wave workgroups
    (1, 2, 1, 1000, 256, False, False, 3.0, None, False),
    (1, 2, 2, 129, 256, True, False, 1.0, -0.2, False),
    (1, 1, 1, 1, 256, True, False, 1.0, None, False),
]


@pytest.mark.parametrize("batch,heads,heads_kv,n,d,causal,padded,sigma,scale,rotate", EXACT)
def test_against_exact_attention_on_dequantised_operands(batch, heads, heads_kv, n, d, causal,
                                                         padded, sigma, scale, rotate):
    w = custom(f"fp8x_b{batch}_h{heads}_kv{heads_kv}_n{n}", batch, heads, n, d, "bf16", causal,
               seed=n * 17 + heads + d, qk_sigma=sigma, padded=padded, heads_kv=heads_kv)
    inp = make_inputs(w, with_grad_out=False)
    print(f"[fp8 exact] b={batch} h={heads} kv={heads_kv} n={n} d={d} causal={causal} "
          f"padded={padded} sigma={sigma} scale={scale} rotate={rotate}", flush=True)
    sc = w.softmax_scale if scale is None else scale
    signs = _signs(d, n) if rotate else None
    kvl = None if inp["kv_len"] is None else inp["kv_len"].cuda()
    o, lse = fa.flash_attn_fp8_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), causal,
                                   sc, kvl, None if signs is None else _dev(signs))
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    qc, qs = _gpu_codes(inp["q"], signs)
    kc, ks = _gpu_codes(inp["k"], signs)
    vc, vs = _gpu_codes(inp["v"], layout="vt")
    g = heads // heads_kv
    for b in range(batch):
        kvb = None if inp["kv_len"] is None else int(inp["kv_len"][b])
        for h in range(heads):
            j = h // g
            _check_exact(o[b, h], lse[b, h], _decode(qc[b, h], qs[b, h])[:n],
                         _decode(kc[b, j], ks[b, j])[:n], _decode(vc[b, j], vs[b, j])[:n], sc,
                         causal, kvb)


def test_exact_attention_full_size_sampled_rows():
    """The long causal size (B=1, H=32, N=16384, d=128, Q, K std 3) in the
    launch configuration the benchmark times: GPU encoder with the rotation,
    then the forward; sampled rows of four heads against exact attention on
    the decoded operands."""
    w = WORKLOADS["long_causal_b1_h32_n16384_d128"]
    n, heads = w.n, w.heads
    g = torch.Generator().manual_seed(w.seed)
    q = (torch.randn(1, 2, n, 128, generator=g) * w.qk_sigma).to(torch.bfloat16)
    k = (torch.randn(1, 2, n, 128, generator=g) * w.qk_sigma).to(torch.bfloat16)
    v = torch.randn(1, 2, n, 128, generator=g).to(torch.bfloat16)
    rep = lambda t: t.repeat(1, heads // 2, 1, 1).contiguous()  # noqa: E731
    signs = _signs(128, 44)
    print(f"[fp8 exact] full size n={n} heads={heads}", flush=True)
    o, lse = fa.flash_attn_fp8_fwd(rep(q).cuda(), rep(k).cuda(), rep(v).cuda(), True,
                                   w.softmax_scale, None, _dev(signs))
    torch.cuda.synchronize()
    qc, qs = _gpu_codes(q, signs)
    kc, ks = _gpu_codes(k, signs)
    vc, vs = _gpu_codes(v, layout="vt")
    rows = np.unique(np.concatenate([np.arange(0, 24), np.random.default_rng(8).integers(0, n, 40),
                                     np.arange(n - 24, n)]))
    ridx = torch.from_numpy(rows).cuda()
    for h in (0, 1, heads - 2, heads - 1):
        hs = h % 2
        og = o[0, h, ridx].float().cpu().numpy()
        lg = lse[0, h, ridx].cpu().numpy()
        _check_exact(og, lg, _decode(qc[0, hs], qs[0, hs])[:n], _decode(kc[0, hs], ks[0, hs])[:n],
                     _decode(vc[0, hs], vs[0, hs])[:n], w.softmax_scale, True, None, rows=rows)


# --------------------------------------------------------------------------
# Quantiser
# --------------------------------------------------------------------------

QUANT = [
    # (batch, heads, n, d, layout, rotate)
    (2, 3, 300, 128, "rows", False),
    (2, 3, 300, 128, "vt", False),
    (1, 2, 1000, 64, "rows", False),
    (1, 2, 1000, 64, "vt", False),
    (2, 2, 257, 128, "rows", True),
    (1, 3, 129, 64, "rows", True),
    (1, 1, 1, 128, "rows", False),
    (1, 1, 1, 128, "vt", False),
    (2, 2, 300, 256, "rows", False),
    (2, 2, 300, 256, "vt", False),
    (1, 2, 257, 256, "rows", True),
]


@pytest.mark.parametrize("batch,heads,n,d,layout,rotate", QUANT)
def test_quantize_matches_oracle(batch, heads, n, d, layout, rotate):
    print(f"[fp8] quantize b={batch} h={heads} n={n} d={d} {layout} rot={rotate}", flush=True)
    g = torch.Generator().manual_seed(n * 7 + d)
    x = (torch.randn(batch, heads, n, d, generator=g) * 2.0).to(torch.bfloat16)
    x[0, 0, :min(n, 128)] *= 1e-3  # a block with its own, much smaller scale
    signs = _signs(d, n) if rotate else None
    codes, scales = fa.fp8_quantize(x.cuda(), None if signs is None else _dev(signs),
                                    layout=layout)
    torch.cuda.synchronize()
    ref_c, ref_s = _oracle_codes(x, signs)
    if layout == "vt":
        ref_c = _vt(ref_c)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert got_c.shape == ref_c.shape and got_s.shape == ref_s.shape
    if not rotate:
        np.testing.assert_array_equal(got_s, ref_s)
        np.testing.assert_array_equal(got_c, ref_c)
        return
    np.testing.assert_array_equal(got_s, ref_s)
    diff = got_c != ref_c
    if diff.any():
        # Only adjacent codes, and only where the exact value sits within
        # fp32 rounding (2^-20 relative) of the boundary between them.
        xr = x.float().numpy().astype(np.float64) @ of.rotation(signs.astype(np.float64))
        blk = np.arange(ref_c.shape[2]) // 128
        e = np.round(np.log2(ref_s.astype(np.float64) * math.sqrt(d)))
        scaled = np.zeros(ref_c.shape)
        scaled[:, :, :n] = xr / np.exp2(e[:, :, blk[:n]])[..., None]
        a, b = of.e4m3_decode(got_c[diff]), of.e4m3_decode(ref_c[diff])
        mid = (a + b) / 2
        assert np.all(np.abs(scaled[diff] - mid) <= 2.0 ** -20 * np.abs(mid))
        assert diff.mean() < 1e-4


# --------------------------------------------------------------------------
# Forward on the oracle's codes
# --------------------------------------------------------------------------

FWD = [
    # (batch, heads, heads_kv, n, causal, padded, qk_sigma, scale, d)
    (2, 4, 2, 300, True, False, 1.0, None, 128),
    (2, 4, 2, 300, False, True, 1.0, None, 128),
    (1, 2, 2, 1000, True, False, 3.0, None, 128),     # peaky rows: frames move
    (1, 2, 1, 1000, False, False, 1.0, None, 128),    # multi-query
    (2, 2, 2, 257, True, True, 1.0, -0.07, 128),      # negative scale
    (1, 2, 2, 200, False, False, 1.0, 0.0, 128),      # zero scale: uniform weights
    (1, 1, 1, 1, True, False, 1.0, None, 128),
    (1, 2, 2, 64, False, False, 1.0, None, 128),
    (1, 2, 2, 513, True, False, 2.0, None, 128),
    (2, 4, 2, 300, True, True, 1.0, None, 64),
    (1, 2, 1, 1000, False, False, 3.0, None, 64),     # peaky, multi-query
    (1, 2, 2, 129, True, False, 1.0, -0.2, 64),
    (1, 1, 1, 1, False, False, 1.0, None, 64),
    (2, 4, 2, 300, True, True, 1.0, None, 256),       # d = 256: 4-wave workgroups
    (1, 2, 1, 1000, False, False, 3.0, None, 256),
]


def _run_codes(q, k, v, n, causal, scale, kv_len, signs=None):
    qc, qs = _oracle_codes(q, signs)
    kc, ks = _oracle_codes(k, signs)
    vc, vs = _oracle_codes(v)
    o, lse = fa.flash_attn_fp8_fwd_codes(_dev(qc), _dev(qs), _dev(kc), _dev(ks), _dev(_vt(vc)),
                                         _dev(vs), n, causal, scale,
                                         None if kv_len is None else kv_len.cuda())
    torch.cuda.synchronize()
    return (qc, qs, kc, ks, vc, vs), o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("batch,heads,heads_kv,n,causal,padded,sigma,scale,d", FWD)
def test_forward_on_oracle_codes(batch, heads, heads_kv, n, causal, padded, sigma, scale, d):
    w = custom(f"fp8_b{batch}_h{heads}_kv{heads_kv}_n{n}", batch, heads, n, d, "bf16", causal,
               seed=n * 13 + heads + d, qk_sigma=sigma, padded=padded, heads_kv=heads_kv)
    inp = make_inputs(w, with_grad_out=False)
    print(f"[fp8] forward b={batch} h={heads} kv={heads_kv} n={n} d={d} causal={causal} "
          f"padded={padded} sigma={sigma} scale={scale}", flush=True)
    sc = w.softmax_scale if scale is None else scale
    (qc, qs, kc, ks, vc, vs), o, lse = _run_codes(inp["q"], inp["k"], inp["v"], n, causal, sc,
                                                  inp["kv_len"])
    g = heads // heads_kv
    for b in range(batch):
        kvb = None if inp["kv_len"] is None else int(inp["kv_len"][b])
        for h in range(heads):
            _check_head(o[b, h], lse[b, h], qc[b, h], qs[b, h], kc[b, h // g], ks[b, h // g],
                        vc[b, h // g], vs[b, h // g], n, sc, causal, kvb)


def test_rotated_codes_forward():
    w = custom("fp8_rot", 1, 4, 700, 128, "bf16", True, seed=77, qk_sigma=2.0, heads_kv=2)
    inp = make_inputs(w, with_grad_out=False)
    signs = _signs(128, 5)
    (qc, qs, kc, ks, vc, vs), o, lse = _run_codes(inp["q"], inp["k"], inp["v"], 700, True,
                                                  w.softmax_scale, None, signs)
    for h in range(4):
        _check_head(o[0, h], lse[0, h], qc[0, h], qs[0, h], kc[0, h // 2], ks[0, h // 2],
                    vc[0, h // 2], vs[0, h // 2], 700, w.softmax_scale, True, None)


# --------------------------------------------------------------------------
# The whole recipe
# --------------------------------------------------------------------------

@pytest.mark.parametrize("rotate,d", [(False, 128), (True, 128), (False, 64), (True, 64),
                                      (True, 256)])
def test_end_to_end_against_oracle(rotate, d):
    """The whole recipe (GPU encoder, then the forward): against exact
    attention on the decoded operands (the primary gate), and against the
    model of the kernel's arithmetic run on the GPU encoder's own codes
    (with a rotation these may differ from the oracle encoder's by one step
    in rare elements, which the quantiser test bounds)."""
    w = custom("fp8_e2e", 2, 4, 600, d, "bf16", True, seed=91 + d, padded=True, heads_kv=2)
    inp = make_inputs(w, with_grad_out=False)
    signs = _signs(d, 9) if rotate else None
    print(f"[fp8] end to end rotate={rotate} d={d}", flush=True)
    o, lse = fa.flash_attn_fp8_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), True,
                                   kv_len=inp["kv_len"].cuda(),
                                   signs=None if signs is None else _dev(signs))
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    qc, qs = _gpu_codes(inp["q"], signs)
    kc, ks = _gpu_codes(inp["k"], signs)
    vc, vs = _gpu_codes(inp["v"], layout="vt")
    for b in range(2):
        kvb = int(inp["kv_len"][b])
        for h in range(4):
            j = h // 2
            _check_exact(o[b, h], lse[b, h], _decode(qc[b, h], qs[b, h])[:600],
                         _decode(kc[b, j], ks[b, j])[:600], _decode(vc[b, j], vs[b, j])[:600],
                         w.softmax_scale, True, kvb)
            _check_head(o[b, h], lse[b, h], qc[b, h], qs[b, h], kc[b, j], ks[b, j], vc[b, j],
                        vs[b, j], 600, w.softmax_scale, True, kvb)


# --------------------------------------------------------------------------
# Full size, sampled rows
# --------------------------------------------------------------------------

def test_full_size_sampled_rows():
    w = WORKLOADS["long_causal_b1_h32_n16384_d128"]
    n, heads = w.n, w.heads
    g = torch.Generator().manual_seed(w.seed)
    # Two heads' worth of inputs with the workload's distribution; every
    # head h of the call gets head h % 2's values (heads are independent).
    q = (torch.randn(1, 2, n, 128, generator=g) * w.qk_sigma).to(torch.bfloat16)
    k = (torch.randn(1, 2, n, 128, generator=g) * w.qk_sigma).to(torch.bfloat16)
    v = torch.randn(1, 2, n, 128, generator=g).to(torch.bfloat16)
    print(f"[fp8] full size n={n} heads={heads}", flush=True)
    qc, qs = _oracle_codes(q)
    kc, ks = _oracle_codes(k)
    vc, vs = _oracle_codes(v)
    rep = lambda a: np.ascontiguousarray(np.tile(a, (1, heads // 2) + (1,) * (a.ndim - 2)))  # noqa: E731
    o, lse = fa.flash_attn_fp8_fwd_codes(_dev(rep(qc)), _dev(rep(qs)), _dev(rep(kc)),
                                         _dev(rep(ks)), _dev(rep(_vt(vc))), _dev(rep(vs)), n,
                                         True, w.softmax_scale)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 40), np.random.default_rng(3).integers(0, n, 48),
                                     np.arange(n - 40, n)]))
    for h in (0, 1, heads - 2, heads - 1):
        hs = h % 2
        og = o[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy()
        lg = lse[0, h, torch.from_numpy(rows).cuda()].cpu().numpy()
        _check_head(og, lg, qc[0, hs], qs[0, hs], kc[0, hs], ks[0, hs], vc[0, hs], vs[0, hs], n,
                    w.softmax_scale, True, None, rows=rows)


def test_fp8_rejects_unsupported_head_dim():
    x = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="FA_E_UNSUPPORTED"):
        fa.fp8_quantize(x)
    q8 = torch.zeros(1, 1, 128, 96, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, 1, 1, device="cuda")
    v8 = torch.zeros(1, 1, 1, 96, 128, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="FA_E_UNSUPPORTED"):
        fa.flash_attn_fp8_fwd_codes(q8, s, q8, s, v8, s, 100)
    assert B.ABI_VERSION == B.fa_abi_version()
