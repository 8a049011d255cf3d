"""GPU parity of the FP8 (E4M3) forward (page 2, "4. FlashAttention 深度剖析",
4.5.4) against the oracle in oracle/fp8.py, through the C ABI.

* Quantiser: codes and scales of fa_fp8_quantize equal the oracle's bit for
  bit without a rotation (the scaling is exact and both round to nearest
  even); with the Hadamard rotation (fp32 butterflies on the GPU, fp64 in
  the oracle) a code may differ only by one step, and only where the
  oracle's exact value lies within fp32 rounding of a rounding boundary.
* Forward on the oracle's own codes (so both sides see identical operands):
  element by element with a tolerance derived from the arithmetic, below.
* The whole recipe (GPU quantiser + forward) against the oracle's.
* The full long-sequence size (B=1, H=32, N=16384, d=128, causal) in the
  launch configuration the benchmark times, on sampled rows.

Tolerance of the forward. The matrix cores accumulate fp8 products in fp32
but not faithfully: a 64-term product was measured off by up to
2^-12.5 * sum |a_k b_k| on random E4M3 operands, so the bound used here is
eps = 2^-10 * sum |a_k b_k| (a 5x margin). A score's base-2 value t then
deviates by at most dt = eps * sum_k |q^_k k^_k| * c + 2^-22 |t|, and a
probability u = 2^(t - f + 8) by a relative delta = ln 2 * dt + 2^-20 (exp2
and fp32 rounding). Where E4M3(u (1 - delta)) != E4M3(u (1 + delta)) the
GPU may legitimately round u to the neighbouring code: that element may move
O_i by the code step times |v_j| / l_i. Probabilities below 2^-5 of the row
frame may be rounded in a finer running frame (or the frame itself may
differ by one): at most 2^-9 each. The row sum l is the sum of the same
rounded values (taken on the matrix cores): it moves by those steps and by
eps * l, and the O product by eps * sum_j P^_ij |v_j|; with numerator error
a and row-sum error b, |dO_i| <= (a + |O_i| b) / (l_i - b). On top: the
bf16 rounding of O (2^-9 relative; 2^-8 is allowed) and 1e-5 absolute.

That envelope holds for any accumulation order the hardware may use, so it
is wide (often a tenth of |O|). Each head must also meet a normwise bound,
|O_gpu - O_oracle| <= 1e-2 |O_oracle|, the bf16 path's bar for O: the bf16
rounding of O alone gives about 2e-3, and the neighbouring-code roundings
above are rare; a wrong key, block scale, frame or tile moves O by far more.
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

@pytest.mark.parametrize("rotate,d", [(False, 128), (True, 128), (False, 64), (True, 64)])
def test_end_to_end_against_oracle(rotate, d):
    w = custom("fp8_e2e", 2, 4, 600, d, "bf16", True, seed=91 + d, padded=True, heads_kv=2)
    inp = make_inputs(w, with_grad_out=False)
    signs = _signs(d, 9) if rotate else None
    print(f"[fp8] end to end rotate={rotate} d={d}", flush=True)
    o, lse = fa.flash_attn_fp8_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), True,
                                   kv_len=inp["kv_len"].cuda(),
                                   signs=None if signs is None else _dev(signs))
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    qc, qs = _oracle_codes(inp["q"], signs)
    kc, ks = _oracle_codes(inp["k"], signs)
    vc, vs = _oracle_codes(inp["v"])
    if not rotate:
        # Identical codes on both sides (the quantiser is exact here).
        for b in range(2):
            for h in range(4):
                _check_head(o[b, h], lse[b, h], qc[b, h], qs[b, h], kc[b, h // 2],
                            ks[b, h // 2], vc[b, h // 2], vs[b, h // 2], 600, w.softmax_scale,
                            True, int(inp["kv_len"][b]))
    ro, rl = of.fp8_attention_fwd(inp["q"].float().numpy(), inp["k"].float().numpy(),
                                  inp["v"].float().numpy(), causal=True,
                                  kv_len=inp["kv_len"].numpy(),
                                  signs=None if signs is None else signs.astype(np.float64))
    err = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    assert err < 4e-3, err
    # LSE: one neighbouring-code rounding of a row's dominant probability
    # moves it by at most ln(1 + 2^-4); such roundings are rare, so the mean
    # deviation stays small.
    dl = np.abs(lse - rl)
    assert dl.max() <= math.log1p(2.0 ** -4) and dl.mean() < 1e-3, (dl.max(), dl.mean())


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
    x = torch.zeros(1, 1, 64, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="FA_E_UNSUPPORTED"):
        fa.fp8_quantize(x)
    q8 = torch.zeros(1, 1, 128, 256, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, 1, 1, device="cuda")
    v8 = torch.zeros(1, 1, 1, 256, 128, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="FA_E_UNSUPPORTED"):
        fa.flash_attn_fp8_fwd_codes(q8, s, q8, s, v8, s, 100)
    assert B.ABI_VERSION == B.fa_abi_version()
