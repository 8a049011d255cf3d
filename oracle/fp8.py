"""FP8 (E4M3) forward of attention: the recipe written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Two roles, kept apart:

* The format and the encoder (E4M3 rounding and decoding, block exponents,
  the Hadamard rotation, ``quantize``) are definitions: they follow the page
  and the format, and the GPU encoder must match them code for code.
* The forward on codes (``fp8_head_forward`` and the functions built on it)
  is a MODEL OF THE KERNEL'S ARITHMETIC, not the definition of what the FP8
  forward computes: the integer row frame and the row sum of the rounded
  probabilities below are the kernel's own design choices (readings the page
  leaves open). It serves as a secondary, tighter diagnostic. The parity
  gate of the FP8 forward is exact attention (``attention.head_forward``)
  on the dequantised operands, within a bound that follows from E4M3
  rounding of the probabilities alone (half an E4M3 step, 2^-4 relative,
  per weight) and fp32 accumulation.

Page 2 ("4. FlashAttention 深度剖析"), 4.5.4 (FP8 support), fixes the recipe:
the forward runs its products on E4M3 operands; every block is scaled once,
when it is loaded, and its scale factor is kept; the FP8 products accumulate
in FP32; a random Hadamard matrix H (entries +-1/sqrt(d), H H^T = I) may be
applied to Q and K, which leaves Q K^T unchanged while spreading outlier
values over all channels. Exercise 3 of the same page fixes the format's
range: largest magnitude 448, smallest normal 2^-6.

Readings (where the page is silent):

* E4M3 is the 1-4-3 format with exponent bias 7, subnormals below 2^-6 in
  steps of 2^-9, no infinities and S.1111.111 as NaN (the only E4M3 variant
  whose largest value is 448). Rounding is to nearest with ties to even; a
  magnitude past 448 saturates to 448 (the scales below never produce one).
* "Block" is a block of 128 consecutive rows of one head (the tile a
  kernel loads): Q per query block, K and V per key block. The page names
  the K blocks; Q and V get the same treatment.
* A block's scale is the power of two 2^e with e the smallest integer such
  that max |x| <= 448 * 2^e (e = 0 for an all-zero block). A power of two
  makes the scaling exact, so the only rounding is E4M3's own. The codes are
  E4M3(x / 2^e); the block is represented by scale * codes.
* The rotation is R = diag(s) H_d with the Sylvester Hadamard matrix H_d
  (entries +-1) and random signs s (an input): R / sqrt(d) is the page's
  random Hadamard matrix. Rotated blocks are scaled on x R, and the stored
  scale is 2^e / sqrt(d), so scale * codes approximates x R / sqrt(d) = x H.
* Both products of the forward use FP8 operands, so the probabilities are
  quantised too. With t = S log2(e) and the row frame f = ceil(max_j t_ij)
  (an integer), u_ij = 2^(t_ij - f + 8) lies in (0, 256] and the largest u
  of a row lies in (128, 256]; P^_ij = E4M3(u_ij). The frame is an integer
  so that a tiled kernel, whose running frames only differ from the final
  one by powers of two, rounds every normal-range u exactly as here, in any
  tile order. The factor 2^8 is the largest power of two that keeps u <= 448.
* The row sum is taken on the rounded probabilities: l_i = sum_j P^_ij, so
  O_i = sum_j P^_ij v^_j / l_i (v^ the dequantised V rows) is a convex
  combination of V rows whose weights sum to exactly 1, and
  LSE_i = ln 2 * (f_i - 8 + log2 l_i), the log-sum-exp of the quantised
  scores up to the rounding of the probabilities (a factor within
  1 +- 2^-4 inside the log).

Masks as in ``attention``: causal (j > i hidden) and key padding
(j >= kv_len[b] hidden); a row with no visible key gives O = 0,
LSE = -inf. Grouped K/V heads: query head h uses K/V head h // (H // H_kv).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import default_scale, visible_mask

E4M3_MAX = 448.0               # page 2 exercise 3: largest finite magnitude
E4M3_MIN_NORMAL = 2.0 ** -6    # page 2 exercise 3: smallest normal magnitude
E4M3_MIN_SUBNORMAL = 2.0 ** -9  # 3 mantissa bits below the smallest normal
BLOCK = 128                    # rows per scaling block
P_SHIFT = 8                    # probabilities are quantised as 2^8 * p


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------- E4M3 format

def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * E4M3_MIN_SUBNORMAL, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value (ties to even), saturating at +-448, as float64.

    In the binade [2^b, 2^(b+1)) (b >= -6) the values are spaced 2^(b-3);
    below 2^-6 the subnormals are spaced 2^-9, the same step as the lowest
    binade. Rounding a / step to the nearest integer with ties to even picks
    the even mantissa.
    """
    x = _f64(x)
    a = np.abs(x)
    _, ex = np.frexp(a)               # a in [2^(ex-1), 2^ex)
    b = np.maximum(ex - 1, -6)
    step = np.ldexp(1.0, b - 3)
    r = np.minimum(np.round(a / step) * step, E4M3_MAX)
    return np.copysign(r, x)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 byte of the rounded value (sign bit kept for zeros)."""
    x = _f64(x)
    r = np.abs(e4m3_round(x))
    _, ex = np.frexp(r)
    normal = r >= E4M3_MIN_NORMAL
    efield = np.where(normal, ex - 1 + 7, 0)
    mant = np.where(normal, r / np.ldexp(1.0, ex - 1) * 8.0 - 8.0, r / E4M3_MIN_SUBNORMAL)
    code = (efield.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code |= np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


# ------------------------------------------------------------- block scaling

def block_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (0 where amax == 0).

    With amax = m 2^E (m in [0.5, 1)) and 448 = 0.875 * 2^9: amax <= 448 * 2^e
    iff E <= e + 9 when m <= 0.875, iff E <= e + 8 otherwise.
    """
    a = _f64(amax)
    m, E = np.frexp(a)
    e = np.where(m <= 0.875, E - 9, E - 8)
    return np.where(a == 0, 0, e).astype(np.int64)


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1:
    H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(signs) -> np.ndarray:
    """R = diag(signs) H_d; R / sqrt(d) is page 2 4.5.4's random Hadamard matrix."""
    s = _f64(signs).reshape(-1)
    if not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be +1 or -1")
    return s[:, None] * hadamard(s.shape[0])


def quantize(x, signs=None) -> tuple[np.ndarray, np.ndarray]:
    """Blockwise E4M3 encoding of x [B, H, n, d] (optionally rotated).

    Returns codes [B, H, nb * 128, d] (uint8; rows past n are zero codes)
    and scales [B, H, nb] (float64) with x (or x H when rotated) ~= scale *
    decode(codes) row-block by row-block, nb = ceil(n / 128).
    """
    x = _f64(x)
    B, H, n, d = x.shape
    post = 1.0
    if signs is not None:
        x = x @ rotation(signs)
        post = 1.0 / math.sqrt(d)
    nb = (n + BLOCK - 1) // BLOCK
    codes = np.zeros((B, H, nb * BLOCK, d), dtype=np.uint8)
    scales = np.ones((B, H, nb))
    for blk in range(nb):
        seg = x[:, :, blk * BLOCK:(blk + 1) * BLOCK, :]
        e = block_exponent(np.abs(seg).max(axis=(2, 3)))
        codes[:, :, blk * BLOCK:blk * BLOCK + seg.shape[2], :] = e4m3_encode(
            seg / np.ldexp(1.0, e)[:, :, None, None])
        scales[:, :, blk] = np.ldexp(1.0, e) * post
    return codes, scales


def dequantize(codes, scales, n: int) -> np.ndarray:
    """scale * decode(codes) for the first n rows of one head ([np, d], [nb])."""
    rows = np.arange(n)
    return e4m3_decode(np.asarray(codes)[:n]) * _f64(scales)[rows // BLOCK][:, None]


# ------------------------------------------------------------------- forward

def _frame(tmax: np.ndarray) -> np.ndarray:
    """Integer row frame: ceil of the row's largest t."""
    return np.ceil(tmax)


def _quantize_p(u: np.ndarray) -> np.ndarray:
    return e4m3_round(u)


def _row_sum(u: np.ndarray, pq: np.ndarray) -> np.ndarray:
    """l_i: the sum of the row's rounded probabilities."""
    return pq.sum(axis=1)


def fp8_head_forward(qc, qs, kc, ks, vc, vs, n: int, scale: float, causal: bool,
                     kv_len_b: int | None = None, parts: bool = False, rows=None) -> dict:
    """Forward of one head from codes and scales (see the module docstring).

    qc, kc, vc: [np, d] codes; qs, ks, vs: [nb] scales. ``rows`` selects
    query rows (each output row depends on its own query row and all keys
    only). Returns dict(o, lse) and, with ``parts``, the intermediate arrays
    (t, f, u, pq, l, vv, tabs, vis) a parity check needs.
    """
    q = dequantize(qc, qs, n)
    if rows is not None:
        q = q[np.asarray(rows, dtype=np.int64)]
    k = dequantize(kc, ks, n)
    vv = dequantize(vc, vs, n)
    vis = visible_mask(n, causal, kv_len_b, rows)
    log2e = 1.0 / math.log(2.0)
    t = np.where(vis, scale * (q @ k.T) * log2e, -np.inf)
    tmax = t.max(axis=1)
    has = np.isfinite(tmax)
    f = np.where(has, _frame(np.where(has, tmax, 0.0)), 0.0)
    u = np.where(vis, np.exp2(t - f[:, None] + P_SHIFT), 0.0)
    pq = _quantize_p(u)
    l = _row_sum(u, pq)
    has = has & (l > 0)
    l_safe = np.where(has, l, 1.0)
    o = np.where(has[:, None], (pq @ vv) / l_safe[:, None], 0.0)
    lse = np.where(has, (f - P_SHIFT + np.log2(l_safe)) * math.log(2.0), -np.inf)
    out = {"o": o, "lse": lse}
    if parts:
        tabs = abs(scale) * (np.abs(q) @ np.abs(k).T) * log2e
        out.update(t=t, f=f, u=u, pq=pq, l=l, vv=vv, tabs=tabs, vis=vis)
    return out


def fp8_attention_fwd_codes(qc, qs, kc, ks, vc, vs, n: int, causal: bool = False,
                            scale: float | None = None, kv_len=None) -> dict:
    """Forward from codes and scales for every (batch, head).

    qc [B, H, np, d], qs [B, H, nb]; kc, vc [B, H_kv, np, d], ks, vs
    [B, H_kv, nb] (row layout for all three). Returns (o [B, H, n, d],
    lse [B, H, n]), float64, natural log.
    """
    qc = np.asarray(qc)
    B, H, _, d = qc.shape
    hkv = np.asarray(kc).shape[1]
    if hkv < 1 or H % hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    g = H // hkv
    sc = default_scale(d) if scale is None else float(scale)
    o = np.zeros((B, H, n, d))
    lse = np.zeros((B, H, n))
    for b in range(B):
        kvb = None if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        for h in range(H):
            r = fp8_head_forward(qc[b, h], qs[b, h], kc[b, h // g], ks[b, h // g],
                                 vc[b, h // g], vs[b, h // g], n, sc, causal, kvb)
            o[b, h], lse[b, h] = r["o"], r["lse"]
    return o, lse


def fp8_attention_fwd(q, k, v, causal: bool = False, scale: float | None = None,
                      kv_len=None, signs=None) -> dict:
    """The whole recipe from unquantised inputs: quantise Q, K (rotated when
    ``signs`` is given) and V per block, then the forward above.
    Returns (o, lse) like ``fp8_attention_fwd_codes``."""
    n = np.asarray(q).shape[2]
    qc, qs = quantize(q, signs)
    kc, ks = quantize(k, signs)
    vc, vs = quantize(v)
    return fp8_attention_fwd_codes(qc, qs, kc, ks, vc, vs, n, causal, scale, kv_len)
