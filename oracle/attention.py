"""Plain fp64 attention: the definition written out, one (batch, head) at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed (all in float64, all N x N matrices materialised):

Forward -- page 1 section 五 (standard attention: S = Q K^T, P = softmax(S),
O = P V), with the 1/sqrt(d) scale that page 2 4.3.2 and page 4 下篇 3.3 write
into S; the scale is a parameter whose default is 1/sqrt(d):

    S_ij   = scale * <q_i, k_j>
    S_ij   = -inf  where key j is hidden from query i (mask below)
    m_i    = max_j S_ij                         (page 1 section 六, safe softmax)
    e_ij   = exp(S_ij - m_i), exactly 0.0 where hidden
    l_i    = sum_j e_ij
    P_ij   = e_ij / l_i
    O_i    = sum_j P_ij v_j
    LSE_i  = m_i + ln l_i                       (page 2 4.3.2, "L_i = m_i + log l_i")

Mask: key j is hidden from query i when (causal and j > i) -- the upper-right
triangle of page 3 第八部分 -- or when j >= kv_len[b] (key padding; the pages
only name an attention-mask argument, so the reading is: padded keys are hidden
from every query row, and every query row, padded or not, is computed).
A row with no visible key (impossible for kv_len >= 1 in these workloads) gives
O_i = 0, LSE_i = -inf and zero gradients.

Backward -- page 1 section 八 and page 2 4.3.4 say only that P is rebuilt from
the saved row statistics (P_ij = exp(S_ij - L_i)) and that dS, dQ, dK, dV are
computed; they print no gradient formula. The reading is ordinary calculus of
f = sum(O * dO) for softmax attention:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij
    dS = P * (dP - D 1^T)
    dQ = scale * dS K
    dK = scale * dS^T Q

Hidden entries have P = 0, hence dS = 0, so dK/dV rows of padded keys are 0.

Grouped K/V heads (GQA / MQA) -- page 1 section 九 notes that several query
heads may share one K/V head, and page 4 下篇 section 六 fixes only that the
query head count H is a multiple of the K/V head count H_kv. The reading
here: contiguous groups, query head h uses K/V head h // (H // H_kv). Each
query head is then plain attention against its K/V head, and because a
shared K/V head enters every query head of its group, its gradients are the
sums over the group:

    dK[g] = sum_{h in group g} dK_h,    dV[g] = sum_{h in group g} dV_h.

Sliding windows and block-sparse masks -- page 4 下篇 section 六 shows the
flash-attn call's ``window_size=(-1, -1)`` argument (full attention by
default, a sliding window otherwise) and page 2 4.8.1 names the sliding
window of Mistral; page 3 第八部分 describes block-sparse attention with a
coarse block-level mask matrix whose fully masked blocks are skipped. The
readings here: a window (left, right) keeps key j for query i iff
i - left <= j <= i + right, where -1 leaves that side unbounded (so causal
is the same as right = 0); a block mask is a boolean matrix over blocks of
BLOCK x BLOCK (query block i // BLOCK, key block j // BLOCK), BLOCK = 128,
and a key is visible only where its block is. Every mask combines with the
others by logical AND; a query row left with no visible key gets O = 0,
LSE = -inf and zero gradients (as above).

Packed variable-length batches -- page 2 4.7.2 and 4.7.4 list attention over
variable-length sequences without padding as a supported call, and 4.9.3
names the padding waste it avoids; none of them fixes a layout or a mask.
The reading here: the sequences of a batch are stored back to back, head by
head ([H, T, d] with T the total length), sequence s occupying rows
cu[s] .. cu[s+1]-1 of every head; each sequence is its own self-attention
problem -- its queries see only its own keys, and the causal triangle
counts positions from the sequence's first row -- so the whole batch is one
block-diagonal attention over the T rows.
"""

from __future__ import annotations

import math

import numpy as np


def default_scale(d: int) -> float:
    """1/sqrt(d), the default softmax scale (page 4 下篇 section 六, the
    ``softmax_scale=None`` argument of the flash-attn call)."""
    return 1.0 / math.sqrt(d)


BLOCK = 128  # side of a block of the block-sparse mask (rows and keys)


def visible_mask(n: int, causal: bool, kv_len_b: int | None = None,
                 rows=None, window=(-1, -1), block_mask=None) -> np.ndarray:
    """Boolean [len(rows), n]: True where key j is visible to query i.

    Causal hides j > i (page 3 第八部分, upper-right triangle); key padding
    hides j >= kv_len_b for every query row; a window (left, right) hides
    j < i - left (left >= 0) and j > i + right (right >= 0); a block mask
    hides j wherever block_mask[i // BLOCK][j // BLOCK] is false.
    """
    i = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(n)
    vis = np.ones((i.shape[0], n), dtype=bool)
    if kv_len_b is not None:
        vis &= (j[None, :] < int(kv_len_b))
    if causal:
        vis &= (j[None, :] <= i[:, None])
    left, right = int(window[0]), int(window[1])
    if left >= 0:
        vis &= (j[None, :] >= i[:, None] - left)
    if right >= 0:
        vis &= (j[None, :] <= i[:, None] + right)
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        vis &= bm[i[:, None] // BLOCK, j[None, :] // BLOCK]
    return vis


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def head_forward(q, k, v, scale: float, causal: bool,
                 kv_len_b: int | None = None, rows=None,
                 want_p: bool = False, window=(-1, -1), block_mask=None) -> dict:
    """Forward of one head. q, k, v: [n, d] (any real dtype, upcast exactly).

    ``rows`` selects query rows (each output row depends on its own query row
    and all keys only, so a subset is the same definition evaluated on fewer
    rows). Returns dict(o=[r, d], lse=[r], and p=[r, n] if ``want_p``).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = k.shape[0]
    qr = q if rows is None else q[np.asarray(rows, dtype=np.int64)]
    vis = visible_mask(n, causal, kv_len_b, rows, window, block_mask)

    s = scale * (qr @ k.T)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has_key = np.isfinite(m)
    m_ref = np.where(has_key, m, 0.0)
    e = np.where(vis, np.exp(s - m_ref[:, None]), 0.0)
    l = e.sum(axis=1)
    l_safe = np.where(has_key, l, 1.0)
    p = e / l_safe[:, None]
    o = p @ v
    lse = np.where(has_key, m_ref + np.log(l_safe), -np.inf)
    out = {"o": o, "lse": lse}
    if want_p:
        out["p"] = p
    return out


def head_backward(q, k, v, do, scale: float, causal: bool,
                  kv_len_b: int | None = None, window=(-1, -1), block_mask=None) -> dict:
    """Gradients of f = sum(O * dO) for one head; q, k, v, do: [n, d].

    Returns dict(dq, dk, dv, d=D vector, o, lse).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    fw = head_forward(q, k, v, scale, causal, kv_len_b, want_p=True, window=window,
                      block_mask=block_mask)
    p = fw.pop("p")
    dv = p.T @ do
    dp = do @ v.T
    dvec = (p * dp).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return {"dq": dq, "dk": dk, "dv": dv, "d": dvec,
            "o": fw["o"], "lse": fw["lse"]}


def _kv_len_of(kv_len, b: int):
    return None if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])


def _group(heads: int, heads_kv: int) -> int:
    if heads_kv < 1 or heads % heads_kv:
        raise ValueError(f"query heads {heads} not a multiple of K/V heads {heads_kv}")
    return heads // heads_kv


def attention_fwd(q, k, v, causal: bool = False, scale: float | None = None,
                  kv_len=None, window=(-1, -1), block_mask=None):
    """Forward over q [B, H, N, d] and k, v [B, H_kv, N, d] (H_kv divides H;
    H_kv = H is ordinary multi-head attention), one query head at a time;
    query head h uses K/V head h // (H // H_kv).

    Returns (o [B,H,N,d] float64, lse [B,H,N] float64, natural log).
    """
    q = _f64(q)
    bsz, heads, n, d = q.shape
    grp = _group(heads, np.shape(k)[1])
    scale = default_scale(d) if scale is None else float(scale)
    o = np.empty_like(q)
    lse = np.empty((bsz, heads, n))
    for b in range(bsz):
        kvl = _kv_len_of(kv_len, b)
        for h in range(heads):
            r = head_forward(q[b, h], k[b, h // grp], v[b, h // grp], scale, causal, kvl,
                             window=window, block_mask=block_mask)
            o[b, h] = r["o"]
            lse[b, h] = r["lse"]
    return o, lse


def attention_bwd(q, k, v, do, causal: bool = False,
                  scale: float | None = None, kv_len=None, window=(-1, -1), block_mask=None):
    """Backward over q, do [B, H, N, d] and k, v [B, H_kv, N, d], one query
    head at a time; dK and dV of a shared K/V head are summed over its group.

    Returns (dq [B,H,N,d], dk [B,H_kv,N,d], dv [B,H_kv,N,d]), float64.
    """
    q = _f64(q)
    bsz, heads, n, d = q.shape
    heads_kv = np.shape(k)[1]
    grp = _group(heads, heads_kv)
    scale = default_scale(d) if scale is None else float(scale)
    dq = np.empty_like(q)
    dk = np.zeros((bsz, heads_kv, n, d))
    dv = np.zeros((bsz, heads_kv, n, d))
    for b in range(bsz):
        kvl = _kv_len_of(kv_len, b)
        for h in range(heads):
            r = head_backward(q[b, h], k[b, h // grp], v[b, h // grp], do[b, h], scale,
                              causal, kvl, window, block_mask)
            dq[b, h] = r["dq"]
            dk[b, h // grp] += r["dk"]
            dv[b, h // grp] += r["dv"]
    return dq, dk, dv


def _spans(cu_seqlens):
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if len(cu) < 2 or cu[0] != 0 or any(b < a for a, b in zip(cu[:-1], cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return list(zip(cu[:-1], cu[1:]))


def varlen_fwd(q, k, v, cu_seqlens, causal: bool = False, scale: float | None = None,
               window=(-1, -1), block_mask=None):
    """Forward over a packed variable-length batch: q [H, T, d], k, v
    [H_kv, T, d]; sequence s is rows cu_seqlens[s] .. cu_seqlens[s+1]-1 of
    every head, attended to on its own (causal positions counted from its
    first row); query head h uses K/V head h // (H // H_kv).

    Returns (o [H, T, d], lse [H, T]) float64; rows past cu_seqlens[-1] stay
    0 and -inf.
    """
    q = _f64(q)
    heads, total, d = q.shape
    grp = _group(heads, np.shape(k)[0])
    scale = default_scale(d) if scale is None else float(scale)
    o = np.zeros_like(q)
    lse = np.full((heads, total), -np.inf)
    for a, e in _spans(cu_seqlens):
        if e == a:
            continue
        for h in range(heads):
            r = head_forward(q[h, a:e], k[h // grp, a:e], v[h // grp, a:e], scale, causal,
                             window=window, block_mask=block_mask)
            o[h, a:e] = r["o"]
            lse[h, a:e] = r["lse"]
    return o, lse


def varlen_bwd(q, k, v, do, cu_seqlens, causal: bool = False,
               scale: float | None = None, window=(-1, -1), block_mask=None):
    """Backward of ``varlen_fwd`` (gradients of sum(O * dO)); dK and dV of a
    shared K/V head are summed over its group. Returns (dq [H,T,d],
    dk [H_kv,T,d], dv [H_kv,T,d]) float64; rows outside every sequence are 0.
    """
    q = _f64(q)
    heads, total, d = q.shape
    heads_kv = np.shape(k)[0]
    grp = _group(heads, heads_kv)
    scale = default_scale(d) if scale is None else float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros((heads_kv, total, d))
    dv = np.zeros((heads_kv, total, d))
    for a, e in _spans(cu_seqlens):
        if e == a:
            continue
        for h in range(heads):
            r = head_backward(q[h, a:e], k[h // grp, a:e], v[h // grp, a:e], do[h, a:e],
                              scale, causal, None, window, block_mask)
            dq[h, a:e] = r["dq"]
            dk[h // grp, a:e] += r["dk"]
            dv[h // grp, a:e] += r["dv"]
    return dq, dk, dv
