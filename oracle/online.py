"""The pages' online-softmax algebra, in their order and notation (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

These are slow, plain-Python/NumPy restatements used to pin the oracle:

* ``softmax_three_pass``        page 2, 4.2.1: m = max x, d = sum e^(x-m),
                                y = e^(x-m)/d (three sweeps).
* ``normalizer_two_pass``       page 2, 4.2.2: the running (m, d) pair,
                                d^(i) = d^(i-1) e^(m^(i-1)-m^(i)) + e^(x_i-m^(i)).
* ``softmax_matmul_one_pass``   page 2, 4.2.3: the running (m, l, O~) triple,
                                O = O~/l at the end.
* ``block_state`` / ``merge``   page 2, 4.2.4: the (m, l, O~) state of a block
                                and the associative merge of two states.
* ``block_update``              page 1, section 六: the per-block update of
                                (m, l, O) for a block of rows, then
                                ``finalize`` O = diag(l)^-1 O.
* ``tiled_forward``             page 2, 4.3.2: Q-outer / KV-inner loops over
                                B_r x B_c tiles with deferred normalisation and
                                the stored L = m + log l; causal tiles with no
                                visible key are skipped.

The empty state is (m=-inf, l=0, O~=0). Rescaling a state whose m is -inf
yields 0 rather than exp(-inf - -inf) = NaN: that state holds nothing, so
any factor leaves it empty; this is the identity of the merge.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def _rescale(m_old, m_new):
    """exp(m_old - m_new), with 0 for an empty (m_old = -inf) state."""
    m_old = np.asarray(m_old, dtype=np.float64)
    m_new = np.asarray(m_new, dtype=np.float64)
    finite = np.isfinite(m_old)
    diff = np.where(finite, m_old - np.where(np.isfinite(m_new), m_new, 0.0), 0.0)
    return np.where(finite, np.exp(diff), 0.0)


def softmax_three_pass(x) -> np.ndarray:
    """Safe softmax of a vector in three sweeps (page 2, 4.2.1)."""
    x = [float(t) for t in x]
    m = NEG_INF
    for t in x:                       # sweep 1: the maximum
        m = max(m, t)
    d = 0.0
    for t in x:                       # sweep 2: the normaliser
        d += math.exp(t - m)
    return np.array([math.exp(t - m) / d for t in x])  # sweep 3


def normalizer_two_pass(x):
    """Running (m, d) over the vector in one sweep (page 2, 4.2.2).

    Returns (m, d, history) where history[i] = (m^(i), d^(i)) after element i.
    The second sweep (y_j = e^(x_j - m)/d) is ``normalised(x, m, d)``.
    """
    m, d = NEG_INF, 0.0
    history = []
    for t in x:
        t = float(t)
        m_new = max(m, t)
        d = d * (math.exp(m - m_new) if m != NEG_INF else 0.0) + math.exp(t - m_new)
        m = m_new
        history.append((m, d))
    return m, d, history


def normalised(x, m: float, d: float) -> np.ndarray:
    """Second sweep of the two-pass form: y_j = e^(x_j - m) / d."""
    return np.array([math.exp(float(t) - m) / d for t in x])


def softmax_matmul_one_pass(x, v):
    """One sweep of the (m, l, O~) recurrence of page 2, 4.2.3.

    x: [n] scores, v: [n, d] values. Returns (m, l, O~); O = O~ / l.
    """
    v = np.asarray(v, dtype=np.float64)
    m, l = NEG_INF, 0.0
    o = np.zeros(v.shape[1])
    for t, vi in zip(x, v):
        t = float(t)
        m_new = max(m, t)
        a = math.exp(m - m_new) if m != NEG_INF else 0.0
        w = math.exp(t - m_new)
        o = o * a + w * vi
        l = l * a + w
        m = m_new
    return m, l, o


def empty_state(dv: int):
    """The merge identity: (m=-inf, l=0, O~=0)."""
    return (NEG_INF, 0.0, np.zeros(dv))


def block_state(x, v):
    """(m_A, l_A, O~_A) of one block (page 2, 4.2.4 definitions)."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if x.size == 0:
        return empty_state(v.shape[1])
    m = float(x.max())
    w = np.exp(x - m)
    return (m, float(w.sum()), w @ v)


def merge(*states):
    """Combine any number of block states into the state of their union
    (page 2, 4.2.4, the merge equation for two blocks, applied to all at
    once). A state (m, l, O~) stands for l = sum e^(x - m) and O~ = sum
    e^(x - m) v over its block; re-expressed against a common reference R
    every sum is multiplied by e^(m - R), after which the sums over disjoint
    blocks simply add. R is the largest m, so no factor exceeds 1 (empty
    states, m = -inf, contribute 0)."""
    if not states:
        raise ValueError("merge needs at least one state")
    ref = max(st[0] for st in states)
    l_tot, o_tot = 0.0, 0.0
    for m_s, l_s, o_s in states:
        factor = float(_rescale(m_s, ref))
        l_tot = l_tot + factor * l_s
        o_tot = o_tot + factor * np.asarray(o_s, dtype=np.float64)
    return (ref, l_tot, o_tot)


def block_update(state, s_block, v_block):
    """Per-block update of page 1, section 六, for a block of rows.

    state = (m [r], l [r], O [r, d]); s_block [r, c] (hidden entries -inf);
    v_block [c, d]:
        m^(j) = max(m^(j-1), rowmax(S^(j)))
        l^(j) = e^(m^(j-1) - m^(j)) * l^(j-1) + rowsum(e^(S^(j) - m^(j)))
        O^(j) = diag(e^(m^(j-1) - m^(j))) O^(j-1) + e^(S^(j) - m^(j)) V^(j)
    """
    m_old, l_old, o_old = state
    s_block = np.asarray(s_block, dtype=np.float64)
    m_new = np.maximum(m_old, s_block.max(axis=1))
    alpha = _rescale(m_old, m_new)
    m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
    p = np.where(np.isfinite(s_block), np.exp(s_block - m_ref[:, None]), 0.0)
    l_new = alpha * l_old + p.sum(axis=1)
    o_new = alpha[:, None] * o_old + p @ np.asarray(v_block, dtype=np.float64)
    return (m_new, l_new, o_new)


def finalize(state):
    """O = diag(l)^-1 O and L = m + ln l (rows with l = 0 give 0 and -inf)."""
    m, l, o = state
    ok = l > 0
    l_safe = np.where(ok, l, 1.0)
    return (np.where(ok[:, None], o / l_safe[:, None], 0.0),
            np.where(ok, m + np.log(l_safe), NEG_INF))


def tiled_forward(q, k, v, scale: float, causal: bool, kv_len_b=None,
                  br: int = 16, bc: int = 16):
    """The tiled forward of page 2, 4.3.2 (fp64, one head).

    Outer loop over B_r-row query tiles, inner loop over B_c-column key tiles;
    per tile S_ij = scale Q_i K_j^T, hidden entries -inf, then
    ``block_update``; after the inner loop O_i = O_i / l_i and
    L_i = m_i + log l_i. For causal masking a key tile is entered only if its
    first key is <= the tile's last query (j B_c <= i B_r + B_r - 1,
    0-based), which skips exactly the tiles that are fully hidden.
    Returns (o [n, d], lse [n]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, dv = q.shape[0], v.shape[1]
    kv = n if kv_len_b is None else int(kv_len_b)
    o = np.zeros((n, dv))
    lse = np.full(n, NEG_INF)
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(i0 + br, n))
        state = (np.full(rows.size, NEG_INF), np.zeros(rows.size),
                 np.zeros((rows.size, dv)))
        for j0 in range(0, n, bc):
            if causal and j0 > rows[-1]:
                break
            cols = np.arange(j0, min(j0 + bc, n))
            s = scale * (q[rows] @ k[cols].T)
            hidden = cols[None, :] >= kv
            if causal:
                hidden = hidden | (cols[None, :] > rows[:, None])
            s = np.where(hidden, NEG_INF, s)
            state = block_update(state, s, v[cols])
        o[rows], lse[rows] = finalize(state)
    return o, lse
