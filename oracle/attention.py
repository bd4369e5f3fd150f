"""Plain float64 attention forward and backward (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
module. It is the definition of softmax attention and of its gradient, written
out with numpy; matrix products are the only library primitive it leans on.

The DASH pages (arXiv 2601.21824: the Dutch technical summary §1, the
Japanese technical summary §1, and the English abstract) state that the
deterministic backward must fix the order in which dQ is accumulated, but they
do not print the attention gradient itself. It follows from calculus:

forward, per head, with scale c and optional causal mask (key s' visible to
query s iff s' <= s, equal query and key lengths)::

    s_ij  = c * q_i . k_j            (-inf where masked)
    LSE_i = log sum_j exp(s_ij)      (natural log)
    P_ij  = exp(s_ij - LSE_i)
    O     = P V

backward, from the GIVEN O and LSE (the forward's outputs, as a fused kernel
receives them)::

    P'_ij  = exp(c q_i . k_j - LSE_i)       (0 where masked)
    dV     = P'^T dO
    dP     = dO V^T
    Delta_i = sum_d dO_id * O_id
    dS     = P' * (dP - Delta 1^T)
    dQ     = c dS K
    dK     = c dS^T Q

Arrays are float64 numpy, shaped [B, H, S, D] (LSE: [B, H, S]). Heads are
independent and are processed one at a time. Long sequences are processed in
blocks of query rows purely to bound memory: each row's quantities are exactly
the formulas above, and the per-row contributions to dK and dV are summed in
row-block order.
"""

from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def _visible(rows: np.ndarray, S: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), S] mask of keys each query row may attend to."""
    keys = np.arange(S)
    if not causal:
        return np.ones((rows.size, S), dtype=bool)
    return keys[None, :] <= rows[:, None]


def forward_head(q, k, v, causal: bool, scale: float, row_block: int = ROW_BLOCK):
    """One head's forward: returns (O [S,D], LSE [S]) in float64."""
    S = q.shape[0]
    o = np.empty_like(q)
    lse = np.empty(S)
    for r0 in range(0, S, row_block):
        rows = np.arange(r0, min(S, r0 + row_block))
        s = scale * (q[rows] @ k.T)
        s = np.where(_visible(rows, S, causal), s, -np.inf)
        m = s.max(axis=1, keepdims=True)            # every row sees key 0
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        lse[rows] = (m + np.log(z))[:, 0]
        o[rows] = (e / z) @ v
    return o, lse


def forward(q, k, v, causal: bool, scale: float, row_block: int = ROW_BLOCK):
    """Forward over all heads: q, k, v [B,H,S,D] -> (O [B,H,S,D], LSE [B,H,S])."""
    B, H, S, D = q.shape
    o = np.empty((B, H, S, v.shape[-1]))
    lse = np.empty((B, H, S))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], causal, scale, row_block)
    return o, lse


def backward_head(q, k, v, o, do, lse, causal: bool, scale: float, row_block: int = ROW_BLOCK):
    """One head's backward from the given O and LSE: returns (dQ, dK, dV)."""
    S = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, S, row_block):
        rows = np.arange(r0, min(S, r0 + row_block))
        vis = _visible(rows, S, causal)
        p = np.where(vis, np.exp(scale * (q[rows] @ k.T) - lse[rows, None]), 0.0)
        dv += p.T @ do[rows]
        dp = do[rows] @ v.T
        delta = (do[rows] * o[rows]).sum(axis=1)
        ds = p * (dp - delta[:, None])
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
    return dq, dk, dv


def backward(q, k, v, o, do, lse, causal: bool, scale: float, row_block: int = ROW_BLOCK):
    """Backward over all heads; every argument is [B,H,S,D] (lse: [B,H,S])."""
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], o[b, h], do[b, h], lse[b, h], causal, scale, row_block)
    return dq, dk, dv


def delta(o, do):
    """Delta_i = sum_d dO_id * O_id, the per-row term of the softmax gradient."""
    return (o * do).sum(axis=-1)


def softmax_probs_head(q, k, causal: bool, scale: float):
    """Materialised attention probabilities P [S,S] of one head (small S only)."""
    S = q.shape[0]
    s = scale * (q @ k.T)
    s = np.where(_visible(np.arange(S), S, causal), s, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def backward_bruteforce_head(q, k, v, do, causal: bool, scale: float):
    """Unfused backward: explicit per-row softmax Jacobian, no Delta shortcut.

    P = softmax(c Q K^T) is materialised, O = P V, dV = P^T dO, dP = dO V^T, and
    for each query row i the S x S Jacobian J_i = diag(p_i) - p_i p_i^T of the
    softmax is formed and applied: dS_i = J_i dP_i. Then dQ = c dS K and
    dK = c dS^T Q. Small S only (it is O(S^3) per head).
    Returns (O, dQ, dK, dV, dS, P).
    """
    p = softmax_probs_head(q, k, causal, scale)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    S = q.shape[0]
    ds = np.empty((S, S))
    for i in range(S):
        jac = np.diag(p[i]) - np.outer(p[i], p[i])
        ds[i] = jac @ dp[i]
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return o, dq, dk, dv, ds, p


def ds_head(q, k, v, o, do, lse, causal: bool, scale: float):
    """dS [S,S] of one head from the given O and LSE (fused form; small S only)."""
    S = q.shape[0]
    vis = _visible(np.arange(S), S, causal)
    p = np.where(vis, np.exp(scale * (q @ k.T) - lse[:, None]), 0.0)
    dp = do @ v.T
    return p * (dp - delta(o, do)[:, None])


def loss(q, k, v, do, causal: bool, scale: float):
    """Scalar L = sum(O * dO) with dO held constant; its gradient is (dQ, dK, dV)."""
    o, _ = forward(q, k, v, causal, scale)
    return float((o * do).sum())


def compare(x, y):
    """Error metrics of an approximation x against a reference y (float64).

    Returns (max_abs, rel_l2) with max_abs = max |x - y| and
    rel_l2 = ||x - y||_2 / ||y||_2 over the whole tensor.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = x - y
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    ny = float(np.sqrt((y * y).sum()))
    rel = float(np.sqrt((d * d).sum())) / ny if ny > 0 else float(np.sqrt((d * d).sum()))
    return max_abs, rel


def backward_rows_head(q, k, v, o, do, lse, causal: bool, scale: float, q_rows, k_rows):
    """The backward of one head restricted to chosen rows (for large S).

    Returns (dq[q_rows], dk[k_rows], dv[k_rows]) from the same formulas as
    backward_head: a dQ row needs its own row of P' and dS; a dK/dV row needs
    one column of P' and dS, hence every query's LSE and Delta. O(S*D) per row.
    """
    S = q.shape[0]
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dlt = delta(o, do)
    keys = np.arange(S)
    # rows of dS for the chosen queries
    vis_q = (keys[None, :] <= q_rows[:, None]) if causal else np.ones((q_rows.size, S), dtype=bool)
    p_q = np.where(vis_q, np.exp(scale * (q[q_rows] @ k.T) - lse[q_rows, None]), 0.0)
    ds_q = p_q * (do[q_rows] @ v.T - dlt[q_rows, None])
    dq = scale * (ds_q @ k)
    # columns of P' and dS for the chosen keys
    vis_k = (keys[:, None] >= k_rows[None, :]) if causal else np.ones((S, k_rows.size), dtype=bool)
    p_k = np.where(vis_k, np.exp(scale * (q @ k[k_rows].T) - lse[:, None]), 0.0)
    ds_k = p_k * (do @ v[k_rows].T - dlt[:, None])
    dv = p_k.T @ do
    dk = scale * (ds_k.T @ q)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Grouped-query attention (query heads sharing K/V heads). Not on the pages:
# the end-to-end models they time are of a family that shares K/V heads across
# query heads, which asks for a second fixed-order reduction of dK/dV. With H
# query heads and Hkv K/V heads (G = H / Hkv), query head h attends with K/V
# head h // G. Each query head is ordinary attention with that K and V, so the
# forward is the per-head definition above; a K/V head is used by G query
# heads, so by the chain rule its gradient is the sum of the G per-use
# gradients (dK, dV of each query head taken with respect to its copy).


def group_of(H: int, Hkv: int, h: int) -> int:
    """K/V head of query head h (consecutive query heads share one)."""
    if Hkv <= 0 or H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    return h // (H // Hkv)


def forward_grouped(q, k, v, causal: bool, scale: float, row_block: int = ROW_BLOCK):
    """q [B,H,S,D], k, v [B,Hkv,S,D] -> (O [B,H,S,D], LSE [B,H,S])."""
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, H, S, v.shape[-1]))
    lse = np.empty((B, H, S))
    for b in range(B):
        for h in range(H):
            g = group_of(H, Hkv, h)
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, g], v[b, g], causal, scale, row_block)
    return o, lse


def backward_grouped(q, k, v, o, do, lse, causal: bool, scale: float, row_block: int = ROW_BLOCK):
    """Gradients for shared K/V heads: dQ [B,H,S,D]; dK, dV [B,Hkv,S,D] summed over each group."""
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = group_of(H, Hkv, h)
            dq[b, h], dkh, dvh = backward_head(q[b, h], k[b, g], v[b, g], o[b, h], do[b, h], lse[b, h], causal,
                                              scale, row_block)
            dk[b, g] += dkh
            dv[b, g] += dvh
    return dq, dk, dv


def loss_grouped(q, k, v, do, causal: bool, scale: float):
    """The scalar sum(O * dO) with shared K/V heads (its gradient is backward_grouped's)."""
    o, _ = forward_grouped(q, k, v, causal, scale)
    return float((o * do).sum())
