"""Plain softmax attention and its analytic gradient in float64 (oracle; test infrastructure only).

Why the plain definition is the oracle
--------------------------------------
The "FlashAttention (v2)" glossary page (its opening definition) says the
method computes attention without approximating the result and that its output
matches standard attention exactly; standard attention is described there as
materialising every token-by-token score.  So the oracle *is* standard
attention, written out from its definition, with the full score matrix of one
(batch, head) materialised at a time:

    S = scale * Q K^T                       (N x N scores)
    S_ij = -inf for j > i  when causal      (top-left aligned, square)
    L_i  = log sum_j exp(S_ij)              (natural-log logsumexp of the
                                             scaled, masked scores)
    P    = exp(S - L)                       (row-stochastic)
    O    = P V

The pages print no formulas for the logsumexp output L or for the gradient;
they are the textbook definition of the row logsumexp and the analytic
derivative of the scalar f = sum(dO * O):

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij
    dS = P * (dP - D 1^T)
    dQ = scale * dS K
    dK = scale * dS^T Q

All arrays are float64 ``[B, H, N, d]`` (or one head ``[N, d]``); L and D are
``[B, H, N]``.  The "Sampled" helpers below evaluate the same definitions for
chosen query rows / key columns only, so that the definition can be checked at
sequence lengths whose N x N matrix would not fit comfortably in host memory;
they evaluate rows one chunk at a time and nothing else.
"""

import numpy as np


# ---------------------------------------------------------------------------
# building blocks (one head)
# ---------------------------------------------------------------------------

def scores(q, k, scale, causal, rows=None):
    """Scaled, masked scores S = scale * q k^T for one head.

    q: [N, d] (or the selected rows), k: [N, d].  ``rows`` gives the absolute
    query index of each row of ``q`` (needed for the causal mask when q is a
    subset).  Causal masking keeps key j for query i iff j <= i (the mask
    described for causal attention on the "FlashAttention-2: Faster Attention
    with Better Parallelism and Work Partitioning" page, closing sentence on
    the causal speed-up).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = float(scale) * (q @ k.T)
    if causal:
        n_q = q.shape[0]
        qi = np.arange(n_q) if rows is None else np.asarray(rows)
        kj = np.arange(k.shape[0])
        s = np.where(kj[None, :] > qi[:, None], -np.inf, s)
    return s


def softmax_rows(s):
    """Row softmax of a score matrix and its natural-log logsumexp.

    Returns (P, L) with L_i = log sum_j exp(S_ij) computed stably as
    m_i + log sum_j exp(S_ij - m_i), m_i = max_j S_ij, and P = exp(S - L).
    Every row must hold at least one finite score (true for causal top-left
    masking, where the diagonal is always kept).
    """
    m = np.max(s, axis=1)
    lse = m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))
    p = np.exp(s - lse[:, None])
    return p, lse


# ---------------------------------------------------------------------------
# full definition (one head, then all heads)
# ---------------------------------------------------------------------------

def forward_head(q, k, v, scale, causal):
    """O, L for one head: O = softmax(scale q k^T, masked) v."""
    s = scores(q, k, scale, causal)
    p, lse = softmax_rows(s)
    o = p @ np.asarray(v, dtype=np.float64)
    return o, lse


def backward_head(q, k, v, do, scale, causal):
    """dQ, dK, dV of f = sum(dO * O) for one head (the analytic gradient)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    s = scores(q, k, scale, causal)
    p, _ = softmax_rows(s)
    dv = p.T @ do
    dp = do @ v.T
    d_row = np.sum(p * dp, axis=1)
    ds = p * (dp - d_row[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def forward(q, k, v, scale, causal):
    """O [B,H,N,d] and L [B,H,N] for every (batch, head), one head at a time."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def backward(q, k, v, do, scale, causal):
    """dQ, dK, dV [B,H,N,d] for every (batch, head), one head at a time."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty((B, H, N, d), dtype=np.float64)
    dv = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# sampled evaluation of the same definitions (one head)
# ---------------------------------------------------------------------------

def forward_rows(q, k, v, scale, causal, rows):
    """O and L of the selected query rows of one head (same definition)."""
    rows = np.asarray(rows)
    s = scores(np.asarray(q, dtype=np.float64)[rows], k, scale, causal, rows=rows)
    p, lse = softmax_rows(s)
    return p @ np.asarray(v, dtype=np.float64), lse


def row_stats(q, k, v, do, scale, causal, chunk=512):
    """L_i and D_i = sum_j P_ij dP_ij for every query row of one head.

    Evaluated ``chunk`` rows at a time from the definition (scores of those
    rows, their softmax, dP = dO V^T of those rows).
    """
    q = np.asarray(q, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    lse = np.empty(n)
    d_row = np.empty(n)
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        s = scores(q[rows], k, scale, causal, rows=rows)
        p, lse[rows] = softmax_rows(s)
        dp = do[rows] @ v.T
        d_row[rows] = np.sum(p * dp, axis=1)
    return lse, d_row


def backward_rows(q, k, v, do, scale, causal, rows):
    """dQ of the selected query rows of one head: dQ_i = scale sum_j dS_ij k_j."""
    rows = np.asarray(rows)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    s = scores(q[rows], k, scale, causal, rows=rows)
    p, _ = softmax_rows(s)
    dp = do[rows] @ v.T
    d_row = np.sum(p * dp, axis=1)
    ds = p * (dp - d_row[:, None])
    return float(scale) * (ds @ k)


def backward_cols(q, k, v, do, scale, causal, cols, stats=None):
    """dK and dV of the selected key columns of one head.

    dV_j = sum_i P_ij dO_i and dK_j = scale sum_i dS_ij q_i need L_i and D_i
    of every row i; pass ``stats=(L, D)`` from ``row_stats`` to reuse them.
    """
    cols = np.asarray(cols)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if stats is None:
        stats = row_stats(q, k, v, do, scale, causal)
    lse, d_row = stats
    n = q.shape[0]
    s = float(scale) * (q @ k[cols].T)                       # [N, c]
    if causal:
        s = np.where(cols[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - lse[:, None])
    dp = do @ v[cols].T
    ds = p * (dp - d_row[:, None])
    dv = p.T @ do
    dk = float(scale) * (ds.T @ q)
    return dk, dv
