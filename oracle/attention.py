"""Plain softmax attention and its analytic gradient in float64 (oracle; test infrastructure only).

Why the plain definition is the oracle
--------------------------------------
The "FlashAttention (v2)" glossary page (its opening definition) says the
method computes attention without approximating the result and that its output
matches standard attention exactly; standard attention is described there as
materialising every token-by-token score.  So the oracle *is* standard
attention, written out from its definition, with the full score matrix of one
(batch, head) materialised at a time:

    S = scale * Q K^T                       (Nq x Nk scores)
    S_ij = -inf for j > i + (Nk - Nq)       when causal
    L_i  = log sum_j exp(S_ij)              (natural-log logsumexp of the
                                             scaled, masked scores)
    P    = exp(S - L)                       (row-stochastic)
    O    = P V

Query and key lengths may differ.  The pages show the causal mask only for
one sequence attending to itself (Nq = Nk: key j is kept for query i iff
j <= i).  For Nq != Nk the reading taken here places the queries at the END
of the key sequence (query i sits at key position i + Nk - Nq, the
"bottom-right" alignment of a query block appended to a key/value cache),
which reduces to the square rule for Nq = Nk.  With Nq > Nk the first
Nq - Nk queries see no key: their softmax is over the empty set, so their L
is -inf (the logsumexp of nothing), their row of P is zero, their output O is
zero, and they contribute nothing to any gradient.

The pages print no formulas for the logsumexp output L or for the gradient;
they are the textbook definition of the row logsumexp and the analytic
derivative of the scalar f = sum(dO * O):

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij
    dS = P * (dP - D 1^T)
    dQ = scale * dS K
    dK = scale * dS^T Q

All arrays are float64 ``[B, H, N, d]`` (or one head ``[N, d]``), with
N = Nq for Q, O, dO, dQ and N = Nk for K, V, dK, dV; L and D are
``[B, H, Nq]``.  The "Sampled" helpers below evaluate the same definitions for
chosen query rows / key columns only, so that the definition can be checked at
sequence lengths whose N x N matrix would not fit comfortably in host memory;
they evaluate rows one chunk at a time and nothing else.
"""

import numpy as np


# ---------------------------------------------------------------------------
# building blocks (one head)
# ---------------------------------------------------------------------------

def causal_offset(n_q, n_k):
    """Key position of query 0 under the bottom-right reading: Nk - Nq."""
    return int(n_k) - int(n_q)


def scores(q, k, scale, causal, rows=None, n_q=None):
    """Scaled, masked scores S = scale * q k^T for one head.

    q: [Nq, d] (or the selected rows), k: [Nk, d].  ``rows`` gives the
    absolute query index of each row of ``q`` (needed for the causal mask when
    q is a subset) and ``n_q`` the total number of query rows (default: the
    rows of q when ``rows`` is None, else Nk, i.e. a square problem).  Causal
    masking keeps key j for query i iff j <= i + Nk - Nq; for Nq = Nk that is
    j <= i, the mask described for causal attention on the "FlashAttention-2:
    Faster Attention with Better Parallelism and Work Partitioning" page
    (closing sentence on the causal speed-up).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = float(scale) * (q @ k.T)
    if causal:
        n_k = k.shape[0]
        if n_q is None:
            n_q = q.shape[0] if rows is None else n_k
        qi = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        kj = np.arange(n_k)
        s = np.where(kj[None, :] > qi[:, None] + causal_offset(n_q, n_k), -np.inf, s)
    return s


def softmax_rows(s):
    """Row softmax of a score matrix and its natural-log logsumexp.

    Returns (P, L) with L_i = log sum_j exp(S_ij) computed stably as
    m_i + log sum_j exp(S_ij - m_i), m_i = max_j S_ij, and P = exp(S - L).
    A row with no finite score (a query that sees no key) has L_i = -inf and
    a zero row of P.
    """
    m = np.max(s, axis=1)
    empty = np.isneginf(m)
    m0 = np.where(empty, 0.0, m)
    z = np.sum(np.exp(s - m0[:, None]), axis=1)
    lse = np.where(empty, -np.inf, m0 + np.log(np.where(empty, 1.0, z)))
    lse0 = np.where(empty, 0.0, lse)
    p = np.where(empty[:, None], 0.0, np.exp(s - lse0[:, None]))
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
    """O [B,H,Nq,d] and L [B,H,Nq] for every (batch, head), one head at a time."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def backward(q, k, v, do, scale, causal):
    """dQ [B,H,Nq,d], dK and dV [B,H,Nk,d] for every (batch, head), one head at a time."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    n_k = np.shape(k)[2]
    dq = np.empty_like(q)
    dk = np.empty((B, H, n_k, d), dtype=np.float64)
    dv = np.empty((B, H, n_k, v.shape[-1]), dtype=np.float64)
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
    q = np.asarray(q, dtype=np.float64)
    s = scores(q[rows], k, scale, causal, rows=rows, n_q=q.shape[0])
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
        s = scores(q[rows], k, scale, causal, rows=rows, n_q=n)
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
    s = scores(q[rows], k, scale, causal, rows=rows, n_q=q.shape[0])
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
    s = float(scale) * (q @ k[cols].T)                       # [Nq, c]
    if causal:
        off = causal_offset(n, k.shape[0])
        s = np.where(cols[None, :] > np.arange(n)[:, None] + off, -np.inf, s)
    # rows that see no key (L = -inf) have every score masked: P = 0 there
    p = np.where(np.isneginf(s), 0.0, np.exp(s - np.where(np.isneginf(lse), 0.0, lse)[:, None]))
    dp = do @ v[cols].T
    ds = p * (dp - d_row[:, None])
    dv = p.T @ do
    dk = float(scale) * (ds.T @ q)
    return dk, dv
