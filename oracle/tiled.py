"""Float64 model of tile-by-tile exact attention (oracle side; test infrastructure only).

This module is not a parity source for the GPU.  It exists to pin the claim
that working one tile at a time reaches *exactly* the plain result ("FlashAttention
(v2)" glossary page, opening definition: attention computed tile by tile in
on-chip memory, without approximating the result; the same page's
twelve-token walk-through in four-by-four tiles), by running the tiled
algorithm in float64 and comparing it to ``attention.forward_head`` /
``attention.backward_head`` in ``tests/test_oracle.py``.

Forward: one query row-block at a time; for each key/value tile a running row
maximum m and row sum l are updated (online softmax) and the output is
rescaled by exp(m_old - m_new); division by l happens once, after the last
tile ("FlashAttention-2" summary page, "How It Works" item 2: scaling moved out
of the inner loop to the end).  L = m + log l.

Causal: tiles lying wholly above the diagonal are skipped and only tiles that
cross the diagonal are masked element by element ("FlashAttention-2: Faster
Attention with Better Parallelism and Work Partitioning" page, closing sentence).

Backward: one key/value column-block at a time, looping over query
row-blocks, recomputing P = exp(S - L) from the stored L, with D_i = sum_k
dO_ik O_ik.
"""

import numpy as np


def _tile_kind(r0, r1, c0, c1, causal):
    """'skip' if the tile [r0,r1) x [c0,c1) is wholly above the diagonal,
    'mask' if it crosses it, 'full' otherwise."""
    if not causal:
        return "full"
    if c0 > r1 - 1:
        return "skip"
    if c1 - 1 > r0:
        return "mask"
    return "full"


def tiled_forward_head(q, k, v, scale, causal, br, bc, log=None):
    """O, L of one head by online softmax over br x bc tiles (float64).

    ``log`` (a list) receives (row_block, col_block, kind) for every tile.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for ib, r0 in enumerate(range(0, n, br)):
        r1 = min(n, r0 + br)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, v.shape[1]))
        for jb, c0 in enumerate(range(0, n, bc)):
            c1 = min(n, c0 + bc)
            kind = _tile_kind(r0, r1, c0, c1, causal)
            if log is not None:
                log.append((ib, jb, kind))
            if kind == "skip":
                continue
            s = scale * (q[r0:r1] @ k[c0:c1].T)
            if kind == "mask":
                qi = np.arange(r0, r1)[:, None]
                kj = np.arange(c0, c1)[None, :]
                s = np.where(kj > qi, -np.inf, s)
            m_new = np.maximum(m, np.max(s, axis=1))
            alpha = np.exp(m - m_new)              # exp(-inf) = 0 on the first tile
            p = np.exp(s - m_new[:, None])
            l = alpha * l + np.sum(p, axis=1)
            acc = alpha[:, None] * acc + p @ v[c0:c1]
            m = m_new
        o[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return o, lse


def tiled_backward_head(q, k, v, o, lse, do, scale, causal, br, bc, log=None):
    """dQ, dK, dV of one head, key/value block by block (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    d_row = np.sum(do * np.asarray(o, dtype=np.float64), axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for jb, c0 in enumerate(range(0, n, bc)):
        c1 = min(n, c0 + bc)
        for ib, r0 in enumerate(range(0, n, br)):
            r1 = min(n, r0 + br)
            kind = _tile_kind(r0, r1, c0, c1, causal)
            if log is not None:
                log.append((ib, jb, kind))
            if kind == "skip":
                continue
            s = scale * (q[r0:r1] @ k[c0:c1].T)
            if kind == "mask":
                qi = np.arange(r0, r1)[:, None]
                kj = np.arange(c0, c1)[None, :]
                s = np.where(kj > qi, -np.inf, s)
            p = np.exp(s - lse[r0:r1, None])
            dv[c0:c1] += p.T @ do[r0:r1]
            dp = do[r0:r1] @ v[c0:c1].T
            ds = p * (dp - d_row[r0:r1, None])
            dk[c0:c1] += scale * (ds.T @ q[r0:r1])
            dq[r0:r1] += scale * (ds @ k[c0:c1])
    return dq, dk, dv
