"""Pins for the CPU oracle (no GPU).

Each check ties the oracle to something other than itself: closed forms of
softmax attention, finite differences of f = sum(dO * O), invariants of the
definition, brute force in pure Python on tiny inputs, and a library special
case (PyTorch's float64 CPU scaled_dot_product_attention with autograd).  The
last test plants plausible mistakes in copies of the oracle and shows that the
pins catch every one.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import attention as A


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# bf16 decoding
# ---------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC040, 0x3F00,
                     0x7F80, 0xFF80, 0x0001, 0x7F7F], dtype=np.uint16)
    got = oracle.bf16_bits_to_float64(bits)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, -3.0, 0.5, np.inf, -np.inf,
            2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127]
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[1])
    assert np.isnan(oracle.bf16_bits_to_float64(np.array([0x7FC0], dtype=np.uint16))[0])
    # int16 views decode the same
    assert np.array_equal(oracle.bf16_bits_to_float64(bits.view(np.int16)), got)


def test_fp16_decode_known_patterns():
    bits = np.array([0x0000, 0x8000, 0x3C00, 0xBC00, 0x4000, 0xC200, 0x3800, 0x7C00, 0xFC00,
                     0x0001, 0x0400, 0x7BFF, 0x3555], dtype=np.uint16)
    got = oracle.fp16_bits_to_float64(bits)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, -3.0, 0.5, np.inf, -np.inf,
            2.0 ** -24, 2.0 ** -14, 65504.0, 1365.0 / 4096.0]   # 0x3555 = 1.0101010101b x 2^-2
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[1])
    assert np.isnan(oracle.fp16_bits_to_float64(np.array([0x7E00], dtype=np.uint16))[0])
    assert np.array_equal(oracle.bits_to_float64(bits.view(np.int16), "fp16"), got)
    assert np.array_equal(oracle.bits_to_float64(bits, "bf16"), oracle.bf16_bits_to_float64(bits))


# ---------------------------------------------------------------------------
# forward closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_give_mean_of_v(causal):
    n, d = 37, 8
    q = np.zeros((n, d))
    k = rand((n, d), 1)
    v = rand((n, d), 2)
    o, lse = A.forward_head(q, k, v, 0.3, causal)
    if causal:
        want_o = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
        want_l = np.log(np.arange(1, n + 1))
    else:
        want_o = np.broadcast_to(v.mean(axis=0), (n, d))
        want_l = np.full(n, np.log(n))
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, want_l, rtol=0, atol=1e-13)


def test_causal_row0_is_v0():
    n, d = 20, 16
    q, k, v = rand((n, d), 3), rand((n, d), 4), rand((n, d), 5)
    scale = 0.25
    o, lse = A.forward_head(q, k, v, scale, True)
    assert np.array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(scale * q[0] @ k[0], abs=1e-15)


def test_single_token():
    q, k, v = rand((1, 4), 6), rand((1, 4), 7), rand((1, 4), 8)
    for causal in (False, True):
        o, lse = A.forward_head(q, k, v, 0.7, causal)
        assert np.array_equal(o, v)
        assert lse[0] == pytest.approx(0.7 * q[0] @ k[0], abs=1e-15)
        dq, dk, dv = A.backward_head(q, k, v, rand((1, 4), 9), 0.7, causal)
        assert np.all(dq == 0) and np.all(dk == 0)
        np.testing.assert_array_equal(dv, rand((1, 4), 9))


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_output(causal):
    n, d = 19, 6
    o, _ = A.forward_head(rand((n, d), 10), rand((n, d), 11), np.ones((n, d)), 0.5, causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_are_row_stochastic(causal):
    n, d = 23, 5
    s = A.scores(rand((n, d), 12), rand((n, d), 13), 0.4, causal)
    p, _ = A.softmax_rows(s)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(n, 1)] == 0)
        assert np.all(p[np.tril_indices(n)] > 0)


def test_brute_force_tiny():
    """Pure-Python loops over the definition on a 5-token, 3-dim head."""
    n, d = 5, 3
    q, k, v = rand((n, d), 14), rand((n, d), 15), rand((n, d), 16)
    scale = 0.8
    for causal in (False, True):
        o, lse = A.forward_head(q, k, v, scale, causal)
        for i in range(n):
            visible = [j for j in range(n) if not (causal and j > i)]
            sij = {j: scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in visible}
            z = math.fsum(math.exp(s) for s in sij.values())
            assert lse[i] == pytest.approx(math.log(z), abs=1e-13)
            for t in range(d):
                want = math.fsum(math.exp(sij[j]) / z * v[j][t] for j in visible)
                assert o[i, t] == pytest.approx(want, abs=1e-13)


# ---------------------------------------------------------------------------
# forward invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    n, d = 17, 8
    q, k, v = rand((n, d), 17), rand((n, d), 18), rand((n, d), 19)
    u = rand(d, 20)
    scale = 0.35
    o1, l1 = A.forward_head(q, k, v, scale, causal)
    o2, l2 = A.forward_head(q, k + u[None, :], v, scale, causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + scale * q @ u, atol=1e-12)


def test_permutation_equivariance_noncausal():
    n, d = 21, 4
    q, k, v = rand((n, d), 21), rand((n, d), 22), rand((n, d), 23)
    o, lse = A.forward_head(q, k, v, 0.5, False)
    pk = np.random.default_rng(24).permutation(n)
    o2, l2 = A.forward_head(q, k[pk], v[pk], 0.5, False)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(l2, lse, atol=1e-13)
    pq = np.random.default_rng(25).permutation(n)
    o3, l3 = A.forward_head(q[pq], k, v, 0.5, False)
    np.testing.assert_allclose(o3, o[pq], atol=1e-13)
    np.testing.assert_allclose(l3, lse[pq], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_linear_in_v(causal):
    n, d = 15, 6
    q, k = rand((n, d), 26), rand((n, d), 27)
    v1, v2 = rand((n, d), 28), rand((n, d), 29)
    o1, _ = A.forward_head(q, k, v1, 0.6, causal)
    o2, _ = A.forward_head(q, k, v2, 0.6, causal)
    o3, _ = A.forward_head(q, k, 2.0 * v1 - 3.0 * v2, 0.6, causal)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, atol=1e-12)


def test_causal_isolation():
    n, d = 16, 8
    q, k, v = rand((n, d), 30), rand((n, d), 31), rand((n, d), 32)
    o, lse = A.forward_head(q, k, v, 0.5, True)
    for i in (0, 5, 14):
        k2, v2 = k.copy(), v.copy()
        k2[i + 1:] += 100.0 * rand((n - i - 1, d), 33)
        v2[i + 1:] -= 50.0
        o2, l2 = A.forward_head(q, k2, v2, 0.5, True)
        np.testing.assert_array_equal(o2[: i + 1], o[: i + 1])
        np.testing.assert_array_equal(l2[: i + 1], lse[: i + 1])


def test_logsumexp_gradient_by_finite_differences():
    """dL_i/dq_i = scale * sum_j P_ij k_j — pins L to the same P that makes O."""
    n, d, scale, h = 7, 4, 0.9, 1e-6
    q, k, v = rand((n, d), 34), rand((n, d), 35), rand((n, d), 36)
    for causal in (False, True):
        p, _ = A.softmax_rows(A.scores(q, k, scale, causal))
        want = scale * (p @ k)
        for i in range(n):
            for t in range(d):
                qp, qm = q.copy(), q.copy()
                qp[i, t] += h
                qm[i, t] -= h
                fd = (A.forward_head(qp, k, v, scale, causal)[1][i]
                      - A.forward_head(qm, k, v, scale, causal)[1][i]) / (2 * h)
                assert fd == pytest.approx(want[i, t], rel=1e-6, abs=1e-8)


# ---------------------------------------------------------------------------
# backward: finite differences, invariants, closed forms
# ---------------------------------------------------------------------------

def fd_check(backward_fn, causal, scale, seed=40, h=1e-6):
    """Max relative error of backward_fn vs central differences of sum(dO*O), B=H=2, N=8, d=4."""
    B, H, n, d = 2, 2, 8, 4
    q, k, v, do = (rand((B, H, n, d), seed + i) for i in range(4))
    dq, dk, dv = backward_fn(q, k, v, do, scale, causal)

    def f(qq, kk, vv):
        o, _ = A.forward(qq, kk, vv, scale, causal)
        return float(np.sum(do * o))

    worst = 0.0
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = ap, am
            fd[idx] = (f(args_p["q"], args_p["k"], args_p["v"])
                       - f(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        err = np.linalg.norm(grad - fd) / max(np.linalg.norm(fd), 1e-300)
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.5, 1.3])  # 0.5 = 1/sqrt(d) at d = 4
def test_gradients_match_finite_differences(causal, scale):
    assert fd_check(A.backward, causal, scale) <= 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    n, d, scale = 29, 8, 0.45
    q, k, v, do = (rand((n, d), 60 + i) for i in range(4))
    dq, dk, dv = A.backward_head(q, k, v, do, scale, causal)
    o, _ = A.forward_head(q, k, v, scale, causal)
    # keys enter only through q k^T: sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    # rows of P sum to one: sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-11)
    # S depends on Q, K only through Q K^T: <Q, dQ> = <K, dK>
    assert np.sum(q * dq) == pytest.approx(np.sum(k * dk), abs=1e-10)
    # D_i = sum_j P_ij dP_ij equals dO_i . O_i
    _, d_row = A.row_stats(q, k, v, do, scale, causal)
    np.testing.assert_allclose(d_row, np.sum(do * o, axis=1), atol=1e-12)
    if causal:
        assert np.all(dq[0] == 0)


def test_backward_closed_form_zero_queries():
    n, d, scale = 11, 5, 0.7
    q = np.zeros((n, d))
    k, v, do = rand((n, d), 70), rand((n, d), 71), rand((n, d), 72)
    dq, dk, dv = A.backward_head(q, k, v, do, scale, False)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    vbar = v.mean(axis=0)
    want = (scale / n) * ((do @ (v - vbar).T) @ k)
    np.testing.assert_allclose(dq, want, atol=1e-13)
    np.testing.assert_allclose(dv, np.broadcast_to(do.sum(axis=0) / n, (n, d)), atol=1e-13)


# ---------------------------------------------------------------------------
# library special case: PyTorch float64 CPU attention + autograd
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    torch = pytest.importorskip("torch")
    B, H, n, d, scale = 2, 3, 33, 16, 0.25
    arrs = [rand((B, H, n, d), 80 + i) for i in range(4)]
    o, lse = A.forward(*arrs[:3], scale, causal)
    dq, dk, dv = A.backward(*arrs, scale, causal)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in arrs[:3])
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.tensor(arrs[3], dtype=torch.float64))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    # L: SDPA over an extra all-ones value column of a shifted problem gives
    # sum_j P_ij = 1; instead use V = e_j one-hot columns of exp-weights:
    # O with V = I (identity, N x N) returns P itself, whose log of the
    # unnormalised scores recovers L_i = S_ij - log P_ij for any visible j.
    eye = torch.eye(n, dtype=torch.float64).expand(B, H, n, n)
    p = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(arrs[0]), torch.tensor(arrs[1]), eye, is_causal=causal, scale=scale).numpy()
    s_diag = scale * np.einsum("bhnd,bhnd->bhn", arrs[0], arrs[1])
    np.testing.assert_allclose(lse, s_diag - np.log(np.einsum("bhnn->bhn", p)), atol=1e-11)


# ---------------------------------------------------------------------------
# sampled evaluation == full definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_sampled_helpers_match_full(causal):
    n, d, scale = 70, 8, 0.3
    q, k, v, do = (rand((n, d), 90 + i) for i in range(4))
    o, lse = A.forward_head(q, k, v, scale, causal)
    dq, dk, dv = A.backward_head(q, k, v, do, scale, causal)
    rows = np.array([0, 1, 33, 69])
    o_r, l_r = A.forward_rows(q, k, v, scale, causal, rows)
    np.testing.assert_allclose(o_r, o[rows], atol=1e-13)
    np.testing.assert_allclose(l_r, lse[rows], atol=1e-13)
    np.testing.assert_allclose(A.backward_rows(q, k, v, do, scale, causal, rows), dq[rows], atol=1e-12)
    stats = A.row_stats(q, k, v, do, scale, causal, chunk=16)
    np.testing.assert_allclose(stats[0], lse, atol=1e-13)
    cols = np.array([0, 7, 50, 69])
    dk_c, dv_c = A.backward_cols(q, k, v, do, scale, causal, cols, stats=stats)
    np.testing.assert_allclose(dk_c, dk[cols], atol=1e-12)
    np.testing.assert_allclose(dv_c, dv[cols], atol=1e-12)


# ---------------------------------------------------------------------------
# tiling is exact (fp64 model of the online-softmax algorithm)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,br,bc", [(1, 4, 4), (12, 4, 4), (13, 4, 4), (128, 32, 16), (128, 16, 64), (100, 64, 32)])
def test_tiled_model_equals_definition(causal, n, br, bc):
    d, scale = 8, 0.37
    q, k, v, do = (rand((n, d), 100 + i) for i in range(4))
    o, lse = A.forward_head(q, k, v, scale, causal)
    to, tl = oracle.tiled_forward_head(q, k, v, scale, causal, br, bc)
    np.testing.assert_allclose(to, o, atol=1e-12)
    np.testing.assert_allclose(tl, lse, atol=1e-12)
    dq, dk, dv = A.backward_head(q, k, v, do, scale, causal)
    tq, tk, tv = oracle.tiled_backward_head(q, k, v, to, tl, do, scale, causal, br, bc)
    np.testing.assert_allclose(tq, dq, atol=1e-12)
    np.testing.assert_allclose(tk, dk, atol=1e-12)
    np.testing.assert_allclose(tv, dv, atol=1e-12)


def test_twelve_token_four_by_four_tiles():
    """Twelve tokens in 4x4 tiles: 3x3 tiles; causal skips 3, masks the 3 diagonal ones."""
    n, d = 12, 4
    q, k, v = (rand((n, d), 110 + i) for i in range(3))
    log = []
    oracle.tiled_forward_head(q, k, v, 0.5, True, 4, 4, log=log)
    kinds = {(i, j): kind for i, j, kind in log}
    assert len(kinds) == 9
    assert sorted(kind for kind in kinds.values()).count("skip") == 3
    assert [kinds[(i, i)] for i in range(3)] == ["mask"] * 3
    assert all(kinds[(i, j)] == "skip" for i in range(3) for j in range(3) if j > i)
    assert all(kinds[(i, j)] == "full" for i in range(3) for j in range(3) if j < i)


# ---------------------------------------------------------------------------
# the pins catch plausible mistakes (planted in copies of the oracle, on the CPU)
# ---------------------------------------------------------------------------

def _bwd_variant(mistake):
    def head(q, k, v, do, scale, causal):
        s = A.scores(q, k, scale, causal)
        p, _ = A.softmax_rows(s)
        dv = p.T @ do if mistake != "transposed_p" else p @ do
        dp = do @ v.T
        d_row = np.sum(p * dp, axis=1) if mistake != "no_d_term" else 0.0 * dp[:, 0]
        ds = p * (dp - d_row[:, None]) if mistake != "sign" else p * (d_row[:, None] - dp)
        dq = (scale if mistake != "no_scale_dq" else 1.0) * (ds @ k)
        dk = scale * (ds.T @ q) if mistake != "dk_uses_k" else scale * (ds.T @ k)
        return dq, dk, dv

    def full(q, k, v, do, scale, causal):
        B, H = q.shape[:2]
        out = [np.empty_like(q) for _ in range(3)]
        for b in range(B):
            for h in range(H):
                r = head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
                for o_, r_ in zip(out, r):
                    o_[b, h] = r_
        return tuple(out)
    return full


@pytest.mark.parametrize("mistake", ["transposed_p", "no_d_term", "sign", "no_scale_dq", "dk_uses_k"])
def test_finite_differences_catch_planted_backward_mistakes(mistake):
    assert fd_check(_bwd_variant(mistake), False, 0.5) > 1e-3


def test_closed_forms_catch_planted_forward_mistakes():
    n, d = 9, 4
    q0 = np.zeros((n, d))
    k, v = rand((n, d), 120), rand((n, d), 121)
    # L in log2 instead of natural log
    s = A.scores(q0, k, 0.5, False)
    m = s.max(axis=1)
    l_log2 = m + np.log2(np.sum(np.exp(s - m[:, None]), axis=1))
    assert not np.allclose(l_log2, np.log(n))
    # causal mask the wrong way round (upper instead of lower triangle)
    s_bad = np.where(np.arange(n)[None, :] < np.arange(n)[:, None], -np.inf,
                     0.5 * rand((n, d), 122) @ k.T)
    p_bad, _ = A.softmax_rows(s_bad)
    assert not np.allclose((p_bad @ v)[0], v[0])


# ---------------------------------------------------------------------------
# query and key lengths that differ (causal mask aligned bottom-right)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nq,nk", [(4, 7), (6, 3), (1, 5)])
def test_brute_force_tiny_rectangular(nq, nk):
    """Pure-Python loops: query i sees key j iff j <= i + nk - nq (causal); empty rows give O = 0, L = -inf."""
    d, scale = 3, 0.7
    q, k, v = rand((nq, d), 200), rand((nk, d), 201), rand((nk, d), 202)
    for causal in (False, True):
        o, lse = A.forward_head(q, k, v, scale, causal)
        assert o.shape == (nq, d) and lse.shape == (nq,)
        for i in range(nq):
            visible = [j for j in range(nk) if not (causal and j > i + nk - nq)]
            if not visible:
                assert lse[i] == -math.inf and np.all(o[i] == 0)
                continue
            sij = {j: scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in visible}
            z = math.fsum(math.exp(x) for x in sij.values())
            assert lse[i] == pytest.approx(math.log(z), abs=1e-13)
            for t in range(d):
                want = math.fsum(math.exp(sij[j]) / z * v[j][t] for j in visible)
                assert o[i, t] == pytest.approx(want, abs=1e-13)


def test_single_query_sees_every_key():
    """Decoding one query against a key/value cache: causal equals non-causal."""
    nk, d, scale = 19, 8, 0.35
    q, do = rand((1, d), 210), rand((1, d), 211)
    k, v = rand((nk, d), 212), rand((nk, d), 213)
    o_c, l_c = A.forward_head(q, k, v, scale, True)
    o_n, l_n = A.forward_head(q, k, v, scale, False)
    np.testing.assert_array_equal(o_c, o_n)
    np.testing.assert_array_equal(l_c, l_n)
    for gc, gn in zip(A.backward_head(q, k, v, do, scale, True), A.backward_head(q, k, v, do, scale, False)):
        np.testing.assert_array_equal(gc, gn)


def test_bottom_right_rows_are_the_tail_of_the_square_problem():
    """Nq < Nk: the queries are the last Nq positions of an Nk-token causal problem."""
    nk, nq, d, scale = 23, 9, 6, 0.5
    qf, k, v, dof = (rand((nk, d), 220 + i) for i in range(4))
    q, do = qf[nk - nq:], dof[nk - nq:]
    o_sq, l_sq = A.forward_head(qf, k, v, scale, True)
    o, lse = A.forward_head(q, k, v, scale, True)
    np.testing.assert_allclose(o, o_sq[nk - nq:], atol=1e-14)
    np.testing.assert_allclose(lse, l_sq[nk - nq:], atol=1e-14)
    # gradient of sum(dO * O) over the last nq rows only = square problem with dO = 0 on the first rows
    do_sq = np.zeros_like(dof)
    do_sq[nk - nq:] = do
    dq_sq, dk_sq, dv_sq = A.backward_head(qf, k, v, do_sq, scale, True)
    dq, dk, dv = A.backward_head(q, k, v, do, scale, True)
    np.testing.assert_allclose(dq, dq_sq[nk - nq:], atol=1e-13)
    np.testing.assert_allclose(dk, dk_sq, atol=1e-13)
    np.testing.assert_allclose(dv, dv_sq, atol=1e-13)


def test_more_queries_than_keys():
    """Nq > Nk: the first Nq - Nk queries see nothing; the rest form a square causal problem."""
    nq, nk, d, scale = 15, 6, 5, 0.6
    q, do = rand((nq, d), 230), rand((nq, d), 231)
    k, v = rand((nk, d), 232), rand((nk, d), 233)
    e = nq - nk
    o, lse = A.forward_head(q, k, v, scale, True)
    assert np.all(o[:e] == 0) and np.all(np.isneginf(lse[:e]))
    o_sq, l_sq = A.forward_head(q[e:], k, v, scale, True)
    np.testing.assert_allclose(o[e:], o_sq, atol=1e-14)
    np.testing.assert_allclose(lse[e:], l_sq, atol=1e-14)
    dq, dk, dv = A.backward_head(q, k, v, do, scale, True)
    dq_sq, dk_sq, dv_sq = A.backward_head(q[e:], k, v, do[e:], scale, True)
    assert np.all(dq[:e] == 0)
    np.testing.assert_allclose(dq[e:], dq_sq, atol=1e-13)
    np.testing.assert_allclose(dk, dk_sq, atol=1e-13)
    np.testing.assert_allclose(dv, dv_sq, atol=1e-13)
    # the sampled helpers agree, empty rows included
    rows = np.array([0, e - 1, e, nq - 1])
    o_r, l_r = A.forward_rows(q, k, v, scale, True, rows)
    np.testing.assert_allclose(o_r, o[rows], atol=1e-14)
    np.testing.assert_array_equal(np.isneginf(l_r), np.isneginf(lse[rows]))
    np.testing.assert_allclose(A.backward_rows(q, k, v, do, scale, True, rows), dq[rows], atol=1e-13)
    cols = np.array([0, 3, nk - 1])
    dk_c, dv_c = A.backward_cols(q, k, v, do, scale, True, cols)
    np.testing.assert_allclose(dk_c, dk[cols], atol=1e-13)
    np.testing.assert_allclose(dv_c, dv[cols], atol=1e-13)


@pytest.mark.parametrize("nq,nk,causal", [(5, 7, False), (5, 7, True), (7, 4, True)])
def test_rectangular_gradients_match_finite_differences(nq, nk, causal):
    d, scale, h = 3, 0.8, 1e-6
    q, do = rand((nq, d), 240), rand((nq, d), 241)
    k, v = rand((nk, d), 242), rand((nk, d), 243)
    grads = A.backward_head(q, k, v, do, scale, causal)

    def f(qq, kk, vv):
        return float(np.sum(do * A.forward_head(qq, kk, vv, scale, causal)[0]))

    for idx, (arr, grad) in enumerate(zip((q, k, v), grads)):
        fd = np.zeros_like(arr)
        for pos in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[pos] += h
            am[pos] -= h
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[idx], args_m[idx] = ap, am
            fd[pos] = (f(*args_p) - f(*args_m)) / (2 * h)
        assert np.linalg.norm(grad - fd) <= 1e-6 * max(np.linalg.norm(fd), 1e-12)


@pytest.mark.parametrize("nq,nk", [(9, 21), (16, 16), (1, 8)])
def test_matches_torch_lower_right_causal_bias(nq, nk):
    """Library special case: PyTorch's float64 SDPA with its lower-right causal bias, plus autograd."""
    torch = pytest.importorskip("torch")
    bias = pytest.importorskip("torch.nn.attention.bias")
    B, H, d, scale = 2, 2, 8, 0.3
    q, do = rand((B, H, nq, d), 250), rand((B, H, nq, d), 251)
    k, v = rand((B, H, nk, d), 252), rand((B, H, nk, d), 253)
    o, _ = A.forward(q, k, v, scale, True)
    dq, dk, dv = A.backward(q, k, v, do, scale, True)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=bias.causal_lower_right(nq, nk), scale=scale)
    to.backward(torch.tensor(do, dtype=torch.float64))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
