"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Bar (fixed for this path): max |O_gpu - O_ref| <= 1e-2, max |L_gpu - L_ref| <= 1e-3,
and ||g_gpu - g_ref||_F / ||g_ref||_F <= 2e-2 for g in dQ, dK, dV.  The GPU
backward consumes the GPU forward's O and L; the oracle recomputes everything
from the same bf16 inputs.

Small shapes are compared element by element against the full oracle.  The
full-size workloads run exactly as bench.py runs them (same entry points and
shapes) and are compared on sampled query rows and key columns of a few heads,
plus properties that hold at any size.
"""

import math

import numpy as np
import pytest

import fa2_inputs as gen
import oracle
from oracle import attention as A

torch = pytest.importorskip("torch")
from exact_tiled_attention_34_amd import fa2  # noqa: E402

pytestmark = pytest.mark.gpu

O_TOL, L_TOL, G_TOL = 1e-2, 1e-3, 2e-2
DEV = "cuda:0"


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def frob_rel(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def run_gpu(arrs, causal, scale):
    q, k, v, do = (to_dev(arrs[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa2.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return {n: t for n, t in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv))}


def decode(arrs):
    return {n: oracle.bf16_bits_to_float64(arrs[n]) for n in ("q", "k", "v", "do")}


def assert_full_parity(arrs, causal, scale, label=""):
    out = run_gpu(arrs, causal, scale)
    x = decode(arrs)
    o_ref, l_ref = A.forward(x["q"], x["k"], x["v"], scale, causal)
    dq_ref, dk_ref, dv_ref = A.backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    o, lse = to_f64(out["o"]), to_f64(out["lse"])
    errs = {
        "O": float(np.max(np.abs(o - o_ref))),
        "L": float(np.max(np.abs(lse - l_ref))),
        "dQ": frob_rel(to_f64(out["dq"]), dq_ref),
        "dK": frob_rel(to_f64(out["dk"]), dk_ref),
        "dV": frob_rel(to_f64(out["dv"]), dv_ref),
    }
    print(label, errs, flush=True)
    assert errs["O"] <= O_TOL, errs
    assert errs["L"] <= L_TOL, errs
    assert errs["dQ"] <= G_TOL and errs["dK"] <= G_TOL and errs["dV"] <= G_TOL, errs
    return out, errs


# ---------------------------------------------------------------------------
# small shapes, every element
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 1, 1), (1, 1, 12), (1, 2, 64), (2, 1, 127), (1, 1, 128),
                                   (1, 2, 129), (2, 2, 200), (1, 1, 256), (1, 1, 333)])
def test_small_shapes(d, causal, B, H, N):
    arrs = gen.make_arrays(B, H, N, d, seed=1000 + N + d)
    assert_full_parity(arrs, causal, 1.0 / math.sqrt(d), f"B{B} H{H} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("scale", [0.05, 0.5])
def test_other_scales(scale):
    arrs = gen.make_arrays(1, 2, 190, 64, seed=7)
    assert_full_parity(arrs, True, scale, f"scale={scale}")


def test_workload_c1_every_element():
    w, arrs = gen.make_workload("c1")
    assert_full_parity(arrs, w.causal, w.scale, w.name)


# ---------------------------------------------------------------------------
# full-size workloads: sampled rows/columns + size-independent properties
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_workload_full_size_sampled(key):
    w, arrs = gen.make_workload(key)
    print(f"workload {key}: {w.name}", flush=True)
    out = run_gpu(arrs, w.causal, w.scale)
    o_g = out["o"].float()
    l_g = out["lse"]
    # finite everywhere
    for n, t in out.items():
        assert torch.isfinite(t.float()).all(), n
    rng = np.random.default_rng(11)
    B, H, N, d = w.B, w.H, w.N, w.d
    heads = [(0, 0), (B - 1, H - 1)]
    worst = {"O": 0.0, "L": 0.0, "dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for b, h in heads:
        xq, xk, xv, xdo = (oracle.bf16_bits_to_float64(arrs[n][b, h]) for n in ("q", "k", "v", "do"))
        rows = np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 13)]))
        if arrs["spike_rows"] is not None:
            rows = np.unique(np.append(rows, arrs["spike_rows"][b, h]))
        cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 14)]))
        o_ref, l_ref = A.forward_rows(xq, xk, xv, w.scale, w.causal, rows)
        stats = A.row_stats(xq, xk, xv, xdo, w.scale, w.causal)
        dq_ref = A.backward_rows(xq, xk, xv, xdo, w.scale, w.causal, rows)
        dk_ref, dv_ref = A.backward_cols(xq, xk, xv, xdo, w.scale, w.causal, cols, stats=stats)
        o = to_f64(out["o"][b, h, torch.as_tensor(rows, device=DEV)])
        lse = to_f64(out["lse"][b, h, torch.as_tensor(rows, device=DEV)])
        dq = to_f64(out["dq"][b, h, torch.as_tensor(rows, device=DEV)])
        dk = to_f64(out["dk"][b, h, torch.as_tensor(cols, device=DEV)])
        dv = to_f64(out["dv"][b, h, torch.as_tensor(cols, device=DEV)])
        worst["O"] = max(worst["O"], float(np.max(np.abs(o - o_ref))))
        worst["L"] = max(worst["L"], float(np.max(np.abs(lse - l_ref))))
        worst["dQ"] = max(worst["dQ"], frob_rel(dq, dq_ref))
        worst["dK"] = max(worst["dK"], frob_rel(dk, dk_ref))
        worst["dV"] = max(worst["dV"], frob_rel(dv, dv_ref))
    print(key, "sampled errors", worst, flush=True)
    assert worst["O"] <= O_TOL and worst["L"] <= L_TOL, worst
    assert worst["dQ"] <= G_TOL and worst["dK"] <= G_TOL and worst["dV"] <= G_TOL, worst

    # properties at full size: O rows are convex combinations of V rows, so each
    # column of O lies within [min V, max V] of that column (bf16 rounding slack)
    v_g = to_dev(arrs["v"]).float()
    vmin = v_g.amin(dim=2, keepdim=True)
    vmax = v_g.amax(dim=2, keepdim=True)
    slack = 1e-2
    assert bool(((o_g >= vmin - slack) & (o_g <= vmax + slack)).all())
    # L_i >= the scaled score of the diagonal (causal) or of key 0 (any mask)
    q_g = to_dev(arrs["q"]).float()
    k_g = to_dev(arrs["k"]).float()
    s0 = w.scale * (q_g * k_g[:, :, :1, :]).sum(-1)
    assert bool((l_g >= s0 - 1e-3).all())
    # sum_j dV_j = sum_i dO_i per (b, h)   (rows of P sum to one)
    dv_sum = out["dv"].float().sum(dim=2)
    do_sum = to_dev(arrs["do"]).float().sum(dim=2)
    rel = (dv_sum - do_sum).norm() / do_sum.norm()
    assert float(rel) <= G_TOL, float(rel)


# ---------------------------------------------------------------------------
# closed forms on the GPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_give_mean_of_v(d, causal):
    N = 300
    arrs = gen.make_arrays(1, 2, N, d, seed=21)
    arrs["q"] = np.zeros_like(arrs["q"])
    out = run_gpu(arrs, causal, 1.0 / math.sqrt(d))
    v = oracle.bf16_bits_to_float64(arrs["v"])
    if causal:
        want_o = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        want_l = np.broadcast_to(np.log(np.arange(1, N + 1)), (1, 2, N))
    else:
        want_o = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        want_l = np.full((1, 2, N), np.log(N))
    assert np.max(np.abs(to_f64(out["o"]) - want_o)) <= O_TOL
    assert np.max(np.abs(to_f64(out["lse"]) - want_l)) <= L_TOL
    # Q = 0: dK = scale dS^T Q = 0 exactly
    assert float(out["dk"].float().abs().max()) == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_ones(causal):
    arrs = gen.make_arrays(1, 1, 257, 128, seed=22)
    arrs["v"] = np.full_like(arrs["v"], 0x3F80)  # 1.0
    out = run_gpu(arrs, causal, 1.0 / math.sqrt(128))
    assert np.max(np.abs(to_f64(out["o"]) - 1.0)) <= 4e-3


@pytest.mark.parametrize("d", [64, 80, 128])
def test_single_token_and_causal_row0(d):
    arrs = gen.make_arrays(2, 3, 1, d, seed=23)
    out = run_gpu(arrs, True, 1.0 / math.sqrt(d))
    x = decode(arrs)
    np.testing.assert_array_equal(to_f64(out["o"]), x["v"])
    np.testing.assert_array_equal(to_f64(out["dv"]), x["do"])
    assert float(out["dq"].float().abs().max()) == 0.0
    assert float(out["dk"].float().abs().max()) == 0.0
    arrs = gen.make_arrays(1, 2, 150, d, seed=24)
    out = run_gpu(arrs, True, 1.0 / math.sqrt(d))
    x = decode(arrs)
    np.testing.assert_array_equal(to_f64(out["o"])[:, :, 0], x["v"][:, :, 0])
    l0 = (1.0 / math.sqrt(d)) * np.sum(x["q"][:, :, 0] * x["k"][:, :, 0], axis=-1)
    assert np.max(np.abs(to_f64(out["lse"])[:, :, 0] - l0)) <= L_TOL


# ---------------------------------------------------------------------------
# causal isolation, poison fill, determinism, errors
# ---------------------------------------------------------------------------

def test_causal_isolation_is_bitwise():
    """Rows i never read keys/values j > i: perturbing those leaves O_i, L_i bit-identical."""
    N, d = 300, 128
    arrs = gen.make_arrays(1, 1, N, d, seed=25)
    base = run_gpu(arrs, True, 1.0 / math.sqrt(d))
    for i in (0, 63, 64, 127, 200):
        pert = dict(arrs)
        noise = gen.make_arrays(1, 1, N, d, seed=26 + i)
        for n in ("k", "v"):
            a = arrs[n].copy()
            a[:, :, i + 1:] = noise[n][:, :, i + 1:]
            pert[n] = a
        out = run_gpu(pert, True, 1.0 / math.sqrt(d))
        assert torch.equal(out["o"][:, :, : i + 1], base["o"][:, :, : i + 1]), i
        assert torch.equal(out["lse"][:, :, : i + 1], base["lse"][:, :, : i + 1]), i


@pytest.mark.parametrize("d", [64, 80, 128])
def test_every_output_element_written(d):
    B, H, N = 1, 3, 333
    arrs = gen.make_arrays(B, H, N, d, seed=27)
    q, k, v, do = (to_dev(arrs[n]) for n in ("q", "k", "v", "do"))
    nan16 = torch.full((B, H, N, d), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)  # 0xFFFF = NaN
    o = nan16.clone()
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    fa2.fwd(q, k, v, causal=True, out=o, lse=lse)
    dq, dk, dv = nan16.clone(), nan16.clone(), nan16.clone()
    ws = torch.full((fa2.bwd_workspace_bytes(B, H, N, d),), 0xFF, dtype=torch.uint8, device=DEV)
    fa2.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all()


def test_run_to_run_determinism():
    w, arrs = gen.make_workload("c1")
    arrs = gen.make_arrays(2, 4, 1000, 128, seed=28)
    a = run_gpu(arrs, True, 1.0 / math.sqrt(128))
    b = run_gpu(arrs, True, 1.0 / math.sqrt(128))
    for n in ("o", "lse", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n
    # dQ accumulates with atomics: the summation order may differ
    assert frob_rel(to_f64(a["dq"]), to_f64(b["dq"])) <= 1e-2


def test_errors_raise():
    q = torch.zeros((1, 1, 16, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa2.FA2Error) as e:
        fa2.fwd(q, q.clone(), q.clone())
    assert e.value.status == 2
    q = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa2.FA2Error) as e:
        fa2.fwd(q, q.clone(), q.clone(), scale=-1.0)
    assert e.value.status == 1
    with pytest.raises(ValueError):
        fa2.fwd(q.float(), q, q)
