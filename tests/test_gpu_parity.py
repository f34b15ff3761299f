"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Bar (fixed for this path): max |O_gpu - O_ref| <= 1e-2, max |L_gpu - L_ref| <= 1e-3,
and ||g_gpu - g_ref||_F / ||g_ref||_F <= 2e-2 for g in dQ, dK, dV.  The GPU
backward consumes the GPU forward's O and L; the oracle recomputes everything
from the same bf16 inputs.

Small shapes are compared element by element against the full oracle.  The
full-size workloads run exactly as bench.py runs them (same entry points and
shapes) and are compared with the oracle on every (batch, head): O and L
element by element, dQ, dK, dV by the Frobenius norm of the whole tensors
(tests/fullsize.py), plus properties that hold at any size.  The largest
tensors the ABI accepts (2^31 elements) are checked on sampled rows and
columns of three heads and on the any-size properties.
"""

import math

import numpy as np
import pytest

import fa2_inputs as gen
import oracle
from oracle import attention as A
from fullsize import compare_all_heads

torch = pytest.importorskip("torch")
from exact_tiled_attention_34_amd import fa2  # noqa: E402

pytestmark = pytest.mark.gpu

O_TOL, L_TOL, G_TOL = 1e-2, 1e-3, 2e-2
DEV = "cuda:0"


def to_dev(bits, dtype="bf16"):
    kind = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(kind)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def frob_rel(got, ref):
    """||got - ref||_F / ||ref||_F.  Where the exact reference is zero (a single
    token has zero dQ and dK) a relative norm is undefined; the denominator is
    then floored at 1e-3, turning the bar into ||got||_F <= 2e-5."""
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-3))


def run_gpu(arrs, causal, scale, dtype="bf16"):
    q, k, v, do = (to_dev(arrs[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa2.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return {n: t for n, t in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv))}


def decode(arrs, dtype="bf16"):
    return {n: oracle.bits_to_float64(arrs[n], dtype) for n in ("q", "k", "v", "do")}


def assert_full_parity(arrs, causal, scale, label="", dtype="bf16"):
    out = run_gpu(arrs, causal, scale, dtype)
    x = decode(arrs, dtype)
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

@pytest.mark.parametrize("d", [64, 80, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 1, 1), (1, 1, 12), (1, 2, 64), (2, 1, 127), (1, 1, 128),
                                   (1, 2, 129), (2, 2, 200), (1, 1, 256), (1, 1, 333),
                                   (1, 2, 520), (1, 1, 777)])
def test_small_shapes(d, causal, B, H, N):
    arrs = gen.make_arrays(B, H, N, d, seed=1000 + N + d)
    assert_full_parity(arrs, causal, 1.0 / math.sqrt(d), f"B{B} H{H} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("scale", [0.05, 0.5])
def test_other_scales(scale):
    arrs = gen.make_arrays(1, 2, 190, 64, seed=7)
    assert_full_parity(arrs, True, scale, f"scale={scale}")


# Query and key lengths that differ (causal mask aligned bottom-right): decode
# (one query), a short query block against a long key/value cache, more
# queries than keys (the first Nq - Nk rows see nothing: O = 0, L = -inf,
# dQ = 0), ragged tails on both sides, all three head dimensions.
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk,d", [(1, 2, 1, 300, 128), (2, 1, 1, 64, 64), (1, 2, 77, 500, 64),
                                         (1, 1, 64, 1000, 128), (2, 2, 300, 130, 80),
                                         (1, 2, 513, 200, 128), (1, 1, 129, 257, 80),
                                         (1, 2, 150, 270, 96), (1, 1, 1, 1, 64), (2, 1, 70, 1, 128),
                                         (1, 3, 200, 333, 128), (1, 2, 600, 190, 64), (1, 1, 800, 300, 96),
                                         (1, 2, 77, 500, 256), (2, 1, 300, 130, 256), (1, 1, 1, 200, 256)])
def test_separate_query_and_key_lengths(causal, B, H, Nq, Nk, d):
    arrs = gen.make_arrays_qk(B, H, Nq, Nk, d, seed=3000 + Nq + Nk + d)
    label = f"B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal}"
    out = run_gpu(arrs, causal, 1.0 / math.sqrt(d))
    x = decode(arrs)
    o_ref, l_ref = A.forward(x["q"], x["k"], x["v"], 1.0 / math.sqrt(d), causal)
    g_ref = A.backward(x["q"], x["k"], x["v"], x["do"], 1.0 / math.sqrt(d), causal)
    o, lse = to_f64(out["o"]), to_f64(out["lse"])
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), label   # exactly the rows that see no key
    assert np.all(o[empty] == 0) and np.all(to_f64(out["dq"])[empty] == 0), label
    errs = {"O": float(np.max(np.abs(o - o_ref))),
            "L": float(np.max(np.abs(lse[~empty] - l_ref[~empty]))) if (~empty).any() else 0.0}
    for n, r in zip(("dq", "dk", "dv"), g_ref):
        errs[n] = frob_rel(to_f64(out[n]), r)
    print(label, errs, flush=True)
    assert errs["O"] <= O_TOL and errs["L"] <= L_TOL, errs
    assert max(errs["dq"], errs["dk"], errs["dv"]) <= G_TOL, errs


# float16 storage: the same kernels with the f16 matrix instruction, through the
# strided entry points (contiguous, [B, N, H, d] views, Nq != Nk)
@pytest.mark.parametrize("d", [64, 80, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 1, 12), (2, 2, 200), (1, 1, 333)])
def test_fp16_small_shapes(d, causal, B, H, N):
    arrs = gen.make_arrays(B, H, N, d, seed=7000 + N + d, dtype="fp16")
    out, _ = assert_full_parity(arrs, causal, 1.0 / math.sqrt(d), f"fp16 B{B} H{H} N{N} d{d} causal={causal}",
                                dtype="fp16")
    assert all(t.dtype == torch.float16 for n, t in out.items() if n != "lse")


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", [(1, 2, 77, 300, 128, True), (2, 2, 250, 100, 80, True),
                                                 (1, 3, 130, 130, 64, False), (1, 2, 1500, 2100, 128, True),
                                                 (2, 1, 1024, 1024, 96, False), (1, 2, 300, 420, 256, True)])
def test_fp16_views_and_lengths(B, H, Nq, Nk, d, causal):
    arrs = gen.make_arrays_qk(B, H, Nq, Nk, d, seed=7100 + Nq + Nk, dtype="fp16")
    q, k, v, do = (to_dev(arrs[n], "fp16") for n in ("q", "k", "v", "do"))
    qs, vs = q.transpose(1, 2).contiguous().transpose(1, 2), v.transpose(1, 2).contiguous().transpose(1, 2)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa2.fwd(qs, k, vs, causal=causal, scale=scale)
    dq, dk, dv = fa2.bwd(qs, k, vs, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    x = decode(arrs, "fp16")
    o_ref, l_ref = A.forward(x["q"], x["k"], x["v"], scale, causal)
    g_ref = A.backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    empty = np.isneginf(l_ref)
    lse64 = to_f64(lse)
    assert np.array_equal(np.isneginf(lse64), empty)
    assert float(np.max(np.abs(to_f64(o) - o_ref))) <= O_TOL
    if (~empty).any():
        assert float(np.max(np.abs(lse64[~empty] - l_ref[~empty]))) <= L_TOL
    for t, r in zip((dq, dk, dv), g_ref):
        assert frob_rel(to_f64(t), r) <= G_TOL


def test_mixed_16bit_types_rejected():
    q = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa2.fwd(q, q.half(), q)


def test_workload_c1_every_element():
    w, arrs = gen.make_workload("c1")
    assert_full_parity(arrs, w.causal, w.scale, w.name)


# ---------------------------------------------------------------------------
# full-size workloads: every head against the oracle, whole-tensor bar
# ---------------------------------------------------------------------------

def to_host(out):
    return {n: t.float().cpu().numpy() for n, t in out.items()}


def assert_whole_tensor_parity(label, out, arrs, w, dtype="bf16"):
    """The bar over whole tensors (every (batch, head) pair against the oracle)."""
    errs = compare_all_heads(to_host(out), arrs, w.scale, w.causal, dtype=dtype)
    print(f"{label} whole tensors: O {errs['O']:.3e} (vs the oracle rounded to {dtype}: "
          f"{errs['O_vs_rounded']:.3e})  L {errs['L']:.3e}  dQ {errs['dQ']:.3e}  dK {errs['dK']:.3e}  "
          f"dV {errs['dV']:.3e}; worst heads {errs['worst_head']}; {errs['workers']} oracle workers",
          flush=True)
    assert errs["O"] <= O_TOL and errs["L"] <= L_TOL, errs
    assert errs["dQ"] <= G_TOL and errs["dK"] <= G_TOL and errs["dV"] <= G_TOL, errs
    return errs


def assert_any_size_properties(key, out, arrs, dtype="bf16"):
    """Properties that hold at any size, on every head: O rows inside the hull of
    V's rows, L at least the score of key 0, rows of P summing to one
    (sum_j dV_j = sum_i dO_i), sum_j dK_j = 0."""
    o_g = out["o"].float()
    v_g = to_dev(arrs["v"], dtype).float()
    slack = 1e-2   # O rows are convex combinations of V rows (16-bit rounding slack)
    inside = bool(((o_g >= v_g.amin(dim=2, keepdim=True) - slack)
                   & (o_g <= v_g.amax(dim=2, keepdim=True) + slack)).all())
    assert inside, "O outside the convex hull of V"
    del o_g, v_g
    q_g = to_dev(arrs["q"], dtype).float()
    k_g = to_dev(arrs["k"], dtype).float()
    s0 = (q_g * k_g[:, :, :1, :]).sum(-1) * float(out["scale"])   # key 0 is visible to every query
    l_ok = bool((out["lse"] >= s0 - 1e-3).all())
    assert l_ok, "L below the score of a visible key"
    del q_g, k_g, s0
    dv_sum = out["dv"].float().sum(dim=2)
    do_sum = to_dev(arrs["do"], dtype).float().sum(dim=2)
    rel = float((dv_sum - do_sum).norm() / do_sum.norm())
    assert rel <= G_TOL, rel
    dk_sum = out["dk"].float().sum(dim=2)
    rel_k = float(dk_sum.norm() / out["dk"].float().norm(dim=(2, 3)).norm())
    print(f"{key} all heads: sum dV vs sum dO {rel:.2e}, |sum dK| / |dK| {rel_k:.2e}", flush=True)
    assert rel_k <= G_TOL, rel_k


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_workload_full_size(key):
    """The full-size workloads exactly as bench.py runs them: every (batch, head)
    against the oracle, O and L element by element and dQ, dK, dV by the
    Frobenius norm of the whole tensors; the x8 spike rows of the range-stress
    workload are among the rows checked."""
    w, arrs = gen.make_workload(key)
    print(f"workload {key}: {w.name}", flush=True)
    out = run_gpu(arrs, w.causal, w.scale)
    for n, t in out.items():
        ok = bool(torch.isfinite(t.float()).all())
        assert ok, f"non-finite values in {n}"
    assert_whole_tensor_parity(key, out, arrs, w)
    if arrs["spike_rows"] is not None:
        # diagnostic: a near one-hot row (the x8 spike) has a tiny dQ whose relative
        # error is dominated by the rounding of O inside delta = rowsum(dO * O)
        b, h = w.B - 1, w.H - 1
        x = {n: oracle.bf16_bits_to_float64(arrs[n][b, h]) for n in ("q", "k", "v", "do")}
        rows = np.array([arrs["spike_rows"][b, h]])
        dq_ref = A.backward_rows(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal, rows)
        print(f"{key} spike row {rows[0]} of head ({b},{h}): dQ rel "
              f"{frob_rel(to_f64(out['dq'][b, h, rows[0]]), dq_ref[0]):.3e}", flush=True)
    out["scale"] = w.scale
    assert_any_size_properties(key, out, arrs)


@pytest.mark.parametrize("B,H,N,causal", [(1, 4, 4096, True), (2, 2, 2000, False)])
def test_head_dim_256_long(B, H, N, causal):
    """Head dimension 256 at a long sequence (many key and query blocks per head,
    a ragged tail in the second case): every head against the oracle."""
    d = 256
    arrs = gen.make_arrays(B, H, N, d, seed=2560 + N)
    w = gen.Workload("d256", f"B{B} H{H} N{N} d256", B, H, N, d, causal)
    out = run_gpu(arrs, causal, w.scale)
    assert_whole_tensor_parity(f"d256 B{B} H{H} N{N} causal={causal}", out, arrs, w)
    out["scale"] = w.scale
    assert_any_size_properties("d256", out, arrs)


# ---------------------------------------------------------------------------
# closed forms on the GPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 80, 96, 128, 256])
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
    err_o = float(np.max(np.abs(to_f64(out["o"]) - want_o)))
    err_l = float(np.max(np.abs(to_f64(out["lse"]) - want_l)))
    assert err_o <= O_TOL, err_o
    assert err_l <= L_TOL, err_l
    # Q = 0: dK = scale dS^T Q = 0 exactly
    dk_max = float(out["dk"].float().abs().max())
    assert dk_max == 0.0, dk_max


# Per-head score growth per 64 keys for test_growing_scores: the running row
# maximum climbs by 12 (far past the 2^8 bound on P, every tile), 6 and 3 (P
# sums past 2^8 on some tiles, no single P near it), 0.5 (never past it after
# the first tile) and falls by 3.
GROWTH = (12.0, 6.0, 3.0, 0.5, -3.0)


@pytest.mark.parametrize("d", [64, 80, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores(d, causal):
    """Scores that ramp along the keys: the forward's softmax must move each
    row's reference maximum tile after tile (and, where P against the old
    reference is first tried, fall back to the maximum pass on exactly the
    tiles that need it).  Q = u + Q0/4 and K_j = t_j sqrt(d) u/|u|^2 + K0/4 for
    a head's first query u, so the scores are about t_j = g j / 64 plus noise.

    O and L are compared element by element.  The gradients are not: with keys
    of norm up to ~t_j and a nearly one-hot softmax, dQ = scale sum_j dS_ij K_j
    cancels almost completely, so the rounding of dS to the storage type alone
    (relative 2^-9, times t_j ~ 80) moves dQ by several per cent of its norm;
    no backward kernel depends on how the forward reached its maximum."""
    N, H = 333, len(GROWTH)
    arrs = gen.make_arrays(1, H, N, d, seed=31 + d)
    x = decode(arrs)
    u = x["q"][:, :, :1, :]
    t = np.array(GROWTH)[None, :, None, None] * np.arange(N)[None, None, :, None] / 64.0
    q = u + 0.25 * x["q"]
    k = t * math.sqrt(d) * u / np.sum(u * u, axis=-1, keepdims=True) + 0.25 * x["k"]
    arrs["q"] = gen.round_to_bf16_bits(q.astype(np.float32))
    arrs["k"] = gen.round_to_bf16_bits(k.astype(np.float32))
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = (to_dev(arrs[n]) for n in ("q", "k", "v"))
    o, lse = fa2.fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    x = decode(arrs)
    o_ref, l_ref = A.forward(x["q"], x["k"], x["v"], scale, causal)
    err_o = float(np.max(np.abs(to_f64(o) - o_ref)))
    err_l = float(np.max(np.abs(to_f64(lse) - l_ref)))
    print(f"growing scores d{d} causal={causal}: O {err_o:.3g} L {err_l:.3g}", flush=True)
    assert err_o <= O_TOL, err_o
    assert err_l <= L_TOL, err_l


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_ones(causal):
    arrs = gen.make_arrays(1, 1, 257, 128, seed=22)
    arrs["v"] = np.full_like(arrs["v"], 0x3F80)  # 1.0
    out = run_gpu(arrs, causal, 1.0 / math.sqrt(128))
    err = float(np.max(np.abs(to_f64(out["o"]) - 1.0)))
    assert err <= 4e-3, err


@pytest.mark.parametrize("d", [64, 80, 96, 128, 256])
def test_single_token_and_causal_row0(d):
    arrs = gen.make_arrays(2, 3, 1, d, seed=23)
    out = run_gpu(arrs, True, 1.0 / math.sqrt(d))
    x = decode(arrs)
    np.testing.assert_array_equal(to_f64(out["o"]), x["v"])
    np.testing.assert_array_equal(to_f64(out["dv"]), x["do"])
    # exact answer 0; delta and dP are two fp32 sums of the same products in a
    # different order, so only rounding noise may remain
    dq_max = float(out["dq"].float().abs().max())
    dk_max = float(out["dk"].float().abs().max())
    assert dq_max <= 1e-5 and dk_max <= 1e-5, (dq_max, dk_max)
    arrs = gen.make_arrays(1, 2, 150, d, seed=24)
    out = run_gpu(arrs, True, 1.0 / math.sqrt(d))
    x = decode(arrs)
    np.testing.assert_array_equal(to_f64(out["o"])[:, :, 0], x["v"][:, :, 0])
    l0 = (1.0 / math.sqrt(d)) * np.sum(x["q"][:, :, 0] * x["k"][:, :, 0], axis=-1)
    err = float(np.max(np.abs(to_f64(out["lse"])[:, :, 0] - l0)))
    assert err <= L_TOL, err


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
        same_o = torch.equal(out["o"][:, :, : i + 1], base["o"][:, :, : i + 1])
        same_l = torch.equal(out["lse"][:, :, : i + 1], base["lse"][:, :, : i + 1])
        assert same_o and same_l, i


@pytest.mark.parametrize("d", [64, 80, 96, 128, 256])
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
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        finite = bool(torch.isfinite(t.float()).all())
        assert finite, f"{name} has unwritten (NaN) elements"


@pytest.mark.parametrize("d", [64, 80, 96, 128, 256])
def test_run_to_run_determinism(d):
    """No kernel accumulates with atomics (dQ has its own pass), so every output,
    dQ included, is bit-identical from run to run."""
    arrs = gen.make_arrays(2, 4, 1000, d, seed=28)
    a = run_gpu(arrs, True, 1.0 / math.sqrt(d))
    b = run_gpu(arrs, True, 1.0 / math.sqrt(d))
    for n in ("o", "lse", "dq", "dk", "dv"):
        same = torch.equal(a[n], b[n])
        assert same, n


def test_errors_raise():
    q = torch.zeros((1, 1, 16, 112), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa2.FA2Error) as e:
        fa2.fwd(q, q.clone(), q.clone())
    assert e.value.status == 2
    q = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa2.FA2Error) as e:
        fa2.fwd(q, q.clone(), q.clone(), scale=-1.0)
    assert e.value.status == 1
    with pytest.raises(ValueError):
        fa2.fwd(q.float(), q, q)


@pytest.mark.parametrize("d,causal,N", [(64, True, 200), (80, False, 129), (96, True, 150), (128, True, 333),
                                        (256, True, 333), (256, False, 200)])
def test_phases_compose_to_bwd(d, causal, N):
    """fa2_bwd == preprocess + dkdv + dq called one by one (the way bench.py times them)."""
    B, H = 2, 2
    arrs = gen.make_arrays(B, H, N, d, seed=31)
    q, k, v, do = (to_dev(arrs[n]) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
    dq_a, dk_a, dv_a = fa2.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    delta, lse2 = fa2.bwd_row_arrays(B, H, N, q.device)
    dq_b, dk_b, dv_b = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    fa2.bwd_preprocess(o, do, lse, delta, lse2)
    fa2.bwd_dkdv(q, k, v, do, lse2, delta, dk_b, dv_b, causal=causal, scale=scale)
    fa2.bwd_dq(q, k, v, do, lse2, delta, dq_b, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for name, a, b in (("dq", dq_a, dq_b), ("dk", dk_a, dk_b), ("dv", dv_a, dv_b)):
        same = torch.equal(a, b)
        assert same, name
    npad = fa2.bwd_rows_padded(N)
    assert tuple(delta.shape) == (B, H, npad)
    pad_delta = float(delta[:, :, N:].abs().max()) if npad > N else 0.0
    pad_inf = bool(torch.isinf(lse2[:, :, N:]).all()) if npad > N else True
    assert pad_delta == 0.0 and pad_inf
    rel = float(((lse2[:, :, :N] - lse * math.log2(math.e)).abs() / lse.abs().clamp_min(1e-3)).max())
    assert rel <= 1e-6, rel


def head_bits(t, b, h):
    """Exact uint16 bit patterns of head (b, h) of a 16-bit device tensor."""
    return t[b, h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_maximum_element_count():
    """The largest tensors the ABI accepts: B*H*N*d just under 2^31 elements (4 GiB per
    bf16 tensor, so byte offsets pass 2^31), a ragged N, causal.  Sampled rows and
    columns of the first, a middle and the last head against the oracle; properties
    that hold at any size on every head."""
    B, H, N, d = 8, 128, 16383, 128
    assert B * H * N * d < 2 ** 31 and 2 * B * H * N * d > 2 ** 31 + 2 ** 30
    causal, scale = True, 1.0 / math.sqrt(d)
    print(f"maximum size: B={B} H={H} N={N} d={d} causal", flush=True)
    x = gen.make_device_tensors(B, H, N, d, seed=7, device=DEV)
    o, lse = fa2.fwd(x["q"], x["k"], x["v"], causal=causal, scale=scale)
    dq, dk, dv = fa2.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"non-finite values in {name}"

    rng = np.random.default_rng(5)
    for b, h, with_cols in [(0, 0, True), (3, 77, False), (B - 1, H - 1, True)]:
        xh = {n: oracle.bf16_bits_to_float64(head_bits(x[n], b, h)) for n in ("q", "k", "v", "do")}
        rows = np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 13)]))
        o_ref, l_ref = A.forward_rows(xh["q"], xh["k"], xh["v"], scale, causal, rows)
        dq_ref = A.backward_rows(xh["q"], xh["k"], xh["v"], xh["do"], scale, causal, rows)
        ri = torch.as_tensor(rows, device=DEV)
        errs = {
            "O": float(np.max(np.abs(to_f64(o[b, h, ri]) - o_ref))),
            "L": float(np.max(np.abs(to_f64(lse[b, h, ri]) - l_ref))),
            "dQ_rows": frob_rel(to_f64(dq[b, h, ri]), dq_ref),
        }
        if with_cols:
            cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 14)]))
            stats = A.row_stats(xh["q"], xh["k"], xh["v"], xh["do"], scale, causal)
            dk_ref, dv_ref = A.backward_cols(xh["q"], xh["k"], xh["v"], xh["do"], scale, causal, cols,
                                             stats=stats)
            ci = torch.as_tensor(cols, device=DEV)
            errs["dK_cols"] = frob_rel(to_f64(dk[b, h, ci]), dk_ref)
            errs["dV_cols"] = frob_rel(to_f64(dv[b, h, ci]), dv_ref)
        print(f"maximum size, head ({b},{h}):", errs, flush=True)
        assert errs["O"] <= O_TOL and errs["L"] <= L_TOL, errs
        assert all(v <= G_TOL for k, v in errs.items() if k not in ("O", "L")), errs

    # every head: O inside the hull of V; rows of P sum to one (sum_j dV_j = sum_i dO_i);
    # sum_j dK_j = 0
    for b in range(B):
        o_g, v_g = o[b].float(), x["v"][b].float()
        assert bool(((o_g >= v_g.amin(dim=1, keepdim=True) - 1e-2)
                     & (o_g <= v_g.amax(dim=1, keepdim=True) + 1e-2)).all()), b
        dv_sum, do_sum = dv[b].float().sum(dim=1), x["do"][b].float().sum(dim=1)
        assert float((dv_sum - do_sum).norm() / do_sum.norm()) <= G_TOL, b
        dk_b = dk[b].float()
        assert float(dk_b.sum(dim=1).norm() / dk_b.norm(dim=(1, 2)).norm()) <= G_TOL, b
        del o_g, v_g, dk_b


@pytest.mark.parametrize("key", ["c2", "c4"])
def test_workload_full_size_fp16(key):
    """The full-size workloads with float16 storage: every (batch, head) against the
    oracle (whole-tensor bar) and the any-size properties on every head."""
    w = gen.WORKLOADS[key]
    arrs = gen.make_arrays(w.B, w.H, w.N, w.d, seed=1, sigma=w.sigma, spike=w.spike, dtype="fp16")
    print(f"workload {key} fp16: {w.name}", flush=True)
    out = run_gpu(arrs, w.causal, w.scale, dtype="fp16")
    for n, t in out.items():
        assert bool(torch.isfinite(t.float()).all()), f"non-finite values in {n}"
    assert_whole_tensor_parity(f"{key} fp16", out, arrs, w, dtype="fp16")
    out["scale"] = w.scale
    assert_any_size_properties(f"{key} fp16", out, arrs, dtype="fp16")
