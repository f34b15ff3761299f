"""GPU: the autograd entry point and the GPT-3-2.7B-shaped attention sublayer against the oracle.

Bar as for the kernels: max |O - O_ref| <= 1e-2 for the attention output and
relative Frobenius error <= 2e-2 for every gradient; the sublayer (bf16 GEMMs
around the kernels) is held to relative Frobenius <= 2e-2 on its output and on
every gradient.  References are float64 on the CPU: the oracle for attention,
numpy products for the projections, the chain rule written out.
"""

import math

import numpy as np
import pytest

import fa2_inputs as gen
import oracle
from oracle import attention as A

torch = pytest.importorskip("torch")
from exact_tiled_attention_34_amd import fa2  # noqa: E402
from exact_tiled_attention_34_amd.autograd import attention, attention_qkvpacked  # noqa: E402
from exact_tiled_attention_34_amd.gpt_block import AttentionBlock  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
O_TOL, G_TOL = 1e-2, 2e-2


def to_dev(bits, grad=False, dtype="bf16"):
    kind = torch.bfloat16 if dtype == "bf16" else torch.float16
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(kind)
    return t.requires_grad_(grad)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-3))


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", [(2, 2, 150, 150, 64, True), (1, 3, 97, 230, 128, True),
                                                 (2, 1, 200, 120, 80, False), (1, 2, 64, 64, 96, True),
                                                 (1, 2, 150, 190, 256, True)])
def test_autograd_attention_matches_oracle(B, H, Nq, Nk, d, causal):
    arrs = gen.make_arrays_qk(B, H, Nq, Nk, d, seed=4000 + Nq + d)
    q, k, v = (to_dev(arrs[n], grad=True) for n in ("q", "k", "v"))
    do = to_dev(arrs["do"])
    o = attention(q, k, v, causal=causal)
    o.backward(do)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    x = {n: oracle.bf16_bits_to_float64(arrs[n]) for n in ("q", "k", "v", "do")}
    o_ref, _ = A.forward(x["q"], x["k"], x["v"], scale, causal)
    g_ref = A.backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    errs = {"O": float(np.max(np.abs(f64(o) - o_ref)))}
    for n, t, r in zip(("dq", "dk", "dv"), (q, k, v), g_ref):
        errs[n] = rel(f64(t.grad), r)
    print(errs, flush=True)
    assert errs["O"] <= O_TOL and max(errs["dq"], errs["dk"], errs["dv"]) <= G_TOL, errs


def block_reference(x, w_qkv, w_out, dy, heads, causal):
    """Forward and gradients of y = attn(split(x W_qkv)) W_out in float64 (oracle attention)."""
    B, S, h = x.shape
    d = h // heads
    scale = float(np.float32(1.0 / math.sqrt(d)))
    x2 = x.reshape(B * S, h)
    qkv = (x2 @ w_qkv).reshape(B, S, 3, heads, d).transpose(2, 0, 3, 1, 4)   # [3, B, H, S, d]
    o, _ = A.forward(qkv[0], qkv[1], qkv[2], scale, causal)
    a2 = o.transpose(0, 2, 1, 3).reshape(B * S, h)
    y = (a2 @ w_out).reshape(B, S, h)
    dy2 = dy.reshape(B * S, h)
    dw_out = a2.T @ dy2
    do = (dy2 @ w_out.T).reshape(B, S, heads, d).transpose(0, 2, 1, 3)
    dq, dk, dv = A.backward(qkv[0], qkv[1], qkv[2], do, scale, causal)
    dqkv = np.stack([dq, dk, dv]).transpose(1, 3, 0, 2, 4).reshape(B * S, 3 * h)
    return y, {"x": (dqkv @ w_qkv.T).reshape(B, S, h), "w_qkv": x2.T @ dqkv, "w_out": dw_out}


@pytest.mark.parametrize("causal", [True, False])
def test_gpt_shaped_block_matches_reference(causal):
    B, S, hidden, heads = 2, 200, 160, 2          # head dim 80, as in the GPT-3 2.7B shape
    arrs = gen.make_gpt_block(B, S, hidden, seed=11, w_std=0.1)
    x = to_dev(arrs["x"], grad=True)
    w_qkv, w_out = to_dev(arrs["w_qkv"], grad=True), to_dev(arrs["w_out"], grad=True)
    block = AttentionBlock(w_qkv, w_out, heads)
    y = block(x, causal=causal)
    y.backward(to_dev(arrs["dy"]))
    torch.cuda.synchronize()
    ref = {n: oracle.bf16_bits_to_float64(arrs[n]) for n in arrs}
    y_ref, g_ref = block_reference(ref["x"], ref["w_qkv"], ref["w_out"], ref["dy"], heads, causal)
    errs = {"y": rel(f64(y), y_ref), "dx": rel(f64(x.grad), g_ref["x"]),
            "dW_qkv": rel(f64(w_qkv.grad), g_ref["w_qkv"]), "dW_out": rel(f64(w_out.grad), g_ref["w_out"])}
    print(errs, flush=True)
    assert max(errs.values()) <= G_TOL, errs


# ---------------------------------------------------------------------------
# strided layouts: the kernels read and write views, no copies
# ---------------------------------------------------------------------------

def bshd(t):
    """The same values as a [B, N, H, d]-stored tensor, seen as [B, H, N, d]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def padded_rows(t, pad=8):
    """The same values in rows of d + pad elements (row stride d + pad)."""
    B, H, N, d = t.shape
    buf = torch.zeros((B, H, N, d + pad), dtype=t.dtype, device=t.device)
    buf[..., :d] = t
    return buf[..., :d]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", [(2, 3, 140, 140, 128, True), (1, 2, 77, 260, 80, False),
                                                 (2, 2, 200, 90, 64, True), (1, 2, 129, 129, 96, False),
                                                 (1, 2, 100, 100, 256, True)])
def test_strided_views_match_oracle(B, H, Nq, Nk, d, causal):
    arrs = gen.make_arrays_qk(B, H, Nq, Nk, d, seed=5000 + Nq + Nk + d)
    q, k, v, do = (to_dev(arrs[n]) for n in ("q", "k", "v", "do"))
    qs, ks, vs, dos = bshd(q), padded_rows(k), bshd(v), padded_rows(do, 16)
    assert not any(t.is_contiguous() for t in (qs, ks, vs, dos))
    o_buf = torch.empty((B, Nq, H, d), dtype=torch.bfloat16, device=DEV)
    o, lse = fa2.fwd(qs, ks, vs, causal=causal, out=o_buf.transpose(1, 2))
    dq_buf = torch.empty((B, Nq, H, d + 8), dtype=torch.bfloat16, device=DEV)
    dq = dq_buf[..., :d].transpose(1, 2)
    dq, dk, dv = fa2.bwd(qs, ks, vs, o, lse, dos, causal=causal, dq=dq)
    torch.cuda.synchronize()
    # the same call on contiguous tensors gives bitwise the same results
    o_c, lse_c = fa2.fwd(q, k, v, causal=causal)
    g_c = fa2.bwd(q, k, v, o_c, lse_c, do, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous(), o_c) and torch.equal(lse, lse_c)
    for a, b in zip((dq, dk, dv), g_c):
        assert torch.equal(a.contiguous(), b)
    scale = 1.0 / math.sqrt(d)
    x = {n: oracle.bf16_bits_to_float64(arrs[n]) for n in ("q", "k", "v", "do")}
    o_ref, _ = A.forward(x["q"], x["k"], x["v"], scale, causal)
    g_ref = A.backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    assert float(np.max(np.abs(f64(o) - o_ref))) <= O_TOL
    for t, r in zip((dq, dk, dv), g_ref):
        assert rel(f64(t), r) <= G_TOL


@pytest.mark.parametrize("d,causal", [(128, True), (80, False)])
def test_largest_row_pitch(d, causal):
    """Rows 2^20 elements apart (the largest pitch the API accepts), a ragged 70-row sequence: the
    tile copies' byte ranges are largest here.  Results equal the contiguous call's bit for bit."""
    B, H, N = 1, 2, 70
    pitch = 1 << 20
    arrs = gen.make_arrays(B, H, N, d, seed=7100 + d)
    q, k, v, do = (to_dev(arrs[n]) for n in ("q", "k", "v", "do"))
    wide = [padded_rows(t, pitch - d) for t in (q, k, v, do)]
    assert all(t.stride(2) == pitch for t in wide)
    o, lse = fa2.fwd(*wide[:3], causal=causal)
    dq, dk, dv = fa2.bwd(*wide[:3], o, lse, wide[3], causal=causal)
    torch.cuda.synchronize()
    o_c, lse_c = fa2.fwd(q, k, v, causal=causal)
    g_c = fa2.bwd(q, k, v, o_c, lse_c, do, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)
    for a, b in zip((dq, dk, dv), g_c):
        assert torch.equal(a, b)
    with pytest.raises(Exception):
        fa2.fwd(padded_rows(q, pitch + 8 - d), k, v, causal=causal)


@pytest.mark.parametrize("B,S,H,d,causal,dtype", [(2, 150, 2, 80, True, "bf16"), (1, 257, 3, 128, False, "bf16"),
                                                   (2, 64, 4, 64, True, "bf16"), (2, 150, 2, 80, True, "fp16"),
                                                   (1, 130, 2, 256, True, "bf16")])
def test_qkvpacked_matches_oracle(B, S, H, d, causal, dtype):
    arrs = gen.make_arrays(B, H, S, d, seed=6000 + S + d, dtype=dtype)
    qkv_bits = np.stack([arrs[n].transpose(0, 2, 1, 3) for n in ("q", "k", "v")], axis=2)  # [B, S, 3, H, d]
    qkv = to_dev(qkv_bits, grad=True, dtype=dtype)
    do = to_dev(np.ascontiguousarray(arrs["do"].transpose(0, 2, 1, 3)), dtype=dtype)       # [B, S, H, d]
    o = attention_qkvpacked(qkv, causal=causal)
    assert o.shape == (B, S, H, d) and o.is_contiguous()
    o.backward(do)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    x = {n: oracle.bits_to_float64(arrs[n], dtype) for n in ("q", "k", "v", "do")}
    o_ref, _ = A.forward(x["q"], x["k"], x["v"], scale, causal)
    g_ref = A.backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    assert float(np.max(np.abs(f64(o).transpose(0, 2, 1, 3) - o_ref))) <= O_TOL
    g = f64(qkv.grad)
    for j, r in enumerate(g_ref):
        assert rel(g[:, :, j].transpose(0, 2, 1, 3), r) <= G_TOL


def test_strides_of_size_one_dimensions_are_ignored():
    """PyTorch may report any stride for a dimension of size 1; such strides never matter."""
    B, H, N, d = 1, 1, 90, 64
    arrs = gen.make_arrays(B, H, N, d, seed=77)
    q, k, v, do = (to_dev(arrs[n]) for n in ("q", "k", "v", "do"))
    odd = [torch.as_strided(t, (B, H, N, d), (7, 3, d, 1)) for t in (q, k, v)]
    assert not odd[0].is_contiguous() or odd[0].stride(0) == 7
    o, lse = fa2.fwd(*odd, causal=True)
    o_c, lse_c = fa2.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)
