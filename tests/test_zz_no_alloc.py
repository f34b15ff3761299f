"""The allocation-free backward (fa2_bwd_qk_noalloc, the library's fixed device
scratch instead of a workspace) against the backward with a caller workspace
(fa2_bwd / fa2_bwd_qk): the same kernels, so the outputs must be bit-identical,
on calls in a row whose sizes shrink (the scratch keeps the previous call's
contents), plus the oracle's bar on one of them."""

import math

import numpy as np
import pytest

import fa2_inputs as gen
import oracle
from oracle import attention as A

torch = pytest.importorskip("torch")
from exact_tiled_attention_34_amd import fa2  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def both_ways(B, H, Nq, Nk, d, causal, seed):
    arrs = gen.make_arrays_qk(B, H, Nq, Nk, d, seed=seed)
    q, k, v, do = (to_dev(arrs[n]) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
    ref = fa2.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    got = fa2.bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return arrs, ref, got


@pytest.mark.parametrize("seq", [
    [(2, 3, 700, 700, 128, True), (1, 2, 150, 150, 64, False)],
    [(1, 2, 500, 500, 256, True), (1, 1, 100, 230, 256, False)],
    [(1, 4, 1024, 1024, 80, True), (2, 1, 77, 300, 96, True), (1, 1, 1, 1, 64, False)],
])
def test_noalloc_matches_workspace_backward(seq):
    for i, (B, H, Nq, Nk, d, causal) in enumerate(seq):
        print(f"call {i}: B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal}", flush=True)
        arrs, ref, got = both_ways(B, H, Nq, Nk, d, causal, seed=900 + i)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            same = torch.equal(a, b)
            assert same, (i, name)
    # the last call against the oracle (the bar of the parity tests)
    x = {n: oracle.bf16_bits_to_float64(arrs[n]) for n in ("q", "k", "v", "do")}
    g_ref = A.backward(x["q"], x["k"], x["v"], x["do"], 1.0 / math.sqrt(d), causal)
    for t, r in zip(got, g_ref):
        err = float(np.linalg.norm(t.float().cpu().numpy() - r) / max(np.linalg.norm(r), 1e-3))
        assert err <= 2e-2, err


def test_noalloc_rejects_sizes_beyond_its_scratch():
    q = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device=DEV)
    assert fa2.bwd_noalloc_max_bytes() == 32 << 20
    big = 1 + fa2.bwd_noalloc_max_bytes() // 8          # rows whose two fp32 arrays overflow it
    qb = torch.zeros((1, 1, big, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((1, 1, big), dtype=torch.float32, device=DEV)
    with pytest.raises(fa2.FA2Error) as e:
        fa2.bwd_noalloc(qb, q, q, qb, lse, qb, torch.empty_like(qb), torch.empty_like(q), torch.empty_like(q))
    assert e.value.status == 3
