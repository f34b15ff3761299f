"""Seeded synthetic inputs for exact attention (shared by tests, bench and smoke).

This module holds no attention arithmetic: it only draws random numbers,
rounds them to bfloat16 and names the workload shapes.  Both the HIP path and
the CPU oracle receive exactly the arrays produced here.

Recipe (every workload):
  * ``numpy.random.Generator(PCG64(seed))``; draws in a fixed order Q, K, V, dO,
    each ``standard_normal(shape, float32) * sigma``;
  * each float32 value is rounded once to bfloat16 with round-to-nearest-even
    on its bit pattern (``round_to_bf16_bits``);
  * the "spike" workload then draws one row index r[b, h] ~ U{0..N-1} per
    (batch, head) from the same generator and multiplies row r of Q and of K
    by 8 before rounding (a power of two, so exact), widening the score range
    the softmax must handle.

Tensors too large to draw on the host (the maximum-size case, up to 2^31
elements each) are drawn on the GPU instead (``make_device_tensors``):
``torch.Generator`` seeded with ``seed``; Q, K, V, dO in that order, each batch
index b in turn, ``torch.randn((H, N, d), float32)`` converted to bfloat16 by
torch's round-to-nearest-even.  The oracle takes the bit patterns of the heads
it checks from those tensors.

Workload shapes follow the attention benchmark sweeps on the "FlashAttention-2:
Faster Attention with Better Parallelism and Work Partitioning" page (Figures
4-7: head dimension 64 / 128, causal and non-causal, sequence lengths up to
16k) and the GPT-3 2.7B-shaped layer of its Table 1 (hidden 2560, 32 heads of
80).  Arrays are uint16 bit patterns ``[B, H, N, d]`` (d fastest).
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    sigma: float = 1.0
    spike: bool = False

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def flops(self, phase: str) -> float:
        """Conventional attention flop count: 4*B*H*N^2*d forward, 2.5x that
        backward, halved when causal."""
        fwd = 4.0 * self.B * self.H * self.N * self.N * self.d
        if self.causal:
            fwd /= 2.0
        return {"fwd": fwd, "bwd": 2.5 * fwd, "fwdbwd": 3.5 * fwd}[phase]


WORKLOADS = {
    "c1": Workload("c1", "single-head B1 H1 N128 d64 non-causal", 1, 1, 128, 64, False),
    "c2": Workload("c2", "B8 H16 N2048 d128 non-causal (hidden 2048)", 8, 16, 2048, 128, False),
    "c3": Workload("c3", "B4 H32 N4096 d64 causal (hidden 2048)", 4, 32, 4096, 64, True),
    "c4": Workload("c4", "long-sequence B1 H16 N16384 d128 causal", 1, 16, 16384, 128, True),
    "c5": Workload("c5", "GPT-2.7B-shaped B2 H32 N8192 d80 causal, sigma 0.5 + one x8 row/head",
                   2, 32, 8192, 80, True, sigma=0.5, spike=True),
}


def round_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    NaN stays a quiet NaN; values past the largest finite bfloat16 round to
    infinity as IEEE round-to-nearest requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), out)
    return out


def round_to_fp16_bits(x) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), round-to-nearest-even (numpy's
    float16 conversion; values past 65504 become infinity)."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _rounder(dtype):
    if dtype == "bf16":
        return round_to_bf16_bits
    if dtype == "fp16":
        return round_to_fp16_bits
    raise ValueError(f"unknown 16-bit type {dtype!r}")


def make_arrays(B, H, N, d, seed=0, sigma=1.0, spike=False, dtype="bf16"):
    """Q, K, V, dO as uint16 bit patterns [B,H,N,d] (bf16, or fp16 with dtype="fp16")
    plus the spike rows (or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    draws = []
    for _ in range(4):
        x = rng.standard_normal(shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        draws.append(x)
    rows = None
    if spike:
        rows = rng.integers(0, N, size=(B, H))
        bi, hi = np.meshgrid(np.arange(B), np.arange(H), indexing="ij")
        draws[0][bi, hi, rows] *= np.float32(8.0)
        draws[1][bi, hi, rows] *= np.float32(8.0)
    q, k, v, do = (_rounder(dtype)(x) for x in draws)
    return {"q": q, "k": k, "v": v, "do": do, "spike_rows": rows}


def make_arrays_qk(B, H, Nq, Nk, d, seed=0, dtype="bf16"):
    """Q, dO as uint16 bit patterns [B,H,Nq,d] and K, V as [B,H,Nk,d] (N(0,1) draws)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, n in (("q", Nq), ("k", Nk), ("v", Nk), ("do", Nq)):
        out[name] = _rounder(dtype)(rng.standard_normal((B, H, n, d), dtype=np.float32))
    out["spike_rows"] = None
    return out


def make_device_tensors(B, H, N, d, seed=0, device="cuda:0"):
    """Q, K, V, dO as bf16 torch tensors [B,H,N,d] drawn on `device` (N(0,1) draws)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for name in ("q", "k", "v", "do"):
        t = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=device)
        for b in range(B):
            t[b] = torch.randn((H, N, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        out[name] = t
    return out


# Attention sublayer of the GPT-3 2.7B shape in Table 1 of the "FlashAttention-2:
# Faster Attention with Better Parallelism and Work Partitioning" page (hidden
# 2560 = 32 heads x 80), at its two context lengths; B x S = 16k tokens each.
GPT_BLOCKS = {
    "2k": dict(B=8, S=2048, hidden=2560, heads=32),
    "8k": dict(B=2, S=8192, hidden=2560, heads=32),
}


def make_gpt_block(B, S, hidden, seed=0, w_std=0.02):
    """Input x [B,S,hidden], weights W_qkv [hidden,3 hidden] and W_out [hidden,hidden]
    (N(0, w_std^2), the usual GPT initialisation scale) and the output gradient
    dy [B,S,hidden], as uint16 bf16 bit patterns; draws in that order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, S, hidden), dtype=np.float32)
    w_qkv = rng.standard_normal((hidden, 3 * hidden), dtype=np.float32) * np.float32(w_std)
    w_out = rng.standard_normal((hidden, hidden), dtype=np.float32) * np.float32(w_std)
    dy = rng.standard_normal((B, S, hidden), dtype=np.float32)
    return {n: round_to_bf16_bits(a) for n, a in (("x", x), ("w_qkv", w_qkv), ("w_out", w_out), ("dy", dy))}


# Further shapes for measurement only (not among the five configured
# workloads): head dimension 256 on a long causal sequence.
EXTRA_WORKLOADS = {
    "d256": Workload("d256", "B1 H16 N8192 d256 causal (head dim 256)", 1, 16, 8192, 256, True),
}


def make_workload(key, seed=0):
    w = WORKLOADS[key] if key in WORKLOADS else EXTRA_WORKLOADS[key]
    return w, make_arrays(w.B, w.H, w.N, w.d, seed=seed, sigma=w.sigma, spike=w.spike)
