"""The C ABI (no GPU): the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before making any HIP call.

Only invalid argument combinations are passed here: each is rejected by the
host-side checks, so the fake (never dereferenced) pointers below never reach
a kernel.  As a second safeguard, the tests that pass fake pointers are skipped
in any process that can see a GPU: they cover host logic only.
"""

import ctypes
import os
import re

import pytest

from exact_tiled_attention_34_amd import fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4

# distinct, 16-byte aligned, far-apart fake device addresses (never dereferenced)
P = [0x10000000 * (i + 1) for i in range(12)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_[a-z0-9_]+)\s*\(", text)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


host_only = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: host-only checks")


@pytest.fixture(scope="module")
def lib():
    return fa2.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fa2_fwd", "fa2_bwd", "fa2_bwd_workspace_bytes", "fa2_strerror"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    # and the binding declares a signature for each of them
    assert set(names) == set(fa2._SIGNATURES)


def fwd(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, N=128, d=64, scale=0.125, causal=0):
    return lib.fa2_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@host_only
@pytest.mark.parametrize("kw,want", [
    (dict(N=0), INVALID), (dict(B=0), INVALID), (dict(H=-1), INVALID),
    (dict(d=112), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(d=192), UNSUPPORTED), (dict(d=512), UNSUPPORTED),
    (dict(causal=2), INVALID), (dict(causal=-1), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-0.125), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(q=None), INVALID), (dict(lse=None), INVALID),
    (dict(k=P[1] + 8), INVALID), (dict(o=P[3] + 2), INVALID),
    (dict(o=P[0]), INVALID),                     # output aliases an input
    (dict(lse=P[3] + 64), INVALID),              # lse inside o
    (dict(B=1024, H=1024, N=4096, d=128), INVALID),  # too many elements for 32-bit rows
])
def test_fwd_rejects(lib, kw, want):
    assert fwd(lib, **kw) == want


def bwd(lib, ws_bytes=None, B=1, H=2, N=128, d=64, scale=0.125, causal=0, **ptrs):
    names = ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"]
    p = dict(zip(names, P))
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.fa2_bwd_workspace_bytes(B, H, N, d)
    return lib.fa2_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                       B, H, N, d, scale, causal, p["ws"], ws_bytes, None)


@host_only
def test_bwd_rejects(lib):
    need = lib.fa2_bwd_workspace_bytes(1, 2, 128, 64)
    assert need == 2 * (2 * 256 * 4)
    assert bwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert bwd(lib, ws_bytes=0) == WORKSPACE
    assert bwd(lib, d=72) == UNSUPPORTED
    assert bwd(lib, causal=3) == INVALID
    assert bwd(lib, scale=-1.0) == INVALID
    assert bwd(lib, ws=None) == INVALID
    assert bwd(lib, dq=P[0]) == INVALID          # dq aliases q
    assert bwd(lib, dk=P[6] + 16) == INVALID     # dk overlaps dq
    assert bwd(lib, ws=P[8] + 4096) == INVALID   # workspace overlaps dv
    assert bwd(lib, do=P[5] + 4) == INVALID      # misaligned


@host_only
def test_phase_entry_points_reject(lib):
    # preprocess(o, dout, lse, delta, lse_log2, B, H, N, d, stream)
    assert lib.fa2_bwd_preprocess(*P[:5], 1, 1, 0, 64, None) == INVALID
    assert lib.fa2_bwd_preprocess(*P[:5], 1, 1, 64, 112, None) == UNSUPPORTED
    assert lib.fa2_bwd_preprocess(P[0], P[1], P[2], P[0], P[4], 1, 1, 64, 64, None) == INVALID
    assert lib.fa2_bwd_preprocess(P[0], P[1], P[2], P[3], P[3] + 256, 1, 1, 64, 64, None) == INVALID
    # dkdv(q, k, v, dout, lse_log2, delta, dk, dv, B, H, N, d, scale, causal, stream)
    assert lib.fa2_bwd_dkdv(*P[:8], 1, 1, 64, 100, 0.1, 0, None) == UNSUPPORTED
    assert lib.fa2_bwd_dkdv(*P[:8], 1, 1, 64, 64, 0.0, 0, None) == INVALID
    assert lib.fa2_bwd_dkdv(*P[:7], None, 1, 1, 64, 64, 0.1, 0, None) == INVALID
    assert lib.fa2_bwd_dkdv(*P[:7], P[6] + 16, 1, 1, 64, 64, 0.1, 0, None) == INVALID
    assert lib.fa2_bwd_dkdv(*P[:6], P[0], P[7], 1, 1, 64, 64, 0.1, 0, None) == INVALID
    # dq(q, k, v, dout, lse_log2, delta, dq, B, H, N, d, scale, causal, stream)
    assert lib.fa2_bwd_dq(*P[:7], 1, 1, 64, 64, 0.1, 5, None) == INVALID
    assert lib.fa2_bwd_dq(*P[:6], P[4], 1, 1, 64, 64, 0.1, 0, None) == INVALID
    assert lib.fa2_bwd_dq(*P[:6], P[6] + 8, 1, 1, 64, 64, 0.1, 0, None) == INVALID


@host_only
def test_separate_length_entry_points_reject(lib):
    # fwd_qk(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, stream)
    assert lib.fa2_fwd_qk(*P[:5], 1, 2, 64, 0, 64, 0.1, 1, None) == INVALID      # no keys
    assert lib.fa2_fwd_qk(*P[:5], 1, 2, 0, 64, 64, 0.1, 1, None) == INVALID      # no queries
    assert lib.fa2_fwd_qk(*P[:5], 1, 2, 64, 64, 72, 0.1, 1, None) == UNSUPPORTED
    assert lib.fa2_fwd_qk(*P[:5], 1, 1 << 16, 1, 1 << 12, 128, 0.1, 0, None) == INVALID  # Nk too long
    # k spans Nk rows: an output placed inside k's (longer) span is rejected
    nk_bytes = 2 * 1000 * 64 * 2
    assert lib.fa2_fwd_qk(P[0], P[1], P[2], P[1] + nk_bytes - 256, P[4], 1, 2, 10, 1000, 64, 0.1, 0,
                          None) == INVALID
    # bwd_qk(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, ws, ws_bytes, stream)
    need = lib.fa2_bwd_workspace_bytes(1, 2, 10, 64)
    assert lib.fa2_bwd_qk(*P[:9], 1, 2, 10, 0, 64, 0.1, 1, P[9], need, None) == INVALID
    assert lib.fa2_bwd_qk(*P[:9], 1, 2, 10, 300, 64, 0.1, 1, P[9], need - 1, None) == WORKSPACE
    assert lib.fa2_bwd_qk(*P[:7], P[1] + 4096, P[8], 1, 2, 10, 300, 64, 0.1, 1, P[9], need,
                          None) == INVALID                                       # dk inside k
    # dkdv_qk / dq_qk: dk, dv hold Nk rows, dq holds Nq rows
    assert lib.fa2_bwd_dkdv_qk(*P[:6], P[6], P[6] + 2 * 10 * 64 * 2, 1, 2, 10, 300, 64, 0.1, 1,
                               None) == INVALID                                  # dv overlaps dk (Nk rows)
    assert lib.fa2_bwd_dkdv_qk(*P[:8], 1, 2, 10, 0, 64, 0.1, 1, None) == INVALID
    assert lib.fa2_bwd_dq_qk(*P[:7], 1, 2, 10, 300, 112, 0.1, 0, None) == UNSUPPORTED
    assert lib.fa2_bwd_dq_qk(*P[:6], P[1] + 2 * 2 * 299 * 64, 1, 2, 10, 300, 64, 0.1, 0,
                             None) == INVALID                                    # dq inside k


@host_only
def test_strided_entry_points_reject(lib):
    S = fa2.Strides
    B, H, N, d = 1, 2, 64, 64
    dense = S(H * N * d, N * d, d)
    bshd = S(N * H * d, d, H * d)

    def fwd_s(sq=dense, so=dense, o=P[3], q=P[0], dtype=0):
        return lib.fa2_fwd_strided(q, ctypes.byref(sq), P[1], None, P[2], None, o, ctypes.byref(so), P[4],
                                   B, H, N, N, d, 0.1, 1, dtype, None)

    assert fwd_s(sq=S(H * N * d, N * d, d + 4)) == INVALID        # row stride not a multiple of 8
    assert fwd_s(sq=S(H * N * d, -8, d)) == INVALID               # negative stride
    assert fwd_s(so=S(H * N * d, N * d, d - 8)) == INVALID        # output rows overlap
    assert fwd_s(so=S(H * N * d, d, d)) == INVALID                # output heads overlap rows
    assert fwd_s(o=P[0] + 2 * d * 3, so=bshd) == INVALID          # output inside q's span
    assert fwd_s(q=P[0] + 8) == INVALID                           # misaligned base
    assert fwd_s(sq=S(H * N * d, N * d, d + 4), dtype=1) == INVALID
    assert fwd_s(dtype=2) == INVALID                              # unknown 16-bit type
    assert fwd_s(sq=S(0, 0, 1 << 24)) == INVALID                  # rows beyond 2^30 elements
    assert fwd_s(sq=S(H * N * d, N * d, (1 << 20) + 8)) == INVALID   # row stride beyond 2^20 elements
    # backward: an output inside an input, the workspace inside an output
    need = lib.fa2_bwd_workspace_bytes(B, H, N, d)
    args = [P[0], None, P[1], None, P[2], None, P[3], None, P[4], P[5], None,
            P[6], None, P[7], None, P[8], None]
    assert lib.fa2_bwd_strided(*args, B, H, N, N, d, 0.1, 1, 0, P[9], need - 1, None) == WORKSPACE
    assert lib.fa2_bwd_strided(*args, B, H, N, N, d, 0.1, 1, 5, P[9], need, None) == INVALID
    bad = list(args)
    bad[13] = P[1] + 64                                          # dk inside k
    assert lib.fa2_bwd_strided(*bad, B, H, N, N, d, 0.1, 1, 1, P[9], need, None) == INVALID
    assert lib.fa2_bwd_strided(*args, B, H, N, N, d, 0.1, 1, 0, P[8] + 256, need, None) == INVALID


def test_workspace_size_query(lib):
    assert lib.fa2_bwd_rows_padded(1) == 256
    assert lib.fa2_bwd_rows_padded(256) == 256
    assert lib.fa2_bwd_rows_padded(257) == 512
    assert lib.fa2_bwd_rows_padded(0) == 0
    assert lib.fa2_bwd_workspace_bytes(1, 1, 1, 112) == 0
    assert lib.fa2_bwd_workspace_bytes(0, 1, 1, 64) == 0
    # delta and L*log2(e), fp32 [B, H, padded rows], each rounded up to 256 bytes
    assert lib.fa2_bwd_workspace_bytes(1, 1, 3, 80) == 2 * 1024
    assert lib.fa2_bwd_workspace_bytes(1, 16, 16384, 128) == 2 * 16 * 16384 * 4
    assert lib.fa2_bwd_workspace_bytes(3, 1, 200, 64) == 2 * 3 * 256 * 4


def test_strerror_and_tiles(lib):
    for s in range(5):
        assert lib.fa2_strerror(s)
    assert b"unknown" in lib.fa2_strerror(99)
    assert lib.fa2_last_error() == b""
    for d in (64, 80, 96, 128, 256):
        t = fa2.tile_config(d)
        assert t["fwd_block_q"] % 32 == 0 and t["bwd_block_k"] % 32 == 0
        assert t["fwd_block_q"] == 32 * t["fwd_waves"]
    with pytest.raises(fa2.FA2Error):
        fa2.tile_config(112)


@host_only
def test_noalloc_backward_rejects_before_any_hip_call(lib):
    """fa2_bwd_qk_noalloc validates like fa2_bwd_qk, and rejects sizes whose row
    arrays exceed its fixed scratch with FA2_ERR_WORKSPACE (checked before the
    scratch's device address is looked up, i.e. before any HIP call)."""
    assert lib.fa2_bwd_noalloc_max_bytes() == 32 << 20
    # (q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, stream)
    assert lib.fa2_bwd_qk_noalloc(*P[:9], 1, 2, 10, 0, 64, 0.1, 1, None) == INVALID
    assert lib.fa2_bwd_qk_noalloc(*P[:9], 1, 2, 10, 10, 72, 0.1, 1, None) == UNSUPPORTED
    assert lib.fa2_bwd_qk_noalloc(*P[:9], 1, 2, 10, 10, 64, -0.1, 1, None) == INVALID
    assert lib.fa2_bwd_qk_noalloc(*P[:8], P[1] + 4096, 1, 2, 10, 300, 64, 0.1, 1, None) == INVALID  # dv in k
    assert lib.fa2_bwd_qk_noalloc(None, *P[1:9], 1, 2, 10, 10, 64, 0.1, 1, None) == INVALID
    # 64 heads of 131072 rows: two fp32 row arrays of 32 MiB each do not fit
    assert lib.fa2_bwd_workspace_bytes(1, 64, 131072, 64) > lib.fa2_bwd_noalloc_max_bytes()
    assert lib.fa2_bwd_qk_noalloc(*P[:9], 1, 64, 131072, 131072, 64, 0.1, 1, None) == WORKSPACE
    assert lib.fa2_last_error() == b""
