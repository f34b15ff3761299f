"""Host-side checks of bench.py (no GPU): the one-GPU guard, the per-kernel flop
and compulsory-byte formulas, and the source hash that keys measured traffic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import fa2_inputs as gen  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def test_kernel_flops_per_launch():
    c4 = gen.WORKLOADS["c4"]   # B1 H16 N16384 d128 causal: 16 * 16384^2 / 2 (query, key) pairs
    pairs = 16 * 16384 ** 2 / 2
    f = bench.kernel_flops(c4)
    assert f["fwd"] == pytest.approx(4 * 128 * pairs)        # S and P V
    assert f["bwd_dkdv"] == pytest.approx(8 * 128 * pairs)   # S, dP, dV, dK
    assert f["bwd_dq"] == pytest.approx(6 * 128 * pairs)     # S, dP, dQ
    c2 = gen.WORKLOADS["c2"]   # non-causal: every pair
    assert bench.kernel_flops(c2)["fwd"] == pytest.approx(4 * 128 * 8 * 16 * 2048 ** 2)


def test_compulsory_bytes():
    c2 = gen.WORKLOADS["c2"]
    tensor = 8 * 16 * 2048 * 128 * 2            # one bf16 [B,H,N,d] tensor: 64 MiB
    rows, prow = 8 * 16 * 2048 * 4, 8 * 16 * 2048 * 4
    b = bench.compulsory_bytes(c2, 2048)
    assert tensor == 64 << 20
    assert b["fwd"] == 4 * tensor + rows                      # Q, K, V in; O, L out
    assert b["bwd_preprocess"] == 2 * tensor + rows + 2 * prow
    assert b["bwd_dkdv"] == 6 * tensor + 2 * prow              # Q, K, V, dO in; dK, dV out
    assert b["bwd_dq"] == 5 * tensor + 2 * prow                # Q, K, V, dO in; dQ out


def test_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_source_hash()
