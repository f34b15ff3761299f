"""Whole-tensor comparison of attention outputs with the float64 oracle, one
(batch, head) at a time in a thread pool (test infrastructure, CPU only).

The parity bar is stated over whole tensors: max |O - O_ref| and max |L - L_ref|
over every element, and ||g - g_ref||_F / ||g_ref||_F for g in dQ, dK, dV with
the norms taken over all (batch, head) pairs.  The oracle materialises one
head's N x N score matrix at a time, so the heads are independent jobs: the
squared norms are summed per head and combined at the end.  Per-head figures
(the worst head of each error) and the error of O against the oracle's O
rounded to the 16-bit storage type (how far the kernel is from the best
representable answer) are reported as diagnostics.
"""

import os
import time
from concurrent.futures import ThreadPoolExecutor, as_completed

import numpy as np

import oracle
from oracle import attention as A


def cpu_share():
    """CPUs this process should use: its affinity set, capped by OMP_NUM_THREADS
    when that is set (a share of a larger host)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(env))) if env.isdigit() else n


def round_to_storage(x, dtype):
    """float64 -> nearest 16-bit value (bf16 / fp16), back as float64 (diagnostic only)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x32.astype(np.float16).astype(np.float64)
    u = x32.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def compare_all_heads(got, arrs, scale, causal, dtype="bf16", workers=None, head_mem_bytes=None):
    """Errors of `got` (host float32 arrays o [B,H,N,d], lse [B,H,N], dq, dk, dv)
    against the oracle on every (batch, head) of the 16-bit inputs in `arrs`.

    Returns {"O", "L", "dQ", "dK", "dV"} over whole tensors plus diagnostics:
    "O_vs_rounded" (O against the oracle's O rounded to the storage type),
    "worst_head" (per error, the largest per-head value and its (b, h)), and
    "workers"."""
    B, H, N, d = arrs["q"].shape
    share = cpu_share()
    if workers is None:
        # about five N x N float64 arrays live per head at the oracle's peak
        per_head = head_mem_bytes or 5 * 8 * N * N
        workers = max(1, min(share, 16, B * H, int(48e9 // max(per_head, 1))))
    blas_threads = max(1, share // workers)

    def one(bh):
        b, h = divmod(bh, H)
        x = {n: oracle.bits_to_float64(arrs[n][b, h], dtype) for n in ("q", "k", "v", "do")}
        o_ref, l_ref = A.forward_head(x["q"], x["k"], x["v"], scale, causal)
        g_ref = A.backward_head(x["q"], x["k"], x["v"], x["do"], scale, causal)
        o = got["o"][b, h].astype(np.float64)
        lse = got["lse"][b, h].astype(np.float64)
        r = {"O": float(np.max(np.abs(o - o_ref))),
             "O_vs_rounded": float(np.max(np.abs(o - round_to_storage(o_ref, dtype)))),
             "L": float(np.max(np.abs(lse - l_ref)))}
        for name, key, ref in zip(("dQ", "dK", "dV"), ("dq", "dk", "dv"), g_ref):
            diff = got[key][b, h].astype(np.float64) - ref
            r[name + "_num"] = float(np.sum(diff * diff))
            r[name + "_den"] = float(np.sum(ref * ref))
        return (b, h), r

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=blas_threads, user_api="blas")
    except Exception:
        limiter = None
    results = []
    t0 = time.perf_counter()
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            futs = [ex.submit(one, bh) for bh in range(B * H)]
            every = max(1, len(futs) // 8)
            for n, f in enumerate(as_completed(futs), 1):
                results.append(f.result())
                if n % every == 0 or n == len(futs):
                    print(f"  oracle: {n}/{len(futs)} heads, {time.perf_counter() - t0:.0f} s", flush=True)
    finally:
        if limiter is not None:
            limiter.unregister()

    out = {"O": max(r["O"] for _, r in results), "O_vs_rounded": max(r["O_vs_rounded"] for _, r in results),
           "L": max(r["L"] for _, r in results), "workers": workers}
    worst = {}
    for name in ("dQ", "dK", "dV"):
        num = sum(r[name + "_num"] for _, r in results)
        den = sum(r[name + "_den"] for _, r in results)
        # a zero exact gradient makes the relative norm undefined: floor the
        # denominator as the small-shape tests do
        out[name] = float(np.sqrt(num) / max(np.sqrt(den), 1e-3))
        per = [(np.sqrt(r[name + "_num"]) / max(np.sqrt(r[name + "_den"]), 1e-3), bh) for bh, r in results]
        worst[name] = max(per)
    for name in ("O", "L"):
        worst[name] = max((r[name], bh) for bh, r in results)
    out["worst_head"] = {k: (round(float(v), 6), bh) for k, (v, bh) in worst.items()}
    return out
