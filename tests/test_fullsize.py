"""The whole-tensor comparison used by the full-size GPU tests, checked on the CPU:
exact answers give (rounding-level) zero error, the per-head sums combine to the
Frobenius norm of the whole tensor, and a mistake planted in one head is found
and attributed to that head."""

import numpy as np

import fa2_inputs as gen
import oracle
from oracle import attention as A
from fullsize import compare_all_heads, round_to_storage


def exact_outputs(arrs, scale, causal):
    x = {n: oracle.bf16_bits_to_float64(arrs[n]) for n in ("q", "k", "v", "do")}
    o, lse = A.forward(x["q"], x["k"], x["v"], scale, causal)
    dq, dk, dv = A.backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def test_exact_answers_have_zero_error():
    arrs = gen.make_arrays(2, 3, 70, 64, seed=3)
    got = exact_outputs(arrs, 0.125, True)
    e = compare_all_heads(got, arrs, 0.125, True, workers=3)
    assert e["O"] < 1e-12 and e["L"] < 1e-12
    assert max(e["dQ"], e["dK"], e["dV"]) < 1e-12
    # against the oracle's O rounded to bf16 the exact O is off by at most half an ulp
    assert 0 < e["O_vs_rounded"] <= np.max(np.abs(got["o"])) * 2.0 ** -8


def test_planted_error_in_one_head_is_found():
    B, H, N, d = 2, 3, 50, 80
    arrs = gen.make_arrays(B, H, N, d, seed=4)
    scale = 1.0 / np.sqrt(d)
    got = exact_outputs(arrs, scale, False)
    ref_dk = got["dk"].copy()
    got["dk"][1, 2] *= 1.1                     # 10 % off in head (1, 2) only
    got["o"][0, 1, 7, 3] += 0.02               # one element of O
    e = compare_all_heads(got, arrs, scale, False, workers=2)
    # whole-tensor norm = sqrt(sum over heads), as computed directly
    want = np.linalg.norm(got["dk"] - ref_dk) / np.linalg.norm(ref_dk)
    assert abs(e["dK"] - want) <= 1e-9 * want
    assert e["worst_head"]["dK"][1] == (1, 2)
    assert abs(e["worst_head"]["dK"][0] - 0.1) < 1e-6
    assert abs(e["O"] - 0.02) < 1e-9 and e["worst_head"]["O"][1] == (0, 1)
    assert e["dQ"] < 1e-12 and e["dV"] < 1e-12


def test_round_to_storage():
    x = np.array([1.0, 1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9, -2.5, 65504.0])
    np.testing.assert_array_equal(round_to_storage(x, "bf16"), [1.0, 1.0, 1.0 + 2.0 ** -7, -2.5, 65536.0])
    y = np.array([1.0 + 2.0 ** -12, 1.0 + 3 * 2.0 ** -12, 65504.0])   # fp16: 10 fraction bits
    np.testing.assert_array_equal(round_to_storage(y, "fp16"), [1.0, 1.0 + 2.0 ** -10, 65504.0])
