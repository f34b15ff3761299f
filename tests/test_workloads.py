"""Host-side checks of the GPT-shaped sublayer workload (no GPU)."""

import numpy as np
import pytest

import fa2_inputs as gen

pytest.importorskip("torch")
from exact_tiled_attention_34_amd.gpt_block import AttentionBlock, model_flops  # noqa: E402


def test_model_flops_formula():
    # 6 S params + 12 layers hidden S^2 per sequence; one layer has 4 hidden^2 weights
    assert model_flops(1, 10, 4) == 6 * 10 * 64 + 12 * 4 * 100
    assert model_flops(8, 2048, 2560) == 8 * (6 * 2048 * 4 * 2560 ** 2 + 12 * 2560 * 2048 ** 2)
    assert model_flops(2, 8, 4, layers=3) == 3 * model_flops(2, 8, 4) - 0.0


def test_gpt_block_inputs_are_seeded_and_shaped():
    a = gen.make_gpt_block(2, 16, 32, seed=5)
    b = gen.make_gpt_block(2, 16, 32, seed=5)
    for n, shape in (("x", (2, 16, 32)), ("w_qkv", (32, 96)), ("w_out", (32, 32)), ("dy", (2, 16, 32))):
        assert a[n].shape == shape and a[n].dtype == np.uint16
        assert np.array_equal(a[n], b[n])
    # the two table shapes hold 16k tokens each and 32 heads of 80
    for cfg in gen.GPT_BLOCKS.values():
        assert cfg["B"] * cfg["S"] == 16384 and cfg["hidden"] // cfg["heads"] == 80


def test_block_rejects_bad_weights():
    import torch
    with pytest.raises(ValueError):
        AttentionBlock(torch.zeros(8, 20), torch.zeros(8, 8), 2)
    with pytest.raises(ValueError):
        AttentionBlock(torch.zeros(8, 24), torch.zeros(8, 8), 3)
