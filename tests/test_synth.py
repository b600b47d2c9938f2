"""The shared seeded input generator: determinism and bf16 rounding (CPU)."""
import numpy as np
import torch

from ring_attention_attn_amd import synth


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact ties
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_block_draws_are_deterministic_and_independent():
    a = synth.blocks_tensor(7, synth.T_K, [3, 4], 8, 2, 4, "f32")
    b = synth.blocks_tensor(7, synth.T_K, [4], 8, 2, 4, "f32")
    assert np.array_equal(a[8:], b)
    c = synth.blocks_tensor(7, synth.T_V, [4], 8, 2, 4, "f32")
    assert not np.array_equal(b, c)
    assert synth.paired_blocks(4, 1) == [1, 6]


def test_head_subsets_draw_the_same_values():
    """A head group drawn on its own equals the same heads of the full draw (the
    head-parallel share's inputs exist without the other groups')."""
    full = synth.blocks_tensor(11, synth.T_Q, [0, 5], 16, 8, 4, "bf16")
    part = synth.blocks_tensor(11, synth.T_Q, [0, 5], 16, range(4, 6), 4, "bf16")
    assert np.array_equal(full[:, 4:6], part)
    assert full.dtype == np.uint16 and full.shape == (32, 8, 4)
