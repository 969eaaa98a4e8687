"""The seeded input generator (shared by the GPU tests and the oracle)."""
import hashlib

import numpy as np
import torch

from logit_source_projection_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        # values exactly half-way between two bf16 numbers (ties to even)
        ((np.arange(1000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38], dtype=np.float32),
    ])
    ours = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_draws_are_deterministic():
    w1 = inputs.draw_weight(600, 1000, 0.02, seed=3)
    w2 = inputs.draw_weight(600, 1000, 0.02, seed=3)
    assert hashlib.sha256(w1.tobytes()).digest() == hashlib.sha256(w2.tobytes()).digest()
    assert not np.array_equal(w1, inputs.draw_weight(600, 1000, 0.02, seed=4))
    x1 = inputs.draw_hidden(8, 512, seed=3)
    assert np.array_equal(x1, inputs.draw_hidden(8, 512, seed=3))


def test_weight_statistics():
    w = inputs.bf16_bits_to_f32(inputs.draw_weight(512, 4096, 0.02, seed=0))
    assert abs(float(w.std()) - 0.02) < 2e-4
    assert abs(float(w.mean())) < 2e-4


def test_rms_normalised_hidden_rows():
    x = inputs.bf16_bits_to_f32(inputs.draw_hidden(64, 4096, seed=0, rms_norm=True))
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 5e-3)


def test_equal_lanes():
    assert inputs.equal_lanes(151936, 4) == [0, 37984, 75968, 113952, 151936]
    assert inputs.equal_lanes(200064, 4)[1] == 50016
    assert inputs.equal_lanes(10, 3) == [0, 4, 7, 10]


def test_near_tie_plan():
    assert inputs.near_tie_rows(1) == [0]
    assert inputs.near_tie_rows(8) == [0]
    assert inputs.near_tie_rows(16) == [0, 8]
    pairs = inputs.near_tie_cols(inputs.equal_lanes(200064, 4))
    assert pairs[0] == (50015, 50016)
    assert 150048 <= pairs[1][0] < pairs[1][1] < 200064
