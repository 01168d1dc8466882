"""The seeded input generators: bf16 rounding against torch's float -> bfloat16 cast
(nearest, ties to even), chunked streams independent of the thread count, and the
drawn distributions."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0),
                        # exact ties in both directions, subnormals, extremes, signed zero, inf
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130,
                                  -2.0 ** -140, 3.3e38, -3.3e38, 0.0, -0.0, np.inf, -np.inf], np.float32)])
    ours = W.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_streams_do_not_depend_on_thread_count(monkeypatch):
    shape = (3, W.CHUNK + 12345)  # several chunks and a ragged last one
    many = W.normal_bf16_outliers(shape, seed=4)
    monkeypatch.setattr(W, "_threads", lambda: 1)
    one = W.normal_bf16_outliers(shape, seed=4)
    assert np.array_equal(many, one)
    # chunk i of a tensor is its own stream: a longer tensor starts with the same values
    assert np.array_equal(W.normal_bf16((W.CHUNK + 7,), seed=2)[:W.CHUNK], W.normal_bf16((W.CHUNK,), seed=2))


def test_distributions():
    b = W.bf16_bits_to_f32(W.normal_bf16((2048, 2048), std=0.02, seed=0, tensor_id=W.T_B)).astype(np.float64)
    assert abs(b.std() - 0.02) < 2e-4 and abs(b.mean()) < 1e-4
    a = W.bf16_bits_to_f32(W.normal_bf16_outliers((512, 4096), seed=0)).astype(np.float64)
    frac = np.mean(np.abs(a) > 8.0)  # N(0,1) alone exceeds 8 with probability ~1e-15
    assert 0.0080 < frac < 0.0095  # P(|50 z| > 8) = 0.873 of the 1% outliers
    # different tensor ids and seeds give different draws
    assert not np.array_equal(W.normal_bf16((64,), seed=0, tensor_id=W.T_A), W.normal_bf16((64,), seed=0, tensor_id=W.T_B))
    assert not np.array_equal(W.normal_bf16((64,), seed=0), W.normal_bf16((64,), seed=1))
