"""The seeded input generator: determinism, rounding, distributions, recipes."""
import math

import numpy as np
import torch

import workloads as W


def test_same_seed_same_bytes():
    a = W.random_inputs(16, 32, 2, 3, 8, "bf16", seed=5)
    b = W.random_inputs(16, 32, 2, 3, 8, "bf16", seed=5)
    c = W.random_inputs(16, 32, 2, 3, 8, "bf16", seed=6)
    for k in ("x", "W_node", "b_node", "V_node", "W_out"):
        assert getattr(a, k).tobytes() == getattr(b, k).tobytes()
        assert getattr(a, k).tobytes() != getattr(c, k).tobytes()


def test_splitmix64_known_values():
    # splitmix64 seeded with 0: its first outputs are the published test values
    # of the reference generator (state advanced by the golden gamma first).
    z = W._mix64(np.array([0x9E3779B97F4A7C15, 0x3C6EF372FE94F82A], dtype=np.uint64))
    assert int(z[0]) == 0xE220A8397B1DCDAF
    assert int(z[1]) == 0x6E789E6AA1B965F4


def test_bf16_round_nearest_even_hand_picked():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),            # tie, even neighbour below
        (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie, even neighbour above
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie
        (-1.0 - 2.0 ** -8, 0xBF80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),                # smallest subnormal
        (2.0 ** -134, 0x0000),                # tie to zero (even)
        (3 * 2.0 ** -134, 0x0002),            # tie, even neighbour above
        (2.0 ** -126, 0x0080),                # smallest normal
        (1e39, 0x7F80),                       # overflow to +inf
        (-3.3895313892515355e38, 0xFF7F),     # largest finite magnitude
    ]
    got = W.round_to_bf16_bits(np.array([v for v, _ in cases]))
    assert [int(g) for g in got] == [bits for _, bits in cases]


def test_bf16_matches_torch_on_float32_values():
    # torch rounds float32 -> bfloat16 to nearest even; on values already in
    # float32 a single rounding from float64 must agree with it.
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    ours = W.round_to_bf16_bits(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    back = W.bf16_bits_to_f64(ours)
    assert np.all(np.abs(back - v) <= np.abs(v) * 2.0 ** -8)


def test_normal_moments():
    z = W.standard_normal(3, 1, 200000)
    assert abs(z.mean()) < 0.01
    assert abs(z.var() - 1.0) < 0.01
    assert abs(np.mean(z ** 4) - 3.0) < 0.05


def test_variances_follow_fan_in():
    inp = W.random_inputs(512, 256, 4, 4, 64, "f32", seed=1)
    f = inp.as_f64()
    assert abs(f["W_node"].var() - 1 / 256) < 0.05 / 256
    assert abs(f["b_node"].std() - 0.1) < 0.02
    assert abs(f["V_node"].var() - 1 / 64) < 0.05 / 64
    assert abs(f["W_out"].var() - 1 / 256) < 0.05 / 256
    assert abs(f["x"].var() - 1.0) < 0.02


def test_unit_rms_rows():
    inp = W.random_inputs(64, 2048, 1, 1, 4, "bf16", unit_rms_x=True)
    x = inp.as_f64()["x"]
    rms = np.sqrt(np.mean(x * x, axis=1))
    assert np.all(np.abs(rms - 1.0) < 2e-3)


def test_decode_workloads_are_prefixes_and_skewed():
    t1 = W.workload("decode_skew_t1")
    t8 = W.workload("decode_skew_t8")
    t64 = W.workload("decode_skew_t64")
    np.testing.assert_array_equal(t64.x[:8], t8.x)
    np.testing.assert_array_equal(t64.x[:1], t1.x)
    for k in ("W_node", "b_node", "V_node", "W_out"):
        np.testing.assert_array_equal(getattr(t1, k), getattr(t64, k))
    f = t64.as_f64()
    norms = np.sqrt((f["W_node"] ** 2).sum(axis=2))
    shifted = f["b_node"][:, [3, 5]] / norms[:, [3, 5]]
    assert np.all(shifted > 2.4) and np.all(shifted < 3.6)
    others = np.delete(f["b_node"], [3, 5], axis=1)
    assert np.abs(others).max() < 0.6


def test_named_shapes():
    s = W.WORKLOADS["opt1p3b_d6"][0]
    assert (s.T, s.d, s.P, s.D, s.h, s.N) == (16384, 2048, 32, 6, 128, 127)
    s = W.WORKLOADS["gpt125m"][0]
    assert (s.T, s.d, s.P, s.D, s.h, s.N) == (8192, 768, 16, 5, 64, 63)
    assert math.isclose(W.workload("tiny").as_f64()["x"].var(), 1.0, rel_tol=0.1)
