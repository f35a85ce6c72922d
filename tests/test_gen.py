"""The seeded input generator: published SplitMix64 values, bfloat16 rounding, determinism."""
import json
import os

import numpy as np

import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_seed0_outputs():
    with open(os.path.join(GOLDEN, "splitmix64_seed0.json")) as f:
        ref = json.load(f)
    k = np.arange(1, 4, dtype=np.uint64)
    with np.errstate(over="ignore"):
        states = k * gen.GAMMA
    got = [f"{int(z):016x}" for z in gen.splitmix64(states)]
    assert got == ref["outputs_hex"]


def test_uniform24_is_top_24_bits():
    u = gen.uniform24(0, np.arange(3, dtype=np.uint64))
    with open(os.path.join(GOLDEN, "splitmix64_seed0.json")) as f:
        ref = json.load(f)
    exp = [(int(h, 16) >> 40) / float(1 << 24) for h in ref["outputs_hex"]]
    assert list(u) == exp
    big = gen.uniform24(987, np.arange(100000, dtype=np.uint64))
    assert big.min() >= 0.0 and big.max() < 1.0
    assert np.all((big * (1 << 24)) == np.floor(big * (1 << 24)))


def test_bf16_round_to_nearest_even_cases():
    with open(os.path.join(GOLDEN, "bf16_rne_cases.json")) as f:
        cases = json.load(f)["cases"]
    x = np.array([c["f32"] for c in cases], dtype=np.float32)
    exp = [int(c["bf16_hex"], 16) for c in cases]
    assert list(gen.f32_to_bf16_bits(x)) == exp
    assert list(gen.f32_to_bf16_bits_native(x)) == exp
    w = gen.bf16_bits_to_f32(np.array(exp, dtype=np.uint16))
    assert np.all(gen.f32_to_bf16_bits(w) == np.array(exp, dtype=np.uint16))


def test_native_generator_matches_numpy_definition():
    for seed, first, n, sigma in [(7, 0, 1001, 1.0), (20261205, 2 << 40, 4097, 3.0), (1, 1 << 40, 1, 1.0)]:
        ref = (gen.normal_f64(seed, first, n) * sigma).astype(np.float32)
        got = gen.normal_f32(seed, first, n, sigma)
        assert np.array_equal(ref, got)
    x = (np.random.default_rng(0).standard_normal(200000) * 50).astype(np.float32)
    assert np.array_equal(gen.f32_to_bf16_bits(x), gen.f32_to_bf16_bits_native(x))


def test_workload_inputs_deterministic_and_distinct():
    w = gen.WORKLOADS["f32_causal_b1h2_s128_d64"]
    (q1, k1, v1), _ = gen.make_inputs(w)
    (q2, k2, v2), _ = gen.make_inputs(w)
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert not np.array_equal(q1.ravel()[:100], k1.ravel()[:100])
    assert q1.shape == (1, 2, 128, 64)
    assert abs(float(q1.std()) - 1.0) < 0.05 and abs(float(q1.mean())) < 0.05


def test_bf16_workload_values_are_bf16():
    w = gen.WORKLOADS["f32_causal_b1h2_s128_d64"]
    (q, k, v), bits = gen.random_case(5, (1, 2, 64, 32), (1, 2, 48, 32), sigma_qk=3.0, dtype="bf16")
    for vals, b in zip((q, k, v), bits):
        assert b.dtype == np.uint16
        assert np.array_equal(gen.bf16_bits_to_f32(b), vals)
        assert np.all((vals.view(np.uint32) & 0xFFFF) == 0)
    assert abs(float(q.std()) - 3.0) < 0.1


def test_f16_rounding_matches_the_binary16_encoding():
    """Known binary16 encodings: exact values, ties to even, the largest finite value,
    subnormals and the overflow to infinity."""
    x = np.array([1.0, -2.0, 0.5, 65504.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -25, 65520.0, 0.0, -0.0], dtype=np.float32)
    want = [0x3C00, 0xC000, 0x3800, 0x7BFF, 0x3C00, 0x3C02, 0x0001, 0x0000, 0x0002, 0x7C00, 0x0000, 0x8000]
    assert gen.f32_to_f16_bits(x).tolist() == want
    back = gen.f16_bits_to_f32(np.array(want, dtype=np.uint16))
    assert back[0] == 1.0 and back[3] == 65504.0 and back[6] == 2.0 ** -24 and np.isinf(back[9])


def test_to_16bit_values_are_exact_images_of_the_bits():
    x = gen.tensor_f32(5, "q", (3, 7), 3.0)
    for dt in ("bf16", "f16"):
        vals, bits = gen.to_16bit(x, dt)
        assert vals.dtype == np.float32 and bits.dtype == np.uint16
        widened = gen.bf16_bits_to_f32(bits) if dt == "bf16" else gen.f16_bits_to_f32(bits)
        assert np.array_equal(vals, widened)
        assert np.abs(vals - x).max() <= (2.0 ** -8 if dt == "bf16" else 2.0 ** -11) * np.abs(x).max()
