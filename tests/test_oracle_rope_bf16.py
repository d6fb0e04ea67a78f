"""Pins for the oracle's bf16 rounding and RoPE relocation (CPU only)."""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import GOLDEN


def test_bf16_round_matches_torch_cast_on_fp32_values():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even; on values that
    # are exactly fp32 the oracle's one-step fp64 rounding must agree with it.
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10 ** rng.uniform(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, -1e-42]]).astype(np.float32)
    # exact halfway cases: low 16 bits = 0x8000 with even and odd kept parts
    halves = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, halves, -halves])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_bits_roundtrip_and_ulp():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    exp_field = (bits.astype(np.uint32) >> 7) & 0xFF
    fin = exp_field != 0xFF                      # drop inf/NaN patterns
    vals = oracle.bf16_bits_to_f64(bits[fin])
    assert np.array_equal(oracle.f64_to_bf16_bits(vals), bits[fin])
    assert oracle.ulp_bf16(1.0) == 2.0 ** -7
    assert oracle.ulp_bf16(1.5) == 2.0 ** -7
    assert oracle.ulp_bf16(0.75) == 2.0 ** -8
    assert oracle.ulp_bf16(1e-40) == 2.0 ** -133


def test_rope_golden_d4():
    g = json.load(open(os.path.join(GOLDEN, "rope_d4.json")))
    got = oracle.rope(np.array(g["x"]), g["position"], g["theta"])
    np.testing.assert_allclose(got, g["expected"], rtol=1e-14, atol=1e-15)


def test_rope_d2_is_plane_rotation():
    # D = 2: omega_0 = 1, so rope is the textbook rotation by p radians.
    for p in [0.0, 0.3, -2.0, 1000.0]:
        rot = np.array([[math.cos(p), -math.sin(p)], [math.sin(p), math.cos(p)]])
        x = np.array([0.7, -1.3])
        np.testing.assert_allclose(oracle.rope(x, p, 1e4), rot @ x, rtol=1e-13, atol=1e-13)


def test_rope_matches_complex_multiplication():
    # Independent formulation: pair (x_j, x_{j+D/2}) as x_j + i x_{j+D/2}, times e^{i p w_j}.
    rng = np.random.default_rng(2)
    D, theta = 16, 1e6
    x = rng.standard_normal(D)
    p = 4097
    z = [complex(x[j], x[j + D // 2]) * cmath.exp(1j * p * theta ** (-2.0 * j / D)) for j in range(D // 2)]
    ref = np.array([c.real for c in z] + [c.imag for c in z])
    np.testing.assert_allclose(oracle.rope(x, p, theta), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D,theta", [(64, 1e4), (128, 1e6)])
def test_relocation_composes(D, theta):
    rng = np.random.default_rng(3)
    k = rng.standard_normal((40, D))
    p = rng.integers(0, 65536, 40)
    delta = rng.integers(-30000, 30000, 40)
    a = oracle.relocate(oracle.rope(k, p, theta), delta, theta)
    b = oracle.rope(k, p + delta, theta)
    np.testing.assert_allclose(a, b, atol=1e-9)  # angles up to ~1e5 rad: fp64 trig ~1e-11
    np.testing.assert_array_equal(oracle.relocate(k, 0, theta), k)
    back = oracle.relocate(oracle.relocate(k, delta, theta), -delta, theta)
    np.testing.assert_allclose(back, k, atol=1e-12)
    half = D // 2
    n0 = k[:, :half] ** 2 + k[:, half:] ** 2
    kr = oracle.relocate(k, delta, theta)
    np.testing.assert_allclose(kr[:, :half] ** 2 + kr[:, half:] ** 2, n0, rtol=1e-12)
