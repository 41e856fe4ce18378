"""Pins of the oracle's building blocks against closed forms, textbook identities
and library routines (CPU only)."""
import math

import numpy as np
import pytest
import torch

from conftest import golden
from oracle import oracle as O

RNG = np.random.default_rng(11)


# ---------------------------------------------------------------- justnorm (dory.rs `justnorm`)

@pytest.mark.parametrize("n", [1, 7, 16, 2048])
def test_justnorm_closed_form(n):
    x = RNG.standard_normal(n).astype(np.float32) * 3
    y = O.justnorm(x)
    nx = np.linalg.norm(x.astype(np.float64))
    assert np.isclose(np.linalg.norm(y.astype(np.float64)), nx / math.sqrt(nx * nx + 1e-6), rtol=2e-7)
    # same direction
    assert np.allclose(y, x / math.sqrt(nx * nx + 1e-6), rtol=1e-6, atol=1e-9)


def test_justnorm_of_zero_is_zero_and_tiny_vectors_shrink():
    assert not O.justnorm(np.zeros(8, np.float32)).any()
    x = np.full(4, 1e-4, np.float32)          # |x|^2 = 4e-8 << eps: the epsilon dominates
    y = O.justnorm(x)
    assert np.allclose(y, x / math.sqrt(4e-8 + 1e-6), rtol=1e-6)


# ---------------------------------------------------------------- slerp (dory.rs `slerp`)

def test_slerp_alpha_zero_is_justnorm_of_x():
    x, o = RNG.standard_normal(64).astype(np.float32), RNG.standard_normal(64).astype(np.float32)
    y = O.slerp(x, o, np.zeros(64, np.float32))
    xh = x / np.linalg.norm(x)
    assert np.allclose(y, xh, atol=1e-6)


def test_slerp_alpha_one_is_justnorm_of_out():
    x, o = RNG.standard_normal(64).astype(np.float32), RNG.standard_normal(64).astype(np.float32)
    y = O.slerp(x, o, np.ones(64, np.float32))
    assert np.allclose(y, o / np.linalg.norm(o), atol=1e-6)


def test_slerp_is_symmetric_at_half_and_cancels_opposites():
    x, o = RNG.standard_normal(32).astype(np.float32), RNG.standard_normal(32).astype(np.float32)
    a = np.full(32, 0.5, np.float32)
    assert np.allclose(O.slerp(x, o, a), O.slerp(o, x, a), atol=1e-6)
    # x^ + 0.5 (-x^ - x^) = 0: the renorm of zero is zero
    assert np.abs(O.slerp(x, -x, a)).max() < 1e-3


def test_slerp_moves_toward_out_by_alpha_per_channel():
    # orthogonal unit x and o: before the renorm the result is (1-a) x + a o exactly
    x = np.zeros(4, np.float32); x[0] = 1
    o = np.zeros(4, np.float32); o[1] = 1
    a = np.array([0.3, 0.3, 0.3, 0.3], np.float32)
    y = O.slerp(x, o, a)
    want = np.array([0.7, 0.3, 0, 0]) / math.hypot(0.7, 0.3)
    assert np.allclose(y, want, atol=1e-6)


# ---------------------------------------------------------------- RoPE

@pytest.mark.parametrize("hd,theta", [(8, 1e4), (16, 1e7), (128, 1e4), (128, 1e7)])
def test_rope_frequencies(hd, theta):
    inv = O.rope_inv(hd, theta)
    assert inv[0] == 1.0
    assert np.all(np.diff(inv) < 0)
    assert np.isclose(inv[-1], theta ** (-(hd - 2) / hd), rtol=1e-6)
    assert np.isclose(inv[1] / inv[0], theta ** (-2 / hd), rtol=1e-6)


@pytest.mark.parametrize("hd", [8, 16, 128])
def test_rope_is_complex_multiplication(hd):
    """Rotate-half RoPE equals multiplying z_j = x_j + i x_{j+hd/2} by e^{i p w_j}."""
    inv = O.rope_inv(hd, 1e4)
    x = RNG.standard_normal(hd).astype(np.float32)
    for p in (0, 1, 17, 4095, 100000):
        y = O.rope_rotate(x, inv, p)
        z = (x[: hd // 2] + 1j * x[hd // 2:]) * np.exp(1j * p * inv.astype(np.float64))
        assert np.allclose(y, np.concatenate([z.real, z.imag]), atol=3e-6), p


def test_rope_identity_at_zero_norm_and_relative_positions():
    hd = 128
    inv = O.rope_inv(hd, 1e7)
    q = RNG.standard_normal(hd).astype(np.float32)
    k = RNG.standard_normal(hd).astype(np.float32)
    assert np.array_equal(O.rope_rotate(q, inv, 0), q)
    for p in (3, 1000, 8191):
        assert np.isclose(np.linalg.norm(O.rope_rotate(q, inv, p)), np.linalg.norm(q), rtol=1e-6)
    d = lambda a, b: float(np.dot(O.rope_rotate(q, inv, a), O.rope_rotate(k, inv, b)))
    assert abs(d(50, 20) - d(150, 120)) < 1e-5
    assert abs(d(7, 7) - float(np.dot(q, k))) < 1e-5


# ---------------------------------------------------------------- activations (dory.rs tests)

def test_silu_matches_library_silu_on_the_pages_case():
    g = golden("silu_case.json")
    n = g["n"]
    for i in range(n):
        gi, ui = (i - 10) * 0.37, 0.1 + 0.01 * i
        want = float(torch.nn.functional.silu(torch.tensor(gi * g["a"], dtype=torch.float64))) * (ui * g["b"])
        got = O.silu_gate(gi, g["a"], ui, g["b"])
        assert abs(got - want) <= g["tol"] * max(abs(want), 1.0), i


def test_sigmoid_gate_matches_library_sigmoid():
    for y, gv, s in [(0.3, 0.7, 2.0), (-1.2, -3.0, 0.5), (0.01, 40.0, 1.0), (2.0, -40.0, 1.0)]:
        want = y * float(torch.sigmoid(torch.tensor(gv * s, dtype=torch.float64)))
        assert abs(O.sigmoid_gate(y, gv, s) - want) <= 1e-6 * max(1.0, abs(want))


# ---------------------------------------------------------------- q8_2f encoder (kv_cache.rs `quant_row`)

@pytest.mark.parametrize("n,group", [(128, 32), (128, 128), (16, 32), (40, 32)])
def test_q8_encode_grid_properties(n, group):
    x = (RNG.standard_normal(n) * RNG.uniform(0.01, 5)).astype(np.float32)
    codes, scales = O.q8_encode(x, None, group)
    assert scales.shape[0] == -(-n // group)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    for gi, g0 in enumerate(range(0, n, group)):
        seg, c = x[g0:g0 + group], codes[g0:g0 + group].astype(np.float64)
        s = float(scales[gi])
        assert np.isclose(s, np.abs(seg).max() / 127, rtol=1e-6)
        assert np.abs(c).max() == 127                         # the absmax channel hits the grid edge
        assert np.all(np.abs(seg - c * s) <= s / 2 * (1 + 1e-5))  # within half a step


def test_q8_encode_rounds_half_away_from_zero_and_floors_zero_groups():
    codes, s = O.q8_encode(np.array([127.0, 0.5, -2.5, 1.5], np.float32), None, 4)
    assert s[0] == 1.0
    assert codes.tolist() == [127, 1, -3, 2]          # half away from zero, not to even
    codes, s = O.q8_encode(np.zeros(8, np.float32), None, 8)
    assert s[0] == np.float32(1e-12) and not codes.any()


def test_q8_encode_divides_by_the_field():
    x = RNG.standard_normal(64).astype(np.float32)
    col = RNG.uniform(0.1, 3.0, 64).astype(np.float32)
    c1, s1 = O.q8_encode(x, col, 32)
    c2, s2 = O.q8_encode(x / col, None, 32)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_q8_freeze_field_is_rms_of_dequantized_rows():
    rows, hd = 64, 128
    x = (RNG.standard_normal((rows, hd)) * np.where(np.arange(hd) % 2 == 0, 4.0, 0.25)).astype(np.float32)
    enc = [O.q8_encode(r, None, 32) for r in x]
    codes = np.stack([e[0] for e in enc]); scales = np.stack([e[1] for e in enc])
    deq = codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 32, axis=1)
    c2, s2, col = O.q8_freeze(codes, scales, 32)
    assert np.allclose(col, np.sqrt((deq ** 2).mean(0)), rtol=1e-5)
    # after the freeze the rows re-encode the dequantized values against the field
    for p in range(rows):
        want_c, want_s = O.q8_encode((codes[p] * np.repeat(scales[p], 32)).astype(np.float32), col, 32)
        assert np.array_equal(c2[p], want_c) and np.array_equal(s2[p], want_s)
    # and the field floors at 1e-6 for a dead channel
    codes[:, 3] = 0
    _, _, col0 = O.q8_freeze(codes, scales, 32)
    assert col0[3] == np.float32(1e-6)
