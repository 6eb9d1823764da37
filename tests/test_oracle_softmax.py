"""Pins of the oracle's row softmax against a library routine (scipy) and the
widening of bf16 logits against torch's own conversion."""
import numpy as np
import pytest
import torch
from scipy.special import softmax


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("V", [1, 2, 7, 32, 1000, 4099])
@pytest.mark.parametrize("T", [1.0, 0.7, 2.0, 0.1])
def test_softmax_f32_matches_scipy(orc, V, T):
    rng = np.random.default_rng(V * 31 + int(T * 10))
    z = (rng.standard_normal(V) * 2.0).astype(np.float32)
    p = orc.softmax_row(z, T)
    ref = softmax(z.astype(np.float64) / np.float64(np.float32(T)))
    assert np.max(np.abs(p - ref)) < 1e-15
    assert abs(p.sum() - 1.0) < 1e-13


@pytest.mark.parametrize("V", [3, 152])
def test_softmax_bf16_widening(orc, V):
    rng = np.random.default_rng(5)
    bits = _bf16_bits(rng.standard_normal(V) * 4.0)
    p = orc.softmax_row(bits, 0.7)
    ref = softmax(_bf16_values(bits) / np.float64(np.float32(0.7)))
    assert np.max(np.abs(p - ref)) < 1e-15


def test_softmax_shift_invariance(orc):
    # adding a constant to every logit leaves the posterior unchanged
    rng = np.random.default_rng(11)
    z = rng.standard_normal(64).astype(np.float32)
    a = orc.softmax_row(z, 1.0)
    b = orc.softmax_row((z.astype(np.float64) + 8.0).astype(np.float32), 1.0)
    assert np.max(np.abs(a - b)) < 1e-6  # fp32 rounding of the shifted logits


def test_minus_inf_is_probability_zero(orc):
    z = np.array([0.0, -np.inf, 1.0, -np.inf], dtype=np.float32)
    p = orc.softmax_row(z, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    e = np.exp(1.0)
    assert abs(p[0] - 1 / (1 + e)) < 1e-16 and abs(p[2] - e / (1 + e)) < 1e-16


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_nan_and_plus_inf_rows_are_invalid(orc, bad):
    z = np.array([0.0, 1.0, bad, 2.0], dtype=np.float32)
    assert orc.softmax_row(z, 1.0) is None


def test_all_minus_inf_row_is_invalid(orc):
    z = np.full(5, -np.inf, dtype=np.float32)
    assert orc.softmax_row(z, 1.0) is None


def test_extreme_finite_logits(orc):
    # largest finite bf16 logits stay finite after widening and division
    bits = np.array([0x7F7F, 0xFF7F, 0x0000], dtype=np.uint16)  # +max, -max, 0
    p = orc.softmax_row(bits, 0.01)
    assert p[0] == 1.0 and p[1] == 0.0 and p[2] == 0.0
