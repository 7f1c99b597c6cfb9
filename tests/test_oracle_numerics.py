"""Pins for the oracle's input widening and the generators' bf16 rounding
(CPU only).

The oracle must read exactly the values the device reads: the foundry
"PagedAttention" page (*How it works*) says storage in blocks is transparent
to the attention math, so any difference between the oracle's and the
kernel's view of a stored value would be the oracle's error.  bf16 patterns
are widened by the oracle with its own bit shift; these tests hold that shift,
and the round-to-nearest-even of the seeded generators, against PyTorch's
bfloat16 conversions, which share no code with either.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import numerics as N

from test_oracle_attention import brute_force, run_oracle, scatter_case


def _torch_widen(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_widening_matches_torch_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = N.bf16_bits_to_f64(bits)
    ref = _torch_widen(bits)
    nan = np.isnan(ref)
    # NaN patterns: 0x7f81..0x7fff and 0xff81..0xffff (254 of them)
    assert int(nan.sum()) == 2 * 127
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros and infinities keep their signs
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_widening_known_values():
    # patterns whose values follow from the binary32 layout alone
    cases = {0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F00: 0.5, 0x3FC0: 1.5, 0x4049: 3.140625,
             0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0x7F80: np.inf, 0xFF80: -np.inf, 0x0000: 0.0}
    bits = np.array(list(cases), dtype=np.uint16)
    np.testing.assert_array_equal(N.bf16_bits_to_f64(bits), np.array(list(cases.values())))
    assert np.signbit(N.bf16_bits_to_f64(np.array([0x8000], np.uint16)))[0]


def test_round_to_bf16_matches_torch_on_edge_values():
    f32 = np.float32
    up = lambda u: np.array([u], np.uint32).view(np.float32)[0]
    vals = [
        0.0, -0.0, 1.0, -1.0, np.inf, -np.inf,
        up(0x3F808000),  # exactly halfway, even below: stays 0x3F80
        up(0x3F818000),  # exactly halfway, odd below: rounds up to 0x3F82
        up(0x3F808001),  # just above halfway: up
        up(0x3F807FFF),  # just below halfway: down
        up(0x7F7FFFFF),  # max finite fp32: rounds to +inf
        up(0x7F7F7FFF),  # max finite bf16 from below
        up(0x7F7F8000),  # halfway above max finite bf16, odd: to +inf
        up(0x00000001),  # smallest subnormal
        up(0x00008000),  # subnormal halfway, even below
        up(0x00018000),  # subnormal halfway, odd below
        up(0x007FFFFF),  # largest subnormal: rounds to the smallest normal
        up(0x80008001),  # negative subnormal above halfway
        f32(3.14159265), f32(-2.718281828), f32(65504.0), f32(1e-40),
    ]
    x = np.array(vals, np.float32)
    ours = W.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # NaN (quiet and signalling, either sign) becomes a NaN pattern
    nans = np.array([0x7FC00000, 0x7F800001, 0xFFC00000, 0xFFFFFFFF], np.uint32).view(np.float32)
    r = W.round_to_bf16(nans)
    assert np.all(np.isnan(_torch_widen(r)))


def test_round_to_bf16_matches_torch_on_random_floats():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(200_000, dtype=np.float32),
                        rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    x = x[~np.isnan(x)]
    ours = W.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def _wrong_widening(kind):
    def widen(bits):
        bits = np.asarray(bits)
        u = bits.astype(np.uint32)
        if kind == "shift15":
            wide = u << np.uint32(15)
        elif kind == "no_sign":
            wide = (u & np.uint32(0x7FFF)) << np.uint32(16)
        elif kind == "lost_mantissa_bit":
            wide = (u & np.uint32(0xFFFE)) << np.uint32(16)
        else:
            raise ValueError(kind)
        return wide.view(np.float32).astype(np.float64)
    return widen


@pytest.mark.parametrize("kind", ["shift15", "no_sign", "lost_mantissa_bit"])
def test_planted_widening_mistakes_are_caught(monkeypatch, kind):
    """A wrong bf16 widening in the oracle fails the brute-force pin, whose
    inputs are widened by torch."""
    rng = np.random.default_rng(91)
    c, lk, lv = scatter_case(rng, [9, 21], 4, 2, 8, 4, dtype=W.BF16)
    expect = brute_force(c, lk, lv)
    np.testing.assert_allclose(run_oracle(c), expect, rtol=0, atol=1e-12)
    monkeypatch.setattr(N, "bf16_bits_to_f64", _wrong_widening(kind))
    got = run_oracle(c)
    assert np.max(np.abs(got - expect)) > 1e-6


def test_scale_widening_is_the_fp32_value():
    s = 1 / np.sqrt(128.0)
    assert N.scale_f64(s) == float(torch.tensor(s, dtype=torch.float32).to(torch.float64))
    assert N.scale_f64(s) != s  # 1/sqrt(128) is not exact in binary32
