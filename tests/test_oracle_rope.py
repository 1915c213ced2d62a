"""Pins of the oracle's RoPE and bf16 rounding against what the pages and the
mathematics fix (no GPU).

RoPE: "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §3 -- per-pair
frequency theta_i = base^(-2i/d), angle = position * theta, rotation by the
complex factor cos + i sin, and the relative-position property of the dot
product.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.full_causal import rope_complex

RNG = np.random.default_rng(1234)


def test_theta_closed_form():
    for D in (8, 64, 128):
        assert oracle.theta(0, D) == 1.0                       # base^0
        for i in range(D // 2):
            assert oracle.theta(i, D) == pytest.approx(10000.0 ** (-2.0 * i / D), rel=1e-15)
    # the last frequency of D = 128 is 10000^(-126/128)
    assert oracle.theta(63, 128) == pytest.approx(math.exp(-126 / 128 * math.log(10000.0)), rel=1e-14)
    # a different base is honoured (the pages mention 1000000 as well)
    assert oracle.theta(1, 64, 1e6) == pytest.approx(1e6 ** (-2 / 64), rel=1e-15)


def test_pair0_rotates_by_position_radians():
    # theta_0 = 1, so the first pair turns by exactly `pos` radians, counter-
    # clockwise: (a, b) -> (a cos p - b sin p, a sin p + b cos p)
    for pos in (1, 2, 255, 1023, 131071):
        for style, (ia, ib) in (("interleaved", (0, 1)), ("half", (0, 32))):
            x = np.zeros(64)
            x[ia] = 1.0
            y = oracle.rope_rotate(x, pos, style=style)
            assert y[ia] == pytest.approx(math.cos(pos), abs=1e-15)
            assert y[ib] == pytest.approx(math.sin(pos), abs=1e-15)
            x = np.zeros(64)
            x[ib] = 1.0
            y = oracle.rope_rotate(x, pos, style=style)
            assert y[ia] == pytest.approx(-math.sin(pos), abs=1e-15)
            assert y[ib] == pytest.approx(math.cos(pos), abs=1e-15)


def test_position_zero_is_identity_bitwise():
    x = RNG.standard_normal((5, 128))
    for style in ("interleaved", "half"):
        y = oracle.rope_rotate(x, 0, style=style)
        assert np.array_equal(x, y)


def test_pairs_stay_in_their_plane():
    D = 64
    for style in ("interleaved", "half"):
        for i in (0, 7, 31):
            ia, ib = (2 * i, 2 * i + 1) if style == "interleaved" else (i, i + D // 2)
            x = np.zeros(D)
            x[ia], x[ib] = 0.3, -1.7
            y = oracle.rope_rotate(x, 977, style=style)
            mask = np.ones(D, bool)
            mask[[ia, ib]] = False
            assert np.all(y[mask] == 0.0)
            angle = 977 * 10000.0 ** (-2.0 * i / D)
            assert y[ia] == pytest.approx(0.3 * math.cos(angle) + 1.7 * math.sin(angle), abs=1e-13)


def test_norm_preserved():
    x = RNG.standard_normal((16, 128))
    for pos in (3, 4095, 131071):
        y = oracle.rope_rotate(x, pos)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_composition():
    x = RNG.standard_normal((4, 64))
    for m, n in ((0, 5), (17, 250), (65535, 65536), (100000, 31071)):
        a = oracle.rope_rotate(oracle.rope_rotate(x, n), m)
        b = oracle.rope_rotate(x, m + n)
        # angles reach ~1.3e5 rad: fp64 angle error ~1e-11 absolute
        np.testing.assert_allclose(a, b, atol=1e-9)


def test_relative_position_identity():
    """(R_m q) . (R_n k) depends on n - m only: equals q . (R_{n-m} k).

    The page prints R_{m-n} on the right-hand side; with its own rotation by
    cos + i sin that form fails for generic vectors, so the identity is
    checked with n - m (and the printed form is shown not to hold)."""
    D = 64
    for _ in range(6):
        q = RNG.standard_normal(D)
        k = RNG.standard_normal(D)
        m, n = (int(v) for v in RNG.integers(0, 131072, 2))
        lhs = oracle.rope_rotate(q, m) @ oracle.rope_rotate(k, n)
        rhs = q @ oracle.rope_rotate(k, n - m)
        assert lhs == pytest.approx(rhs, abs=1e-9 * np.linalg.norm(q) * np.linalg.norm(k))
        # same dot product for any common shift of both positions
        lhs2 = oracle.rope_rotate(q, m + 1000) @ oracle.rope_rotate(k, n + 1000)
        assert lhs2 == pytest.approx(lhs, abs=1e-9 * np.linalg.norm(q) * np.linalg.norm(k))
    q = RNG.standard_normal(D)
    k = RNG.standard_normal(D)
    lhs = oracle.rope_rotate(q, 37) @ oracle.rope_rotate(k, 250)
    printed = q @ oracle.rope_rotate(k, 37 - 250)
    assert abs(lhs - printed) > 1e-3


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_matches_independent_complex_numpy(style):
    # the NumPy recompute rotates through complex multiplication, written
    # separately from the C loops
    x = RNG.standard_normal((1, 3, 128))
    for pos in (1, 511, 8191, 131071):
        a = oracle.rope_rotate(x[0], pos, style=style)
        b = rope_complex(x, np.array([pos]), style=style)[0]
        # the two compute theta_i in different (equally valid) ways, 1 ulp
        # apart; at position p the angles then differ by ~p * 2^-52
        np.testing.assert_allclose(a, b, atol=max(1e-14, pos * 2e-16 * 4), rtol=0)


def test_half_style_is_a_permutation_of_interleaved():
    D = 128
    x = RNG.standard_normal(D)
    perm = np.empty(D, int)            # interleaved slot 2i <- half slot i, 2i+1 <- i + D/2
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    for pos in (9, 4000):
        yh = oracle.rope_rotate(x, pos, style="half")
        yi = oracle.rope_rotate(x[perm], pos, style="interleaved")
        np.testing.assert_array_equal(yh[perm], yi)


# ----------------------------------------------------------- bf16 rounding

def _torch_bf16_bits(x32):
    import torch
    t = torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_fp32_values():
    # fp32 inputs: a single rounding from fp64 equals torch's fp32 -> bf16 cast
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    extra = np.array([0.0, -0.0, 1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 3.3895314e38,
                      3.39e38, -3.4e38, 1e-40, 2**-133, 2**-134, 3 * 2**-135, 1.5 * 2**-126,
                      np.float32(np.finfo(np.float32).tiny) * 0.75], np.float32)
    vals = np.concatenate([vals, extra])
    want = _torch_bf16_bits(vals)
    got = np.array([oracle.bf16_bits(float(v)) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, want)


def test_bf16_rounding_ties_and_single_rounding():
    assert oracle.round_to_bf16(1.0 + 2**-8) == 1.0                   # tie -> even
    assert oracle.round_to_bf16(1.0 + 3 * 2**-8) == 1.0 + 2**-6      # tie -> even (up)
    assert oracle.round_to_bf16(-(1.0 + 3 * 2**-8)) == -(1.0 + 2**-6)
    # just above a tie: one rounding from fp64 goes up; rounding through
    # fp32 first would land on the tie and then go down to even
    x = 1.0 + 2**-8 + 2**-40
    assert np.float32(x) == np.float32(1.0 + 2**-8)
    assert oracle.round_to_bf16(x) == 1.0 + 2**-7
    assert oracle.bf16_bits(float("inf")) == 0x7F80
    assert oracle.bf16_bits(float("-inf")) == 0xFF80
    assert oracle.bf16_bits(float("nan")) & 0x7FFF == 0x7FC0
    assert oracle.round_to_bf16(3.4e38) == math.inf                  # above max + half ulp
    assert oracle.round_to_bf16(2.0**-134) == 0.0                    # half of the smallest subnormal, tie -> 0
    assert oracle.round_to_bf16(2.0**-134 + 2.0**-160) == 2.0**-133
