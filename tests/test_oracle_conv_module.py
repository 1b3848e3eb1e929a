"""Pins of the oracle's conv module ("[Spec] DFlash2", code excerpt of the
grouped conv module: base kernel [input/output side, tap, channel] that
starts as the identity; one bias-free projection of the input gives both
sides' coefficients as [2, T, G]; prepare convolves the input with side 0 and
passes side 1's coefficients to finish).  Each pin fixes the result by
something other than the oracle: the module's identity start, one-hot
projection rows read back through the documented layout, brute-force exact
sums with integer rounding, and which side each half uses."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import dflash_oracle as O


def _bf16(rng, shape, scale):
    return O.round_to_bf16(rng.standard_normal(shape) * scale)


def _identity_base(T, H):
    base2 = np.zeros((2, T, H))
    base2[:, 0] = 1.0
    return base2


def test_module_starts_as_the_identity():
    # base kernel at its initial value (tap 0 = 1, other taps 0) and a zero
    # projection: prepare returns its input, finish returns its input, and
    # side 1's coefficients are zero
    rng = np.random.default_rng(3)
    N, H, T, gs, B = 12, 16, 3, 4, 4
    x = _bf16(rng, (N, H), 1.0)
    y = _bf16(rng, (N, H), 1.0)
    w = np.zeros((2 * T * (H // gs), H))
    out, coeff = O.conv_prepare(x, w, _identity_base(T, H), B, gs, "bf16")
    assert np.array_equal(out, x)
    assert not coeff.any()
    assert np.array_equal(O.conv_finish(y, coeff, _identity_base(T, H), B, gs), y)


@pytest.mark.parametrize("side,tap,group", [(0, 0, 0), (0, 2, 1), (1, 1, 3), (1, 2, 2)])
def test_projection_outputs_are_ordered_side_tap_group(side, tap, group):
    # a single one-hot projection row at index side*T*G + tap*G + group picks
    # input channel k: that coefficient equals x[:, k] and every other is 0
    rng = np.random.default_rng(4)
    N, H, T, gs = 6, 16, 3, 4
    G = H // gs
    x = _bf16(rng, (N, H), 1.0)
    w = np.zeros((2 * T * G, H))
    k = 5
    w[side * T * G + tap * G + group, k] = 1.0
    _, coeff = O.conv_prepare(x, w, _identity_base(T, H), 3, gs, "bf16")
    expect = np.zeros((N, 2, T, G))
    expect[:, side, tap, group] = x[:, k]
    assert np.array_equal(coeff, expect)


def test_prepare_uses_side_zero_and_finish_side_one():
    # a one-hot coefficient on one side only changes that side's convolution:
    # out[i, c] = x[i, c] + [i mod B >= t] * x[i, k] * x[i - t, c] for channels c
    # of group g on the side that carries it, and stays x (resp. y) on the other
    rng = np.random.default_rng(5)
    N, H, T, gs, B = 8, 8, 2, 4, 4
    G = H // gs
    x = _bf16(rng, (N, H), 1.0)
    y = _bf16(rng, (N, H), 1.0)
    k, t, g = 3, 1, 1
    for side in (0, 1):
        w = np.zeros((2 * T * G, H))
        w[side * T * G + t * G + g, k] = 1.0
        base2 = _identity_base(T, H)
        out, coeff = O.conv_prepare(x, w, base2, B, gs, "bf16")
        fin = O.conv_finish(y, coeff, base2, B, gs)
        want_out, want_fin = x.copy(), y.copy()
        src, want = (x, want_out) if side == 0 else (y, want_fin)
        for i in range(N):
            if i % B >= t:
                for c in range(g * gs, (g + 1) * gs):
                    want[i, c] += x[i, k] * src[i - t, c]
        assert np.array_equal(out, want_out), side
        assert np.array_equal(fin, want_fin), side


def _nearest_bf16(exact: Fraction) -> float:
    """bfloat16 rounding of an exact rational (8 significant bits, ties to an
    even significand) by integer arithmetic: the significand m in [128, 256)
    and a power-of-two step with a = m * step."""
    if exact == 0:
        return 0.0
    sign = -1 if exact < 0 else 1
    a = abs(exact)
    step = Fraction(1)
    while a / step >= 256:
        step *= 2
    while a / step < 128:
        step /= 2
    m = a / step
    whole = m.numerator // m.denominator
    frac = m - whole
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    return sign * float(whole * step)


def test_projection_is_the_exact_sum_rounded_once():
    # brute force: exact rational sums of the bf16 products, rounded once by
    # integer arithmetic (independent of the oracle's float rounding)
    rng = np.random.default_rng(6)
    N, H, P = 3, 9, 12
    x = _bf16(rng, (N, H), 1.0)
    w = _bf16(rng, (P, H), 0.3)
    got = O.conv_projection(x, w, "bf16")
    for n in range(N):
        for p in range(P):
            exact = sum(Fraction(float(x[n, k])) * Fraction(float(w[p, k])) for k in range(H))
            assert got[n, p] == _nearest_bf16(exact), (n, p)


def test_projection_in_fp32_of_small_integers_is_exact():
    # integer inputs whose sums stay below 2^24 are exact in fp32: the
    # coefficients equal the integer dot products
    rng = np.random.default_rng(7)
    xi = rng.integers(-20, 21, size=(4, 8))
    wi = rng.integers(-20, 21, size=(6, 8))
    got = O.conv_projection(xi.astype(np.float64), wi.astype(np.float64), "f32")
    for n in range(4):
        for p in range(6):
            assert got[n, p] == sum(int(xi[n, k]) * int(wi[p, k]) for k in range(8))


def test_planted_rounding_mistake_is_caught():
    # the brute-force pin above rejects a projection that truncates instead
    # of rounding to nearest: 1 + 3/256 rounds up to 1 + 1/64 in bf16
    x = np.array([[1.0, 3.0 / 256.0]])
    w = np.array([[1.0, 1.0]])
    exact = Fraction(1) + Fraction(3, 256)
    assert O.conv_projection(x, w, "bf16")[0, 0] == _nearest_bf16(exact) == 1.0 + 1.0 / 64.0
    truncated = np.floor(259.0 / 2) * 2 / 256.0            # keep 8 significant bits, drop the rest
    assert truncated != _nearest_bf16(exact)
