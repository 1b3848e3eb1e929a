"""Pins of the oracle's candidates-from-hidden step ("[Spec] DFlash2",
implementation breakdown: compute_candidates is the hidden rows times the
dense target head, then the unary transform and the deterministic top-k;
reading: the head's logits are rounded once to the storage dtype).  Each
pin fixes the result by something other than the oracle itself: closed
forms, brute-force sums over exact rationals, hand-worked rounding cases,
planted structure."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import dflash_oracle as O


def _bf16_values(rng, shape, scale):
    return O.round_to_bf16(rng.standard_normal(shape) * scale)


def test_identity_head_reduces_to_topk_of_the_hidden_values():
    # W = I (exact in bf16): the logits are the hidden values themselves
    rng = np.random.default_rng(1)
    h = _bf16_values(rng, (5, 24), 3.0)
    ids, unary = O.compute_candidates(h, np.eye(24), valid_vocab=24, top_k=4, multiplier=1.0, softcap=0.0,
                                      dtype="bf16")
    for n in range(5):
        order = sorted(range(24), key=lambda v: (-h[n, v], v))[:4]
        assert list(ids[n]) == order
        assert np.array_equal(unary[n], h[n, order])


def _nearest_bf16(exact: Fraction) -> float:
    """Round an exact rational to bfloat16 (8 significant bits, ties to an
    even significand) with integer arithmetic only."""
    if exact == 0:
        return 0.0
    sign = -1 if exact < 0 else 1
    a = abs(exact)
    e = a.numerator.bit_length() - a.denominator.bit_length()     # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (e - 7)                                  # significands 128..255
    m = a / step
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * float(lo * step)


def test_brute_force_exact_sums_then_one_rounding():
    # exact rational sums of the bf16 products, rounded once (RNE) by integer
    # arithmetic
    rng = np.random.default_rng(2)
    h = _bf16_values(rng, (3, 7), 1.0)
    w = _bf16_values(rng, (9, 7), 1.0)
    got = O.lm_head_logits(h, w, "bf16")
    for n in range(3):
        for v in range(9):
            exact = sum(Fraction(float(h[n, k])) * Fraction(float(w[v, k])) for k in range(7))
            assert got[n, v] == _nearest_bf16(exact), (n, v)


def test_rounding_happens_after_the_sum_with_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to even gives 1.
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6: gives 1 + 2^-6.
    # Rounding each product before summing would give 1 + 2^-8 -> 1 and
    # 1 + 3 * 2^-8 unchanged terms; the sum rounding is what is pinned.
    h = np.array([[1.0, 2.0 ** -8], [1.0, 3 * 2.0 ** -8], [1.0, 2.0 ** -9]])
    w = np.array([[1.0, 1.0]])
    z = O.lm_head_logits(h, w, "bf16")[:, 0]
    assert z[0] == 1.0 and z[1] == 1.0 + 2.0 ** -6 and z[2] == 1.0


def test_planted_row_is_top1_and_ties_go_to_the_lower_id():
    rng = np.random.default_rng(3)
    H, V = 32, 50
    h = _bf16_values(rng, (4, H), 1.0)
    w = _bf16_values(rng, (V, H), 0.05)
    w[17] = h[0] * 4          # dominates row 0
    w[40] = w[11]             # identical rows: equal logits everywhere
    ids, _ = O.compute_candidates(h, w, valid_vocab=V, top_k=3, multiplier=1.0, softcap=30.0, dtype="bf16")
    assert ids[0, 0] == 17
    z = O.lm_head_logits(h, w, "bf16")
    for n in range(4):
        pos = {int(v): i for i, v in enumerate(ids[n])}
        if 11 in pos and 40 in pos:
            assert pos[11] < pos[40]
        assert not (40 in pos and 11 not in pos and z[n, 11] == z[n, 40])


def test_padded_ids_of_the_head_are_never_selected():
    rng = np.random.default_rng(4)
    h = _bf16_values(rng, (3, 16), 1.0)
    w = _bf16_values(rng, (30, 16), 1.0)
    w[25:] = h[0] * 10        # huge logits in the padded tail
    ids, _ = O.compute_candidates(h, w, valid_vocab=25, top_k=5, multiplier=1.0, softcap=0.0, dtype="bf16")
    assert ids.max() < 25


def test_sum_bound_covers_an_fp32_accumulation():
    rng = np.random.default_rng(5)
    h = _bf16_values(rng, (6, 300), 1.0)
    w = _bf16_values(rng, (20, 300), 1.0)
    exact = h @ w.T
    acc = np.zeros((6, 20), np.float32)
    for k in range(300):              # one fp32 chain, products exact in fp32
        acc = (acc + (h[:, k:k + 1].astype(np.float32) * w[:, k].astype(np.float32))).astype(np.float32)
    assert np.all(np.abs(acc.astype(np.float64) - exact) <= O.lm_head_sum_bound(h, w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logits_are_in_the_storage_dtype(dtype):
    rng = np.random.default_rng(6)
    h = _bf16_values(rng, (2, 10), 1.0)
    w = _bf16_values(rng, (8, 10), 1.0)
    z = O.lm_head_logits(h, w, dtype)
    assert np.array_equal(O.round_to_dtype(z, dtype), z)
