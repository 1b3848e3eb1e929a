"""Pins of the oracle's unary transform and per-slot top-K against what the
pages fix: the transform's disabled defaults and its softcap bounds ("[Spec]
DFlash2", implementation breakdown), deterministic selection with lowest-id
ties, and that padded ids are never taken ("DSpark padded-vocab d2t fix")."""
import math

import numpy as np
import pytest

from conftest import load_golden
from oracle import dflash_oracle as O


def test_transform_disabled_defaults_are_identity():
    z = np.array([-7.5, -1.0, 0.0, 2.25, 100.0, -np.inf])
    np.testing.assert_array_equal(O.transform(z, 1.0, 0.0), z)


def test_transform_multiplier_only_scales():
    z = np.array([-3.0, 0.5, 8.0])
    np.testing.assert_array_equal(O.transform(z, 0.5, 0.0), 0.5 * z)


def test_transform_softcap_bounds_symmetry_and_slope():
    z = np.linspace(-500, 500, 2001)
    for m, cap in [(1.0, 30.0), (0.5, 30.0), (2.0, 5.0)]:
        y = O.transform(z, m, cap)
        assert np.all(np.abs(y) <= cap)
        assert np.all(np.abs(y[np.abs(m * z) < 10 * cap]) < cap)
        np.testing.assert_allclose(O.transform(-z, m, cap), -y, rtol=0, atol=0)
        assert np.all(np.diff(y) >= 0)
        eps = 1e-6
        np.testing.assert_allclose(O.transform(np.array([eps]), m, cap)[0] / eps, m, rtol=1e-9)


def test_transform_closed_form_point():
    # m*z/cap = atanh(1/2)  =>  y = cap / 2
    m, cap = 0.5, 30.0
    z = cap * math.atanh(0.5) / m
    assert abs(O.transform(np.array([z]), m, cap)[0] - cap / 2) < 1e-12


def test_transform_keeps_masked_entries_masked():
    assert O.transform(np.array([-np.inf]), 0.5, 30.0)[0] == -np.inf


@pytest.mark.parametrize("case", load_golden("topk_ties.json")["cases"], ids=lambda c: c["why"][:30])
def test_golden_tie_and_mask_cases(case):
    z = np.array([float(v) for v in case["z"]])[None, :]
    ids, unary = O.topk(z, case["valid_vocab"], case["k"], 1.0, 0.0)
    assert ids[0].tolist() == case["ids"]
    np.testing.assert_array_equal(unary[0], z[0, ids[0]])


def _selection_is_valid(z, valid, k, ids):
    """Independent check of a top-K answer: every selected entry beats every
    unselected eligible entry under (value desc, id asc), the list is in that
    order, ids are unique and eligible."""
    ids = list(ids)
    assert len(set(ids)) == k and all(0 <= i < valid for i in ids)

    def better(a, b):
        return z[a] > z[b] or (z[a] == z[b] and a < b)

    for a, b in zip(ids, ids[1:]):
        assert better(a, b)
    chosen = set(ids)
    worst = ids[-1]
    for j in range(valid):
        if j not in chosen:
            assert better(worst, j)


@pytest.mark.parametrize("seed", range(6))
def test_selection_property_on_random_rows_with_ties(seed):
    rng = np.random.default_rng(seed)
    V = 97
    valid = 90
    k = [1, 4, 8, 16, 32, 90][seed]
    # coarse values force many ties; a few -inf
    z = np.round(rng.standard_normal((5, V)) * 2) / 2
    z[:, rng.integers(0, V, 6)] = -np.inf
    z[:, valid:] = 50.0      # padding holds the largest values but is never eligible
    ids, _ = O.topk(z, valid, k, 1.0, 0.0)
    for n in range(z.shape[0]):
        _selection_is_valid(z[n], valid, k, ids[n])


def test_planted_peak_is_top1():
    rng = np.random.default_rng(11)
    z = rng.standard_normal((4, 1000)) * 3
    planted = rng.integers(0, 1000, 4)
    z[np.arange(4), planted] = z.max(axis=1) + 8
    ids, _ = O.topk(z, 1000, 8, 1.0, 30.0)
    np.testing.assert_array_equal(ids[:, 0], planted)


def test_ids_do_not_depend_on_transform_parameters():
    rng = np.random.default_rng(12)
    z = np.round(rng.standard_normal((6, 300)) * 8) / 4
    ref, _ = O.topk(z, 300, 16, 1.0, 0.0)
    for m, cap in [(0.5, 30.0), (2.0, 1.0), (1.0, 30.0)]:
        ids, unary = O.topk(z, 300, 16, m, cap)
        np.testing.assert_array_equal(ids, ref)
        assert np.all(np.diff(unary, axis=1) <= 0)


def test_valid_vocab_equals_neg_inf_padding():
    rng = np.random.default_rng(13)
    z = rng.standard_normal((3, 200)) * 3
    z_pad = z.copy(); z_pad[:, 180:] = -np.inf
    a, _ = O.topk(z, 180, 12, 0.5, 30.0)
    b, _ = O.topk(z_pad, 200, 12, 0.5, 30.0)
    c, _ = O.topk(z_pad, 180, 12, 0.5, 30.0)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_k_equal_to_vocab_is_a_permutation():
    z = np.array([[3.0, -1.0, 3.0, 0.0, 7.0]])
    ids, _ = O.topk(z, 5, 5, 1.0, 0.0)
    assert ids[0].tolist() == [4, 0, 2, 3, 1]


def test_rejects_nan_and_bad_k():
    with pytest.raises(ValueError):
        O.topk(np.array([[1.0, np.nan, 2.0]]), 3, 1, 1.0, 0.0)
    with pytest.raises(ValueError):
        O.topk(np.array([[1.0, 2.0]]), 1, 2, 1.0, 0.0)
