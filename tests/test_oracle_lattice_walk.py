"""Pins of the oracle's projection, lattice and walk against what the DFlash2
pages fix ("[Spec] DFlash2: local convolution + candidate selector"): the
edge formula of the executive summary, the anchor as slot 0's predecessor
(draft-sampler excerpt), greedy rows emitting a point mass and sampled rows
the softmax q they drew from (walk-kernel excerpt and executive summary),
mixed-batch greedy determinism (test list of the PR), and brute-force
enumeration of every K^S path on tiny inputs."""
import itertools
import math

import numpy as np
import pytest

from conftest import load_golden
from oracle import dflash_oracle as O

F32 = np.float32


def test_projection_with_one_hot_rows_selects_coordinates():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((3, 5, 16))
    P = np.zeros((4, 16)); P[0, 3] = 1; P[1, 0] = 1; P[2, 15] = 1; P[3, 7] = -2
    u = O.project(h, P)
    np.testing.assert_array_equal(u, np.stack([h[..., 3], h[..., 0], h[..., 15], -2 * h[..., 7]], -1))


def test_golden_lattice_and_walks():
    g = load_golden("lattice_walk_small.json")
    ids = np.array(g["ids"]); unary = np.array(g["unary"], float)
    scores = O.lattice(ids, unary, np.array(g["u"], float), np.array(g["anchor"]),
                       np.array(g["sel_a"], float), np.array(g["sel_b"], float))
    np.testing.assert_allclose(scores, np.array(g["scores"], float), rtol=0, atol=1e-15)
    R, S, K = ids.shape
    tok, q, _ = O.walk(scores, ids, np.zeros((R, S), F32), np.ones(R, F32), np.ones(R, bool))
    assert tok.tolist() == g["greedy_tokens"]
    np.testing.assert_array_equal(q, np.array(g["greedy_q"], F32))
    tok, q, _ = O.walk(scores, ids, np.array(g["sampled_uniforms"], F32),
                       np.full(R, g["sampled_temperature"], F32), np.zeros(R, bool))
    assert tok.tolist() == g["sampled_tokens"]
    assert abs(float(q[0, 0, 0]) - g["sampled_q_slot0_first"]) < 1e-6


def _random_lattice(rng, R=3, S=4, K=5, r=6, V=40):
    ids = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(S)]) for _ in range(R)])
    unary = rng.standard_normal((R, S, K))
    u = rng.standard_normal((R, S, r))
    anchor = rng.integers(0, V, R)
    A, B = rng.standard_normal((V, r)), rng.standard_normal((V, r))
    return ids, unary, u, anchor, A, B


def test_lattice_with_zero_selector_is_unary():
    rng = np.random.default_rng(1)
    ids, unary, u, anchor, A, B = _random_lattice(rng)
    for zero in ("A", "u"):
        s = O.lattice(ids, unary, 0 * u if zero == "u" else u, anchor, 0 * A if zero == "A" else A, B)
        np.testing.assert_array_equal(s, np.broadcast_to(unary[:, :, None, :], s.shape))


def test_lattice_rank_one_closed_form():
    rng = np.random.default_rng(2)
    ids, unary, u, anchor, A, B = _random_lattice(rng, r=1)
    s = O.lattice(ids, unary, u, anchor, A, B)
    R, S, K = ids.shape
    for r in range(R):
        for t in range(S):
            for j in range(K):
                p = anchor[r] if t == 0 else ids[r, t - 1, j]
                for c in range(K):
                    want = A[p, 0] * u[r, t, 0] * B[ids[r, t, c], 0] + unary[r, t, c]
                    assert abs(s[r, t, j, c] - want) < 1e-12


def test_slot_zero_rows_are_identical():
    rng = np.random.default_rng(3)
    s = O.lattice(*_random_lattice(rng))
    for j in range(1, s.shape[2]):
        np.testing.assert_array_equal(s[:, 0, j], s[:, 0, 0])


def test_greedy_rows_are_point_masses_with_lowest_index_ties():
    scores = np.zeros((1, 2, 3, 3), F32)
    scores[0, 0, 0] = [1.0, 3.0, 3.0]           # tie between index 1 and 2 -> 1
    scores[0, 1, 1] = [5.0, 5.0, 5.0]           # all tied -> 0
    ids = np.array([[[10, 11, 12], [20, 21, 22]]])
    tok, q, idx = O.walk(scores, ids, np.full((1, 2), 0.99, F32), np.ones(1, F32), np.ones(1, bool))
    assert idx.tolist() == [[1, 0]] and tok.tolist() == [[11, 20]]
    np.testing.assert_array_equal(q, np.array([[[0, 1, 0], [1, 0, 0]]], F32))


def test_mixed_batch_greedy_rows_are_deterministic():
    # Greedy rows must not depend on the uniforms, the temperatures, the other
    # rows' modes, or on being run alone.
    rng = np.random.default_rng(4)
    R, S, K = 6, 5, 8
    scores = (rng.standard_normal((R, S, K, K)) * 3).astype(F32)
    ids = rng.integers(0, 1000, (R, S, K))
    greedy = np.array([True, False, True, False, True, True])
    base_tok, base_q, _ = O.walk(scores, ids, rng.random((R, S)).astype(F32),
                                 rng.uniform(0.1, 2, R).astype(F32), greedy)
    for trial in range(3):
        g2 = greedy.copy(); g2[1] = bool(trial % 2)
        tok, q, _ = O.walk(scores, ids, rng.random((R, S)).astype(F32),
                           rng.uniform(0.1, 2, R).astype(F32), g2)
        for r in np.flatnonzero(greedy):
            np.testing.assert_array_equal(tok[r], base_tok[r])
            np.testing.assert_array_equal(q[r], base_q[r])
    for r in np.flatnonzero(greedy):
        tok, q, _ = O.walk(scores[r:r + 1], ids[r:r + 1], np.zeros((1, S), F32), np.ones(1, F32),
                           np.ones(1, bool))
        np.testing.assert_array_equal(tok[0], base_tok[r])


def test_sampled_q_is_a_distribution():
    rng = np.random.default_rng(5)
    R, S, K = 4, 6, 32
    scores = (rng.standard_normal((R, S, K, K)) * 5).astype(F32)
    ids = rng.integers(0, 1000, (R, S, K))
    tok, q, idx = O.walk(scores, ids, rng.random((R, S)).astype(F32), np.full(R, 0.7, F32),
                         np.zeros(R, bool))
    assert np.all(q > 0) or np.all(q >= 0)
    np.testing.assert_allclose(q.astype(np.float64).sum(-1), 1.0, atol=1e-6)


def test_two_candidate_closed_form():
    # K = 2: softmax(row/T)[0] = 1 / (1 + exp((s1 - s0)/T)); the draw is index
    # 1 exactly when u >= that probability.
    rng = np.random.default_rng(6)
    for _ in range(200):
        s0, s1 = (rng.standard_normal(2) * 4).astype(F32)
        T = F32(rng.uniform(0.2, 3.0))
        p0 = 1.0 / (1.0 + math.exp((float(s1) - float(s0)) / float(T)))
        u = F32(rng.random())
        if abs(float(u) - p0) < 1e-5:
            continue
        scores = np.array([[[[s0, s1], [s0, s1]]]], F32)
        tok, q, idx = O.walk(scores, np.array([[[0, 1]]]), np.array([[u]], F32), np.array([T]),
                             np.zeros(1, bool))
        assert idx[0, 0] == (1 if u >= p0 else 0)
        assert abs(float(q[0, 0, 0]) - p0) < 1e-6


def test_clamped_temperature_reduces_to_greedy():
    # At T -> 0 (clamped to 1e-5) a sampled row picks the argmax wherever the
    # top-2 gap is far above 1e-5.
    rng = np.random.default_rng(7)
    R, S, K = 5, 6, 8
    scores = (np.round(rng.standard_normal((R, S, K, K)) * 8) / 4).astype(F32)
    for r in range(R):
        for s in range(S):
            for j in range(K):
                row = scores[r, s, j]
                row[np.argmax(row)] += 0.5      # unique max with a wide gap
    ids = rng.integers(0, 100, (R, S, K))
    g_tok, _, _ = O.walk(scores, ids, np.zeros((R, S), F32), np.ones(R, F32), np.ones(R, bool))
    s_tok, _, _ = O.walk(scores, ids, rng.random((R, S)).astype(F32), np.zeros(R, F32), np.zeros(R, bool))
    np.testing.assert_array_equal(g_tok, s_tok)


def _all_paths(K, S):
    return list(itertools.product(range(K), repeat=S))


def test_brute_force_enumeration_of_every_path():
    # Tiny lattice (K=4, S=3: 64 paths).  The path probabilities must sum to
    # one; for any uniform vector the walk's path must be the one whose u-box
    # contains it, and the product of the q entries it took must equal the
    # path's probability.
    rng = np.random.default_rng(8)
    K, S = 4, 3
    scores = (rng.standard_normal((1, S, K, K)) * 1.5).astype(F32)
    ids = np.arange(S * K).reshape(1, S, K)
    T = F32(0.9)
    paths = _all_paths(K, S)
    probs = np.array([O.path_probability(scores[0], T, p) for p in paths])
    assert abs(probs.sum() - 1.0) < 1e-12
    for _ in range(300):
        u = rng.random((1, S)).astype(F32)
        tok, q, idx = O.walk(scores, ids, u, np.array([T]), np.zeros(1, bool))
        path = tuple(int(i) for i in idx[0])
        # the u-box of this path: per slot, [C_{c-1}, C_c) under its own row
        prev = 0
        for s, c in enumerate(path):
            row = scores[0, s, prev].astype(np.float64) / float(T)
            p = np.exp(row - row.max()); p /= p.sum()
            cdf = np.cumsum(p)
            lo = 0.0 if c == 0 else cdf[c - 1]
            hi = cdf[c] if c < K - 1 else 1.0
            assert lo - 1e-6 <= float(u[0, s]) < hi + 1e-6
            prev = c
        got = float(np.prod([q[0, s, c] for s, c in enumerate(path)]))
        assert abs(got - probs[paths.index(path)]) < 1e-5


def test_path_frequencies_match_probabilities():
    # Monte-Carlo chi-square: walking with many uniform vectors reproduces the
    # enumerated path distribution.
    rng = np.random.default_rng(9)
    K, S = 3, 3
    scores = (rng.standard_normal((1, S, K, K)) * 1.0).astype(F32)
    ids = np.arange(S * K).reshape(1, S, K)
    T = F32(1.0)
    paths = _all_paths(K, S)
    probs = np.array([O.path_probability(scores[0], T, p) for p in paths])
    n = 20000
    counts = np.zeros(len(paths))
    us = rng.random((n, S)).astype(F32)
    reps = np.repeat(scores, n, axis=0)
    _, _, idx = O.walk(reps, np.repeat(ids, n, axis=0), us, np.full(n, T, F32), np.zeros(n, bool))
    for row in idx:
        counts[paths.index(tuple(int(i) for i in row))] += 1
    expected = probs * n
    keep = expected > 5
    chi2 = float((((counts - expected) ** 2)[keep] / expected[keep]).sum())
    dof = int(keep.sum()) - 1
    # 99.9% quantile of chi-square is below dof + 5 sqrt(2 dof) + 10 for these dof
    assert chi2 < dof + 5 * math.sqrt(2 * dof) + 10, (chi2, dof)


def test_walk_starts_from_anchor_row_and_follows_previous_index():
    # A wrong predecessor row would pick index 0 in slot 1.
    scores = np.zeros((1, 2, 3, 3), F32)
    scores[0, 0, :] = [0.0, 0.0, 9.0]      # slot 0: every row prefers index 2
    scores[0, 1, 0] = [9.0, 0.0, 0.0]      # row 0 of slot 1 would give index 0
    scores[0, 1, 2] = [0.0, 9.0, 0.0]      # row 2 (the taken predecessor) gives 1
    tok, _, idx = O.walk(scores, np.array([[[5, 6, 7], [8, 9, 10]]]), np.zeros((1, 2), F32),
                         np.ones(1, F32), np.ones(1, bool))
    assert idx.tolist() == [[2, 1]] and tok.tolist() == [[7, 9]]


def test_config_pairing_rules():
    O.validate_config(0, 0, 0, 0)
    O.validate_config(4, 64, 64, 8, hidden_size=4096)
    for bad in [(4, 0, 0, 0), (0, 64, 0, 0), (0, 0, 64, 0), (0, 0, 0, 8)]:
        with pytest.raises(ValueError):
            O.validate_config(*bad)
    with pytest.raises(ValueError):
        O.validate_config(4, 48, 0, 0, hidden_size=4096 + 16)
    with pytest.raises(ValueError):
        O.validate_config(0, 0, 8, 4, output_multiplier=0.0)
    with pytest.raises(ValueError):
        O.validate_config(0, 0, 8, 4, final_logit_softcapping=-1.0)


def test_uniform_on_a_cdf_value_counts_that_entry():
    # The draw counts CDF entries at or below u: with four equal scores the CDF
    # is exactly 0.25, 0.5, 0.75, 1 and u = 0.25 selects index 1, u = 0.75
    # selects index 3 (a strict comparison would give 0 and 2).
    scores = np.zeros((2, 1, 4, 4), F32)
    ids = np.tile(np.arange(4), (2, 1, 1))
    _, q, idx = O.walk(scores, ids, np.array([[0.25], [0.75]], F32), np.ones(2, F32), np.zeros(2, bool))
    assert idx[:, 0].tolist() == [1, 3]
    np.testing.assert_array_equal(q, np.full((2, 1, 4), 0.25, F32))


def test_temperature_is_clamped_at_1e_minus_5():
    # T = 0 is staged as 1e-5: a score gap of 1e-5 then becomes a logit gap of
    # exactly 1, so q = (1/(1+e), e/(1+e)) and u = 0.1 draws index 0.
    gap = F32(1e-5)
    scores = np.array([[[[0.0, gap], [0.0, gap]]]], F32)
    _, q, idx = O.walk(scores, np.array([[[0, 1]]]), np.array([[0.1]], F32), np.zeros(1, F32),
                       np.zeros(1, bool))
    p0 = 1.0 / (1.0 + math.e)
    assert idx[0, 0] == 0
    assert abs(float(q[0, 0, 0]) - p0) < 1e-6 and abs(float(q[0, 0, 1]) - (1 - p0)) < 1e-6
