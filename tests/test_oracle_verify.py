"""Pins of the oracle's verify and commit ("[Spec] DFlash2", executive summary
and walk-kernel excerpt: verify checks the drafted tokens against the
distribution the walk actually drew them from, a point mass on greedy rows;
reading: the standard rejection rule of speculative sampling).  The pins fix
the result by the theorem the rule exists for (the committed token is
distributed exactly as the target, found by bisecting the uniforms), greedy
equivalence with the target's own argmax decoding, and hand-built blocks."""
import numpy as np
import pytest

from oracle import dflash_oracle as O


def _one(target, cand, q, tokens, ua, ur, temp=1.0, greedy=False, valid=None):
    target = np.asarray(target, np.float64)
    V = target.shape[-1]
    acc, com = O.verify(target[None], V if valid is None else valid, np.asarray(cand)[None],
                        np.asarray(q, np.float64)[None], np.asarray(tokens)[None], np.asarray(ua, np.float64)[None],
                        np.array([ur], np.float64), np.array([temp]), np.array([greedy]))
    return int(acc[0]), com[0]


def _bisect(f, lo=0.0, hi=1.0, steps=60):
    """Smallest u in [lo, hi) with f(u) true, for f false-then-true on [lo, hi)."""
    if not f(hi * (1 - 1e-15)):
        return hi
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        if f(mid):
            hi = mid
        else:
            lo = mid
    return hi


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_committed_first_token_is_distributed_as_the_target(seed):
    # one slot (S = 1), V = 7, K = 3 candidates drawn from q: for every
    # candidate x the acceptance region of u_accept and, on rejection, the
    # region of u_residual behind every token are found by bisection; the
    # probability of committing v must equal the target's p(v)
    rng = np.random.default_rng(seed)
    V, K = 7, 3
    z = rng.standard_normal((2, V)) * 1.5          # rows: slot 0, bonus position
    T = 0.8
    p = O.target_distribution(z[0], V, T, False)
    cand = rng.choice(V, size=K, replace=False)
    q = rng.dirichlet(np.ones(K))
    prob = np.zeros(V)
    for j, x in enumerate(cand):
        accept = lambda u: _one(z, cand[None], q[None], [x], [u], 0.5, T)[0] == 1
        tau = _bisect(lambda u: not accept(u))         # accepted for u < tau
        prob[x] += q[j] * tau
        if tau < 1.0:
            commit = lambda ur: _one(z, cand[None], q[None], [x], [0.999999], ur, T)[1][0]
            edges = [0.0] + [_bisect(lambda ur, v=v: commit(ur) >= v) for v in range(1, V)] + [1.0]
            for v in range(V):
                prob[v] += q[j] * (1.0 - tau) * (edges[v + 1] - edges[v])
    np.testing.assert_allclose(prob, p, atol=1e-12)


def test_draft_equal_to_the_target_is_always_accepted():
    # every token is a candidate and q = p: min(1, p/q) = 1, all S accepted,
    # the bonus token comes from the last row
    rng = np.random.default_rng(4)
    V, S = 5, 3
    z = rng.standard_normal((S + 1, V))
    cand = np.tile(np.arange(V), (S, 1))
    q = np.stack([O.target_distribution(z[s], V, 1.0, False) for s in range(S)])
    tokens = [1, 4, 0]
    for ua in (0.0, 0.5, 0.9999999):
        acc, com = _one(z, cand, q, tokens, [ua] * S, 0.3)
        assert acc == S and list(com[:S]) == tokens
        bonus_p = O.target_distribution(z[S], V, 1.0, False)
        assert com[S] == int(np.sum(np.cumsum(bonus_p) <= 0.3))


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_greedy_requests_commit_the_targets_own_greedy_decoding(seed):
    # greedy rows: q is a point mass on the drafted token and the target is a
    # point mass on its argmax (lowest id on ties); the committed tokens are
    # the target's argmax at every position up to and including the first
    # mismatch (or the bonus position), whatever the uniforms
    rng = np.random.default_rng(seed)
    V, K, S = 12, 4, 5
    z = np.round(rng.standard_normal((S + 1, V)) * 2) / 2     # coarse values: ties occur
    top = [min(range(V), key=lambda v: (-z[s, v], v)) for s in range(S + 1)]
    for n_match in range(S + 1):
        tokens = [top[s] if s < n_match else (top[s] + 1) % V for s in range(S)]
        cand = np.array([[t] + [int(v) for v in rng.choice([u for u in range(V) if u != t], K - 1, replace=False)]
                         for t in tokens])
        q = np.zeros((S, K))
        q[:, 0] = 1.0
        acc, com = _one(z, cand, q, tokens, rng.random(S), float(rng.random()), greedy=True)
        assert acc == n_match
        assert list(com[:n_match + 1]) == top[:n_match + 1]
        assert all(c == -1 for c in com[n_match + 1:])


def test_rejection_at_a_middle_slot_stops_the_block():
    # slot 0's token has p = q (kept for any u); slot 1's token has p = 0
    # (always rejected); the correction comes from max(0, p - q) of row 1
    V = 4
    z = np.array([[0.0, 0.0, 0.0, 0.0], [5.0, -np.inf, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    cand = np.array([[0, 1, 2], [1, 2, 3], [0, 1, 2]])
    q = np.array([[0.25, 0.5, 0.25], [0.6, 0.3, 0.1], [1.0, 0.0, 0.0]])
    acc, com = _one(z, cand, q, [0, 1, 2], [0.9, 0.0, 0.0], 0.0)
    assert acc == 1 and com[0] == 0 and com[2] == -1 and com[3] == -1
    p1 = O.target_distribution(z[1], V, 1.0, False)
    residual = np.maximum(0.0, p1 - np.array([0.0, 0.6, 0.3, 0.1]))
    assert com[1] == 0 and residual[0] > 0            # u_residual = 0 picks the first positive entry


def test_padded_ids_are_never_committed():
    # logits past valid_vocab are huge but excluded, in the residual and the bonus
    V, valid = 6, 4
    z = np.array([[0.0, 0.1, 0.2, 0.3, 50.0, 50.0], [0.0, 0.0, 0.0, 1.0, 90.0, 90.0]])
    cand = np.array([[0, 1, 2]])
    q = np.array([[1.0, 0.0, 0.0]])
    for ur in (0.0, 0.5, 0.999):
        for ua in (0.0, 0.99):
            _, com = _one(z, cand, q, [0], [ua], ur, valid=valid)
            assert all(c < valid for c in com if c >= 0)
