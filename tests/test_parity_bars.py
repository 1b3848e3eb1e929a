"""CPU pins of the parity tests' own bars and checkers (tests/parity_bars.py).

The lattice bar must hold an fp32 evaluation of the edge formula and must
reject the precision mistake it exists for -- a lattice built from a
projection rounded to bf16 ("[Spec] DFlash2: local convolution + candidate
selector", executive summary: edge(p -> c) = <A[p] (.) project(h), B[c]> +
unary[c]).  The top-K checker must accept the oracle's top-K and reject each
plausible wrong selection (order, ties, padding, a missing entry)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import dflash_oracle as O
from parity_bars import (fp32_sum_bound, lattice_bar, lattice_term_magnitude, softmax_shift,
                         topk_violations)


def test_lattice_bar_hand_worked():
    # R = 1, S = 2, K = 2, r = 2.  Token tables (rows = token ids 0..2):
    A = np.array([[1.0, -2.0], [0.5, 0.0], [3.0, 1.0]])
    B = np.array([[2.0, 1.0], [-1.0, 4.0], [0.0, -0.5]])
    ids = np.array([[[1, 2], [0, 1]]])
    anchor = np.array([2])
    unary = np.array([[[0.5, -1.0], [2.0, -3.0]]])
    u = np.array([[[1.0, -1.0], [2.0, 0.5]]])
    # slot 0: predecessor = anchor 2 for both rows; |A_2 u| = (3, 1)
    #   c = 1 (B_1 = (-1, 4)): 3 * 1 + 1 * 4 = 7, + |unary| 0.5 -> 7.5
    #   c = 2 (B_2 = (0, -0.5)): 0 + 0.5 = 0.5, + 1 -> 1.5
    # slot 1: rows j -> predecessor ids (1, 2); u = (2, 0.5)
    #   p = 1: |A_1 u| = (1, 0); c = 0 (B_0 = (2, 1)): 2, + 2 -> 4; c = 1: 1, + 3 -> 4
    #   p = 2: |A_2 u| = (6, 0.5); c = 0: 12 + 0.5 = 12.5, + 2 -> 14.5; c = 1: 6 + 2 = 8, + 3 -> 11
    want = np.array([[[[7.5, 1.5], [7.5, 1.5]], [[4.0, 4.0], [14.5, 11.0]]]])
    np.testing.assert_array_equal(lattice_term_magnitude(ids, unary, u, anchor, A, B), want)
    np.testing.assert_allclose(lattice_bar(ids, unary, u, anchor, A, B), 1e-4 * (1 + want), rtol=0, atol=0)
    # -inf unary (a masked candidate) adds nothing to the magnitude
    un2 = unary.copy()
    un2[0, 0, 1] = -np.inf
    assert lattice_term_magnitude(ids, un2, u, anchor, A, B)[0, 0, 0, 1] == 0.5


def _selector_case(name, n_req, seed):
    """A lattice case with the shapes and value distributions of a named
    workload: hidden rows ~ N(0, 1) in the storage dtype, tables and
    projection from the workload's recipe, candidate ids uniform."""
    w = W.WORKLOADS[name].replace(n_req=n_req)
    inp = W.make_inputs(w, device="cpu", parts=("selector",), seed=seed)
    h = W.normal((w.n_req, w.slots, w.hidden), 1.0, w.dtype, seed, "hidden", "cpu").to(torch.float64).numpy()
    A = inp["sel_a"].to(torch.float64).numpy()
    B = inp["sel_b"].to(torch.float64).numpy()
    P = inp["proj"].to(torch.float64).numpy()
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, w.valid_vocab, size=(w.n_req, w.slots, w.top_k))
    unary = rng.normal(0.0, 3.0, size=ids.shape)
    anchor = inp["anchor"].numpy()
    return w, h, A, B, P, ids, unary, anchor


def _fp32_lattice(ids, unary, u32, anchor, A, B):
    """The edge formula evaluated in fp32 throughout (the product A * u and
    every accumulation rounded to fp32)."""
    A32, B32, un32 = A.astype(np.float32), B.astype(np.float32), unary.astype(np.float32)
    R, S, K = ids.shape
    out = np.empty((R, S, K, K))
    for r in range(R):
        for s in range(S):
            prev = np.full(K, anchor[r]) if s == 0 else ids[r, s - 1]
            wgt = (A32[prev] * u32[r, s]).astype(np.float32)
            out[r, s] = (wgt @ B32[ids[r, s]].T).astype(np.float32) + un32[r, s][None, :]
    return out


@pytest.mark.parametrize("name,n_req", [("bf16_b16_v151936", 4), ("padded_v201024_k16", 2),
                                        ("stress_r1024_k32", 2)])
def test_lattice_bar_holds_fp32_and_rejects_bf16_projection(name, n_req):
    w, h, A, B, P, ids, unary, anchor = _selector_case(name, n_req, seed=1234)
    u = O.project(h, P)                                       # exact (float64)
    ref = O.lattice(ids, unary, u, anchor, A, B)
    bar = lattice_bar(ids, unary, u, anchor, A, B)
    # an fp32 evaluation (projection accumulated in fp32, then the edge)
    u32 = (h.astype(np.float32) @ P.astype(np.float32).T).astype(np.float32)
    got32 = _fp32_lattice(ids, unary, u32, anchor, A, B)
    r32 = float(np.max(np.abs(got32 - ref) / bar))
    assert r32 <= 0.1, r32                                    # passes with a wide margin
    # the planted mistake: the projection rounded to bf16 before the edge
    u_bf = O.round_to_bf16(u).astype(np.float32)
    got_bf = _fp32_lattice(ids, unary, u_bf, anchor, A, B)
    rbf = float(np.max(np.abs(got_bf - ref) / bar))
    assert rbf > 1.5, rbf                                     # fails the bar
    # the old fp32 worst-case bound is loose enough to pass it (why it is not the bar)
    loose = fp32_sum_bound(ids, unary, h, P, anchor, A, B)
    assert np.all(np.abs(got32 - ref) <= loose)
    print(f"[bar] {name}: fp32 err/bar {r32:.4f}, bf16-projection err/bar {rbf:.2f}, "
          f"bf16 err / fp32 worst-case bound {float(np.max(np.abs(got_bf - ref) / loose)):.3f}")


def _split_bf16_lattice(ids, unary, u32, anchor, A, B):
    """The edge formula with w = A * u rounded to fp32 and then split as
    hi = bf16(w), lo = bf16(w - hi); each of hi * B and lo * B is exact (bf16
    x bf16), summed here exactly (float64) -- the arithmetic of a matrix-core
    tile that keeps the terms bf16 but carries w to ~16 significant bits."""
    A32 = A.astype(np.float32)
    R, S, K = ids.shape
    out = np.empty((R, S, K, K))
    for r in range(R):
        for s in range(S):
            prev = np.full(K, anchor[r]) if s == 0 else ids[r, s - 1]
            w = (A32[prev] * u32[r, s]).astype(np.float32).astype(np.float64)
            hi = O.round_to_bf16(w)
            lo = O.round_to_bf16(w - hi)
            out[r, s] = (hi + lo) @ B[ids[r, s]].T + unary[r, s][None, :].astype(np.float32)
    return out


@pytest.mark.parametrize("name,n_req", [("bf16_b16_v151936", 4), ("stress_r1024_k32", 2)])
def test_lattice_bar_holds_the_split_bf16_tile(name, n_req):
    # The two-term bf16 split of w keeps each product within 2^-18 |w B| of
    # w B: far inside the bar (a single bf16 rounding, 2^-9, breaks it).
    w, h, A, B, P, ids, unary, anchor = _selector_case(name, n_req, seed=99)
    u = O.project(h, P)
    ref = O.lattice(ids, unary, u, anchor, A, B)
    bar = lattice_bar(ids, unary, u, anchor, A, B)
    u32 = (h.astype(np.float32) @ P.astype(np.float32).T).astype(np.float32)
    got = _split_bf16_lattice(ids, unary, u32, anchor, A, B)
    ratio = float(np.max(np.abs(got - ref) / bar))
    assert ratio <= 0.1, ratio
    print(f"[bar] {name}: split-bf16 tile err/bar {ratio:.4f}")


def test_softmax_shift_bounds_random_perturbations():
    rng = np.random.default_rng(7)
    for _ in range(200):
        K = int(rng.integers(2, 33))
        x = rng.normal(0, 4, K)
        d = float(rng.uniform(1e-6, 0.5))
        y = x + rng.uniform(-d, d, K)
        p = np.exp(x - x.max()); p /= p.sum()
        q = np.exp(y - y.max()); q /= q.sum()
        b = float(softmax_shift(d))
        assert np.all(np.abs(p - q) <= b * (1 + 1e-12))
        assert np.all(np.abs(np.cumsum(p) - np.cumsum(q)) <= b * (1 + 1e-12))


def _rows(seed, n, V):
    rng = np.random.default_rng(seed)
    z = np.round(rng.normal(0, 3, (n, V)) * 4) / 4          # coarse: many ties
    z[0] = 0.0                                                # all tied
    z[1, ::3] = -0.0                                          # -0 and +0 mixed
    z[2, V // 2:] = -np.inf
    return z.astype(np.float32)


@pytest.mark.parametrize("K", [1, 5, 32])
def test_topk_checker_accepts_the_oracle_and_rejects_wrong_selections(K):
    V, valid, n = 700, 650, 12
    z = _rows(K, n, V)
    ids, _ = O.topk(z.astype(np.float64), valid, K, 1.0, 0.0)
    assert topk_violations(z, ids, valid).size == 0
    # every planted mistake is caught in the row it is planted in
    mistakes = {}
    row = 3
    # (a) an entry swapped for the next one in the order
    full = np.lexsort((np.arange(valid), -z[row, :valid].astype(np.float64)))[: K + 1]
    m = ids.copy(); m[row, -1] = full[K]; mistakes["next entry instead of the K-th"] = m
    # (b) a padded id
    m = ids.copy(); m[row, -1] = valid + 1; mistakes["padded id"] = m
    # (c) a duplicate
    if K > 1:
        m = ids.copy(); m[row, 1] = m[row, 0]; mistakes["duplicate"] = m
        # (d) order reversed
        m = ids.copy(); m[row] = m[row, ::-1]; mistakes["reversed order"] = m
    # (e) ties resolved to the highest id (all-tied row 0)
    m = ids.copy(); m[0] = np.arange(valid - 1, valid - 1 - K, -1); mistakes["ties to the highest id"] = m
    # (f) ties in the right set but highest-id-first order
    if K > 1:
        m = ids.copy(); m[0] = np.sort(ids[0])[::-1]; mistakes["tie order id descending"] = m
    for what, m in mistakes.items():
        bad = topk_violations(z, m, valid)
        assert bad.size >= 1, what
        assert set(bad.tolist()) <= {0, row}, what


def test_topk_checker_on_a_workload_batch_against_the_oracle():
    # rows with the shapes and values of the padded workload (-inf tail)
    w = W.WORKLOADS["padded_v201024_k16"].replace(n_req=2)
    z = W.make_inputs(w, device="cpu", parts=("logits",))["logits"].to(torch.float32).numpy()[:6]
    ids, _ = O.topk(z.astype(np.float64), w.valid_vocab, w.top_k, w.multiplier, w.softcap)
    assert topk_violations(z, ids, w.valid_vocab).size == 0
    m = ids.copy()
    m[4, 7], m[4, 8] = m[4, 8], m[4, 7]
    assert topk_violations(z, m, w.valid_vocab).tolist() == [4]
