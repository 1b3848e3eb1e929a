"""Tolerances and property checks of the parity tests.

Test infrastructure, like the oracle, but kept apart from it: nothing here is
the method's arithmetic.  These helpers turn the oracle's exact values into
pass/fail bars and check properties that pin a result at any size.

* ``lattice_bar`` -- the lattice entry tolerance
      |got - ref| <= 1e-4 (1 + |unary_c| + sum_k |A_pk u_k B_ck|)
  for the edge formula of "[Spec] DFlash2: local convolution + candidate
  selector" (executive summary: edge(p -> c) = <A[p] (.) project(h), B[c]> +
  unary[c]).  It is relative to the magnitude of the terms summed, so it
  holds an fp32 evaluation (rounding error about sqrt(r) 2^-24 of that
  magnitude) with a wide margin, while a lattice built from a projection
  rounded to bf16 (2^-9 relative per u_k) breaks it: the CPU tests plant
  exactly that mistake.
* ``fp32_sum_bound`` -- the rigorous worst case of an fp32 evaluation in any
  summation order, (H + 8) 2^-24 M1 + (r + 8) 2^-24 M2; printed beside the bar,
  never used as one (it is loose enough to pass bf16 rounding).
* ``softmax_shift`` -- how far softmax entries and CDF values can move when
  every input moves by at most delta.
* ``topk_violations`` -- a complete validity check of one batch of top-K rows
  against its logits, without sorting: it pins the selected set and its order
  exactly (see the docstring), so every row of a large batch can be checked.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
LATTICE_REL = 1e-4


def _pred_rows(ids: np.ndarray, anchor: np.ndarray, r: int, s: int, K: int) -> np.ndarray:
    """Predecessor token ids of every row j of slot s of request r: the
    anchor for slot 0 (every row), else the previous slot's candidates."""
    return np.full(K, anchor[r]) if s == 0 else ids[r, s - 1]


def lattice_term_magnitude(ids, unary, u, anchor, sel_a, sel_b) -> np.ndarray:
    """M[r,s,j,c] = |unary_c| + sum_k |A_pk u_k B_ck| (float64)."""
    A = np.abs(np.asarray(sel_a, np.float64))
    B = np.abs(np.asarray(sel_b, np.float64))
    au = np.abs(np.asarray(u, np.float64))
    un = np.abs(np.where(np.isfinite(unary), unary, 0.0))
    R, S, K = ids.shape
    M = np.empty((R, S, K, K))
    for r in range(R):
        for s in range(S):
            M[r, s] = (A[_pred_rows(ids, anchor, r, s, K)] * au[r, s]) @ B[ids[r, s]].T + un[r, s][None, :]
    return M


def lattice_bar(ids, unary, u, anchor, sel_a, sel_b) -> np.ndarray:
    """Per-entry tolerance 1e-4 (1 + |unary_c| + sum_k |A_pk u_k B_ck|), u the
    exact projection of the hidden rows the GPU used."""
    return LATTICE_REL * (1.0 + lattice_term_magnitude(ids, unary, u, anchor, sel_a, sel_b))


def fp32_sum_bound(ids, unary, h, proj, anchor, sel_a, sel_b) -> np.ndarray:
    """Worst-case rounding error of an fp32 evaluation in any order:
    (H + 8) 2^-24 M1 + (r + 8) 2^-24 M2 with
    M1 = sum_k |A_pk||B_ck| sum_h |P_kh h_h| (the projection's accumulation)
    and M2 = sum_k |A_pk u_k B_ck| + |unary_c| (the edge's accumulation)."""
    h = np.asarray(h, np.float64)
    P = np.asarray(proj, np.float64)
    A = np.abs(np.asarray(sel_a, np.float64))
    B = np.abs(np.asarray(sel_b, np.float64))
    absu = np.abs(h) @ np.abs(P).T
    M2 = lattice_term_magnitude(ids, unary, h @ P.T, anchor, sel_a, sel_b)
    R, S, K = ids.shape
    M1 = np.empty((R, S, K, K))
    for r in range(R):
        for s in range(S):
            M1[r, s] = (A[_pred_rows(ids, anchor, r, s, K)] * absu[r, s]) @ B[ids[r, s]].T
    return (h.shape[-1] + 8) * U32 * M1 + (P.shape[0] + 8) * U32 * M2


def input_shift_bound(ids, dh, proj, anchor, sel_a, sel_b) -> np.ndarray:
    """Bound on how far the exact lattice moves when the hidden rows move by
    dh: sum_k |A_pk||B_ck| |sum_h P_kh dh_h| (the projection is linear)."""
    du = np.abs(np.asarray(dh, np.float64) @ np.asarray(proj, np.float64).T)
    A = np.abs(np.asarray(sel_a, np.float64))
    B = np.abs(np.asarray(sel_b, np.float64))
    R, S, K = ids.shape
    out = np.empty((R, S, K, K))
    for r in range(R):
        for s in range(S):
            out[r, s] = (A[_pred_rows(ids, anchor, r, s, K)] * du[r, s]) @ B[ids[r, s]].T
    return out


def softmax_shift(delta) -> np.ndarray:
    """If every input of a softmax moves by at most delta, every output p_j
    stays within [p_j e^-2delta, p_j e^2delta], so it moves by at most
    e^(2 delta) - 1 (p_j <= 1), and so does every partial sum (CDF value)."""
    return np.expm1(2.0 * np.asarray(delta, np.float64))


def topk_violations(z: np.ndarray, ids: np.ndarray, valid_vocab: int) -> np.ndarray:
    """Rows (indices into z) whose selection is not the top-K under the order
    (value descending, id ascending) over ids < valid_vocab.

    z [n, V] (float32 or float64; -0 == +0 compare equal, -inf ranks last),
    ids [n, K].  Row n passes iff
      (1) every id is < valid_vocab and the K ids are distinct,
      (2) consecutive entries are in order: z strictly decreasing, or equal
          with increasing id,
      (3) the last entry (z_K, id_K) has exactly K - 1 valid entries ahead of
          it: #{v : z_v > z_K} + #{v < id_K : z_v == z_K} == K - 1.
    (1)-(3) make the selection exactly the K first entries of the order: by
    (3) the K-th entry sits at position K, and by (1)-(2) the other K - 1
    selected ids are distinct entries ahead of it, i.e. all of them."""
    z = np.asarray(z)
    ids = np.asarray(ids, np.int64)
    n, K = ids.shape
    bad = np.zeros(n, bool)
    bad |= np.any((ids < 0) | (ids >= valid_vocab), axis=1)
    srt = np.sort(ids, axis=1)
    bad |= np.any(srt[:, 1:] == srt[:, :-1], axis=1)
    safe = np.clip(ids, 0, z.shape[1] - 1)
    zi = np.take_along_axis(z, safe, axis=1)
    if K > 1:
        ok_pair = (zi[:, :-1] > zi[:, 1:]) | ((zi[:, :-1] == zi[:, 1:]) & (ids[:, :-1] < ids[:, 1:]))
        bad |= ~np.all(ok_pair, axis=1)
    zk, idk = zi[:, -1:], ids[:, -1:]
    zv = z[:, :valid_vocab]
    ahead = np.count_nonzero(zv > zk, axis=1)
    col = np.arange(valid_vocab)[None, :]
    ahead += np.count_nonzero((zv == zk) & (col < idk), axis=1)
    bad |= ahead != K - 1
    return np.flatnonzero(bad)
