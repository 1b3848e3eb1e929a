"""Plain CPU oracle of the DFlash2 draft-block path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, calls or links this module; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` do.
It shares no code, table or constant with the HIP path.

Every function is the plain definition written out, slowly and readably, in
numpy float64 (bf16 and fp32 inputs decode to float64 exactly), except the
walk, whose precision the pages fix at fp32.  Sources (page titles; sections):

  [DF2]  "[Spec] DFlash2: local convolution + candidate selector"
         (sglang PR 35371): executive summary (the edge formula and the
         lossless q contract), implementation breakdown (the six config
         fields, their pairing, the unary transform, the deterministic
         top-k), and the code excerpts for the grouped conv, the selector
         lattice hand-off, the draft sampler and the walk kernel.
  [DSP]  "DSpark padded-vocab d2t fix" (vllm PR 55133): logical vocab
         200058 vs physical 201024, and the requirement that padded ids are
         never sampled.

Readings where the pages are silent:
  * conv: coefficient index is the OUTPUT token i with tap t, applied to
    x[i - t]; delta carries a tap axis, delta[i, t, g]; block position is the
    flat token index modulo the block size.
  * transform: y = m * z, then y = cap * tanh(y / cap) when cap > 0; entries
    that are -inf stay -inf.  The transform's body is not printed, so its
    exact form is "parity unpinned" beyond identity, bounds, symmetry and
    slope at 0.
  * top-k order: transformed value descending, ties by lowest token id; ids
    at or beyond the logical vocab are never selected.
  * lattice: A and B are [V, r] per-token tables, project(h) = P h with
    P [r, H]; slot 0's predecessor is the anchor.
  * candidates from hidden states: the dense head's logits are the exact
    sums rounded once to the storage dtype, and the top-k ranks them.
  * conv module: the kernel projection's output (both sides' coefficients)
    is the exact sums rounded once to the storage dtype; its 2*T*G outputs
    per token are ordered (side, tap, group).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------------------
# Number formats (decoding/rounding only; no method arithmetic)
# ---------------------------------------------------------------------------

def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64.  bfloat16 = 1 sign, 8 exponent bits (the fp32 range), 8
    significant bits.  Done directly from float64 (no detour through fp32,
    which would round twice)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    finite = np.isfinite(v) & (v != 0)
    f, e = np.frexp(v[finite])          # v = f * 2**e, 0.5 <= |f| < 1
    # normal bf16: 8 significant bits -> step 2**(e-8); below 2**-126 the
    # step is fixed at 2**-133 (subnormals).
    step_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(f, e - step_exp))   # rint = round half to even
    r = np.ldexp(q, step_exp)
    r[np.abs(r) >= 2.0 ** 128] = np.copysign(np.inf, r[np.abs(r) >= 2.0 ** 128])
    # the largest bf16 is (2 - 2**-7) * 2**127; anything that rounds above it
    # is infinite (handled by the line above since q*2**step would be 2**128)
    out[finite] = r
    return out


def round_to_dtype(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(v)
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Config contract  [DF2] implementation breakdown (config fields, pairing) and
# the grouped-conv module constructor (hidden % group_size).
# ---------------------------------------------------------------------------

def validate_config(conv_kernel_size: int, conv_group_size: int, selector_rank: int,
                    selector_top_k: int, output_multiplier: float = 1.0,
                    final_logit_softcapping: float = 0.0, hidden_size: Optional[int] = None,
                    block_size: Optional[int] = None) -> None:
    """Raise ValueError if the draft config breaks the pages' contract.

    The conv fields come as a pair and so do the selector fields: both zero
    (feature off) or both positive.  A conv group size must divide the hidden
    width.  Multiplier must be positive and finite (the top-k order is taken
    on raw logits, which needs a strictly increasing transform) and the
    softcap non-negative (0 = off)."""
    if (conv_kernel_size > 0) != (conv_group_size > 0) or conv_kernel_size < 0 or conv_group_size < 0:
        raise ValueError("conv_kernel_size and conv_group_size must be set together")
    if (selector_rank > 0) != (selector_top_k > 0) or selector_rank < 0 or selector_top_k < 0:
        raise ValueError("selector_rank and selector_top_k must be set together")
    if not (math.isfinite(output_multiplier) and output_multiplier > 0):
        raise ValueError("output_multiplier must be finite and > 0")
    if not (math.isfinite(final_logit_softcapping) and final_logit_softcapping >= 0):
        raise ValueError("final_logit_softcapping must be finite and >= 0")
    if hidden_size is not None and conv_group_size > 0 and hidden_size % conv_group_size:
        raise ValueError("conv_group_size must divide hidden_size")
    if block_size is not None and block_size < 1:
        raise ValueError("block_size must be >= 1")


# ---------------------------------------------------------------------------
# Step 1: block-causal grouped dynamic depthwise convolution
# [DF2] code excerpt of the grouped conv: out[i,c] = sum_t (base + delta) x[i-t,c],
# with taps that reach before the start of the token's block zeroed.
# ---------------------------------------------------------------------------

def conv(x: np.ndarray, base: np.ndarray, delta: np.ndarray, block_size: int,
         group_size: int) -> np.ndarray:
    """x [N, H], base [T, H], delta [N, T, G] -> out [N, H] (float64).

    Walks each block on its own (the block start is r * B), so the in-block
    position is the loop index j, with no modulo or bit trick."""
    x = np.asarray(x, np.float64)
    base = np.asarray(base, np.float64)
    delta = np.asarray(delta, np.float64)
    N, H = x.shape
    T = base.shape[0]
    if N % block_size:
        raise ValueError("token count must be a whole number of blocks")
    out = np.zeros((N, H))
    for b0 in range(0, N, block_size):
        for j in range(block_size):
            i = b0 + j
            for t in range(min(T, j + 1)):          # taps before the block start are zero
                coeff = base[t] + np.repeat(delta[i, t], group_size)   # channel c uses group c // gs
                out[i] += coeff * x[i - t]
    return out


# ---------------------------------------------------------------------------
# Step 1b: the conv module's kernel projection and its two sides
# [DF2] code excerpt of the grouped conv module: the base kernel is laid out
# [input/output side, tap, channel] and starts as the identity (tap 0 = 1);
# one bias-free linear map of a token's input gives 2 * T * G coefficients,
# read as [2, T, G]; prepare convolves the input with side 0 and hands side
# 1's coefficients on, and finish convolves the sublayer output with side 1.
# ---------------------------------------------------------------------------

def conv_projection(x: np.ndarray, weight: np.ndarray, dtype: str) -> np.ndarray:
    """x [N, H], weight [2*T*G, H] (the linear map's [out, in] layout) ->
    coefficients [N, 2*T*G]: each the exact sum of its H products, rounded
    once to the storage dtype (the map's output dtype)."""
    z = np.asarray(x, np.float64) @ np.asarray(weight, np.float64).T
    return round_to_dtype(z, dtype)


def conv_prepare(x: np.ndarray, weight: np.ndarray, base2: np.ndarray, block_size: int,
                 group_size: int, dtype: str):
    """x [N, H], weight [2*T*G, H], base2 [2, T, H] -> (out [N, H] float64,
    unrounded; coefficients [N, 2, T, G] in dtype).  out convolves x with
    side 0; side 1's coefficients, coefficients[:, 1], are what finish uses."""
    N, H = np.asarray(x).shape
    T = np.asarray(base2).shape[1]
    G = H // group_size
    coeff = conv_projection(x, weight, dtype).reshape(N, 2, T, G)
    return conv(x, np.asarray(base2)[0], coeff[:, 0], block_size, group_size), coeff


def conv_finish(y: np.ndarray, coeff: np.ndarray, base2: np.ndarray, block_size: int,
                group_size: int) -> np.ndarray:
    """y [N, H] (the sublayer output), coeff [N, 2, T, G] from conv_prepare ->
    y convolved with side 1 (float64, unrounded)."""
    return conv(y, np.asarray(base2)[1], np.asarray(coeff)[:, 1], block_size, group_size)


# ---------------------------------------------------------------------------
# Step 2: unary transform  [DF2] implementation breakdown: output_multiplier
# and final_logit_softcapping jointly define the unary logit transform.
# ---------------------------------------------------------------------------

def transform(z: np.ndarray, multiplier: float, softcap: float) -> np.ndarray:
    z = np.asarray(z, np.float64)
    y = multiplier * z
    if softcap > 0:
        y = softcap * np.tanh(y / softcap)
    return np.where(np.isneginf(z), -np.inf, y)


# ---------------------------------------------------------------------------
# Step 3: per-slot top-K  [DF2] implementation breakdown (deterministic top-k)
# and [DSP] (padded ids must never be sampled).
# ---------------------------------------------------------------------------

def topk(logits: np.ndarray, valid_vocab: int, top_k: int, multiplier: float,
         softcap: float):
    """logits [rows, V] -> ids [rows, K] int64, unary [rows, K] float64.

    Each row is fully sorted by (eligible first, value descending, id
    ascending) and the first K entries are taken.  Eligible = id <
    valid_vocab.  The transform is strictly increasing for multiplier > 0, so
    ranking the raw logit equals ranking the transformed value (taken on the
    exact input values; -0 and +0 are equal)."""
    z = np.asarray(logits, np.float64)
    rows, V = z.shape
    if np.isnan(z).any():
        raise ValueError("NaN logits are outside the method's domain")
    if not (0 < top_k <= valid_vocab <= V):
        raise ValueError("need 0 < top_k <= valid_vocab <= vocab")
    ids = np.arange(V)
    ineligible = ids >= valid_vocab
    out_ids = np.empty((rows, top_k), np.int64)
    for n in range(rows):
        order = np.lexsort((ids, -z[n], ineligible))   # last key is the primary key
        out_ids[n] = order[:top_k]
    unary = transform(np.take_along_axis(z, out_ids, axis=1), multiplier, softcap)
    return out_ids, unary


# ---------------------------------------------------------------------------
# Candidates straight from the slot hidden states  [DF2] implementation
# breakdown and risk notes: compute_candidates multiplies the hidden rows by
# the target lm_head weight taken as a dense matrix, then applies the unary
# transform and the deterministic top-k.
# Reading: the dense head's product is returned in the model's storage dtype
# (a bf16 matmul returns bf16), so the logits are the exact sums rounded once
# to that dtype, and the top-k ranks those rounded values.
# ---------------------------------------------------------------------------

def lm_head_logits(h: np.ndarray, weight: np.ndarray, dtype: str) -> np.ndarray:
    """h [rows, H], weight [V, H] -> logits [rows, V]: every product summed
    exactly enough in float64 (each bf16 x bf16 product is exact, and float64
    holds the sum of H of them to far below the bf16 step), then rounded once
    to the storage dtype."""
    z = np.asarray(h, np.float64) @ np.asarray(weight, np.float64).T
    return round_to_dtype(z, dtype)


def lm_head_sum_bound(h: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """Per logit, a bound on how far an fp32 accumulation of the H exact
    products (in any order) can land from the exact sum: H * 2^-24 *
    sum_k |h_k| |w_k| (the classic n*u bound for a sum of n terms)."""
    a = np.abs(np.asarray(h, np.float64))
    b = np.abs(np.asarray(weight, np.float64))
    return a.shape[1] * 2.0 ** -24 * (a @ b.T)


def compute_candidates(h: np.ndarray, weight: np.ndarray, valid_vocab: int, top_k: int,
                       multiplier: float, softcap: float, dtype: str):
    """h [rows, H] -> (ids [rows, K], unary [rows, K]): the top-k of the
    rounded head logits, as topk() ranks any logits."""
    return topk(lm_head_logits(h, weight, dtype), valid_vocab, top_k, multiplier, softcap)


# ---------------------------------------------------------------------------
# Step 4 and 5: rank-r projection and the selector lattice
# [DF2] executive summary: edge(p -> c) = <A[p] (.) project(h), B[c]> + unary[c],
# scored over adjacent slots; slot 0's predecessor is the verified anchor
# (draft-sampler code excerpt: position 0 of the block is the anchor).
# ---------------------------------------------------------------------------

def project(h: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """h [..., H], proj [r, H] -> u [..., r] = P h (float64 matmul)."""
    return np.asarray(h, np.float64) @ np.asarray(proj, np.float64).T


def lattice(ids: np.ndarray, unary: np.ndarray, u: np.ndarray, anchor: np.ndarray,
            sel_a: np.ndarray, sel_b: np.ndarray) -> np.ndarray:
    """ids [R,S,K], unary [R,S,K], u [R,S,r], anchor [R], A,B [V,r]
    -> scores [R,S,K(prev),K(cur)] float64."""
    A = np.asarray(sel_a, np.float64)
    Bt = np.asarray(sel_b, np.float64)
    R, S, K = ids.shape
    scores = np.empty((R, S, K, K))
    for r in range(R):
        for s in range(S):
            prev = np.full(K, anchor[r]) if s == 0 else ids[r, s - 1]
            left = A[prev] * u[r, s]                       # A[p] (.) project(h), one row per p
            scores[r, s] = left @ Bt[ids[r, s]].T + unary[r, s][None, :]
    return scores


# ---------------------------------------------------------------------------
# Step 6: the per-request walk  [DF2] walk-kernel code excerpt and executive
# summary (greedy rows emit a point mass; sampled rows return the softmax q
# they drew from).  The pages' walk loads scores as fp32 and draws with fp32
# uniforms, so this walk is evaluated in fp32, in the pages' order: divide by
# the temperature, subtract the row max, exponentiate, normalise by the sum,
# accumulate the CDF, and count the CDF entries at or below the uniform.
# Sums and the CDF run left to right.  exp is the fp32 value nearest e^x
# (float64 exp rounded once).  Temperatures are clamped to >= 1e-5, as the
# sampler's staging step does.
# ---------------------------------------------------------------------------

def _softmax_cdf_f32(row: np.ndarray, temperature: float):
    t = max(F32(temperature), F32(1e-5))
    scaled = (row.astype(F32) / t).astype(F32)
    shifted = (scaled - scaled.max()).astype(F32)
    e = np.exp(shifted.astype(np.float64)).astype(F32)
    total = F32(0)
    for v in e:                                   # left-to-right sum
        total = F32(total + v)
    p = (e / total).astype(F32)
    cdf = np.empty_like(p)
    acc = F32(0)
    for j, v in enumerate(p):                     # left-to-right CDF
        acc = F32(acc + v)
        cdf[j] = acc
    return p, cdf


def walk(scores: np.ndarray, ids: np.ndarray, uniforms: np.ndarray,
         temperatures: np.ndarray, greedy: np.ndarray, return_margins: bool = False):
    """scores [R,S,K,K] (fp32 values), ids [R,S,K], uniforms [R,S] fp32,
    temperatures [R], greedy [R] bool -> tokens [R,S] int64, q [R,S,K] fp32,
    idx [R,S] int64 (+ margins [R,S] float64: greedy top1 - top2, sampled
    min_j |u - C_j| over the boundaries that can change the draw)."""
    sc = np.asarray(scores).astype(F32)
    R, S, K = ids.shape
    tokens = np.empty((R, S), np.int64)
    idxs = np.empty((R, S), np.int64)
    q = np.zeros((R, S, K), F32)
    margins = np.full((R, S), np.inf)
    for r in range(R):
        prev = 0                                  # start from the anchor's row
        for s in range(S):
            row = sc[r, s, prev]
            if greedy[r]:
                best = row.max()
                idx = int(np.flatnonzero(row == best)[0])      # lowest index among ties
                q[r, s, idx] = 1.0
                if K > 1:
                    margins[r, s] = float(best) - float(np.sort(row)[-2])
            else:
                u = F32(uniforms[r, s])
                p, cdf = _softmax_cdf_f32(row, float(temperatures[r]))
                idx = min(int(np.count_nonzero(u >= cdf)), K - 1)
                q[r, s] = p
                if K > 1:
                    margins[r, s] = float(np.min(np.abs(np.float64(u) - cdf[: K - 1].astype(np.float64))))
            tokens[r, s] = ids[r, s, idx]
            idxs[r, s] = idx
            prev = idx
    if return_margins:
        return tokens, q, idxs, margins
    return tokens, q, idxs


def path_probability(scores: np.ndarray, temperature: float, path) -> float:
    """Probability (float64) that a sampled walk over one request's scores
    [S,K,K] follows ``path`` (candidate indices per slot): the product of the
    per-slot softmax(row / T) entries along the path, starting from row 0."""
    t = max(float(F32(temperature)), float(F32(1e-5)))
    prev, prob = 0, 1.0
    for s, c in enumerate(path):
        row = np.asarray(scores[s, prev], np.float64) / t
        w = np.exp(row - row.max())
        prob *= w[c] / w.sum()
        prev = c
    return prob


# ---------------------------------------------------------------------------
# Whole block  [DF2] draft-sampler code excerpt: drop the anchor position,
# select candidates per slot, build the lattice, walk.
# ---------------------------------------------------------------------------

def propose_block(inp: Dict[str, np.ndarray], *, block_size: int, group_size: int,
                  valid_vocab: int, top_k: int, multiplier: float, softcap: float,
                  dtype: str, side: int = 0, h_override: Optional[np.ndarray] = None):
    """End-to-end oracle from raw inputs (all float64 arrays holding the input
    bits).  Returns a dict with conv_out (float64), conv_out_q (rounded to the
    storage dtype), ids, unary, u, scores, tokens, q, idx, margins.

    The proposal hidden state of slot s of request r is conv-output row
    r*B + 1 + s (a stand-in for the draft stack, which sits between the conv
    and the selector on the pages and is outside this path)."""
    x = inp["x"]
    T = inp["base"].shape[1]
    base = inp["base"][side]
    delta = inp["delta"][:, side]
    out = conv(x, base, delta, block_size, group_size)
    out_q = round_to_dtype(out, dtype)
    R = x.shape[0] // block_size
    S = block_size - 1
    H = x.shape[1]
    h = (out_q if h_override is None else h_override).reshape(R, block_size, H)[:, 1:, :]
    ids, unary = topk(inp["logits"], valid_vocab, top_k, multiplier, softcap)
    ids = ids.reshape(R, S, top_k)
    unary = unary.reshape(R, S, top_k)
    u = project(h, inp["proj"])
    scores = lattice(ids, unary, u, inp["anchor"], inp["sel_a"], inp["sel_b"])
    tokens, q, idx, margins = walk(scores.astype(F32), ids, inp["uniforms"], inp["temperatures"],
                                   inp["greedy_mask"], return_margins=True)
    return dict(conv_out=out, conv_out_q=out_q, h=h, ids=ids, unary=unary, u=u, scores=scores,
                tokens=tokens, q=q, idx=idx, margins=margins)


# ---------------------------------------------------------------------------
# Verify and commit  [DF2] executive summary and walk-kernel excerpt: verify
# is lossless because the proposal distribution it checks against is the one
# the walk actually drew from (a point mass on greedy rows, the softmax the
# token was sampled from otherwise); the worker then commits the accepted
# block with the bonus token placed after it.  The pages do not print the
# verify itself; this is the standard rejection rule of speculative sampling
# (accept a drafted token x with probability min(1, p(x) / q(x)); on the
# first rejection draw from max(0, p - q) renormalised; after S acceptances
# draw a bonus token from the next position's p).
# ---------------------------------------------------------------------------

def target_distribution(z: np.ndarray, valid_vocab: int, temperature: float, greedy: bool) -> np.ndarray:
    """z [V] target logits -> p [V] (float64): the point mass at the lowest-id
    maximum for a greedy request, softmax(z / T) with T clamped to >= 1e-5
    otherwise; ids at or past valid_vocab (and -inf logits) get 0."""
    z = np.asarray(z, np.float64)[:valid_vocab]
    p = np.zeros(valid_vocab)
    if greedy:
        p[int(np.argmax(z))] = 1.0                   # argmax returns the first (lowest) id of the max
        return p
    y = z / max(float(temperature), 1e-5)
    e = np.exp(y - np.max(y))
    return e / np.sum(e)


def inverse_cdf(weights: np.ndarray, u: float) -> int:
    """The first index whose running sum (in index order) exceeds u times the
    total: #{v : C_v <= u * C_last}, capped at the last positive entry."""
    c = np.cumsum(np.asarray(weights, np.float64))
    v = int(np.sum(c <= u * c[-1]))
    last = int(np.flatnonzero(np.asarray(weights) > 0)[-1])
    return min(v, last)


def verify(target_logits: np.ndarray, valid_vocab: int, cand_ids: np.ndarray, q: np.ndarray,
           tokens: np.ndarray, u_accept: np.ndarray, u_residual: np.ndarray, temperatures: np.ndarray,
           greedy_mask: np.ndarray):
    """target_logits [R, S+1, V] (row s: the target's logits for the token at
    slot s given the block before it; row S: after the whole block);
    cand_ids [R, S, K], q [R, S, K] (the walk's candidates and the
    distribution each token was drawn from), tokens [R, S];
    u_accept [R, S], u_residual [R] uniforms in [0, 1).
    Returns (accepted [R]: drafted tokens kept, committed [R, S+1]: those
    tokens then the correction or bonus token, -1 after)."""
    R, S = np.asarray(tokens).shape
    accepted = np.zeros(R, np.int64)
    committed = np.full((R, S + 1), -1, np.int64)
    for r in range(R):
        greedy = bool(greedy_mask[r])
        n = 0
        while n < S:
            x = int(tokens[r, n])
            p = target_distribution(target_logits[r, n], valid_vocab, temperatures[r], greedy)
            hits = np.flatnonzero(np.asarray(cand_ids[r, n]) == x)
            qx = float(q[r, n, hits[0]]) if len(hits) else 0.0   # a token outside the candidates has q = 0
            px = float(p[x]) if x < valid_vocab else 0.0
            if not (float(u_accept[r, n]) * qx < px):         # rejected: draw from max(0, p - q)
                residual = p.copy()
                for jj, v in enumerate(np.asarray(cand_ids[r, n])):
                    if v < valid_vocab:
                        residual[v] = max(0.0, residual[v] - float(q[r, n, jj]))
                if not np.any(residual > 0):
                    residual = p
                committed[r, :n] = tokens[r, :n]
                committed[r, n] = inverse_cdf(residual, float(u_residual[r]))
                break
            n += 1
        if n == S:                                            # every drafted token kept: bonus token
            p = target_distribution(target_logits[r, S], valid_vocab, temperatures[r], greedy)
            committed[r, :S] = tokens[r]
            committed[r, S] = inverse_cdf(p, float(u_residual[r]))
        accepted[r] = n
    return accepted, committed


# ---------------------------------------------------------------------------
# Counter-based uniforms for a captured step  [DF2] worker excerpt: the
# sampler draws its uniforms inside the captured graph with a counter-based
# generator (Philox), so every replay can draw fresh numbers without host
# work.  Philox-4x32-10 as published by Salmon, Moraes, Dror and Shaw
# ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds of
# two 32x32 -> 64-bit multiplications with the Weyl-sequence key schedule.
# ---------------------------------------------------------------------------

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)
_MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """counter: 4 words, key: 2 words (unsigned 32-bit) -> 4 output words."""
    x0, x1, x2, x3 = (int(c) & _MASK32 for c in counter)
    k0, k1 = (int(k) & _MASK32 for k in key)
    for rnd in range(10):
        p0 = _PHILOX_M[0] * x0
        p1 = _PHILOX_M[1] * x2
        x0, x1, x2, x3 = ((p1 >> 32) ^ x1 ^ k0, p1 & _MASK32, (p0 >> 32) ^ x3 ^ k1, p0 & _MASK32)
        k0 = (k0 + _PHILOX_W[0]) & _MASK32
        k1 = (k1 + _PHILOX_W[1]) & _MASK32
    return (x0, x1, x2, x3)


def philox_uniforms(seed: int, offset: int, n: int) -> np.ndarray:
    """n uniforms in [0, 1) (float32 values, multiples of 2^-24): element i is
    word i % 4 of block offset + i // 4 (64-bit counter in the first two
    counter words, the others zero; key = the seed's two 32-bit halves),
    keeping its top 24 bits."""
    out = np.empty(n, np.float64)
    key = (seed & _MASK32, (seed >> 32) & _MASK32)
    for b in range((n + 3) // 4):
        c = (offset + b) & 0xFFFFFFFFFFFFFFFF
        words = philox4x32_10((c & _MASK32, c >> 32, 0, 0), key)
        for j in range(4):
            i = 4 * b + j
            if i < n:
                out[i] = (words[j] >> 8) * 2.0 ** -24
    return out
