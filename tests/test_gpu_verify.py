"""GPU parity of dflash_verify (verify and commit of a drafted block, "[Spec]
DFlash2" executive summary and walk-kernel excerpt; the rule is the standard
rejection rule of speculative sampling) against the oracle.

Bar: accepted counts and committed tokens equal the oracle's exactly.  Both
sides decide in fp64; a decision may differ only where the two fp64
evaluations straddle it (|u q(x) - p(x)| or the inverse-CDF crossing within
1e-9 relative), and such a case must show that margin when it occurs.
Greedy requests are also checked structurally: the committed tokens are the
target's own argmax decoding."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
from gpu_helpers import DEV, f64, require_gpu, say
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu


def _inputs(R, S, V, K, seed, dtype=torch.bfloat16, valid=None, greedy_frac=0.5, match_frac=0.7):
    """Target logits and a drafted block whose tokens often agree with the
    target (so blocks run past the first slots): candidates are distinct ids
    holding the target's argmax with probability match_frac, q a softmax over
    them, tokens drawn from q."""
    g = torch.Generator().manual_seed(seed)
    valid = V if valid is None else valid
    z = (torch.randn((R, S + 1, V), generator=g) * 3.0).to(dtype)
    if valid < V:
        z[:, :, valid:] = 60.0                      # padded ids: large but excluded
    zf = z.float()
    cand = torch.zeros((R, S, K), dtype=torch.int64)
    q = torch.zeros((R, S, K), dtype=torch.float32)
    tok = torch.zeros((R, S), dtype=torch.int64)
    greedy = (torch.rand(R, generator=g) < greedy_frac).to(torch.uint8)
    for r in range(R):
        for s in range(S):
            top = int(torch.argmax(zf[r, s, :valid]))
            ids = torch.randperm(valid, generator=g)[:K]
            if float(torch.rand(1, generator=g)) < match_frac and not bool((ids == top).any()):
                ids[0] = top
            cand[r, s] = ids
            w = torch.softmax(zf[r, s, ids] + torch.randn(K, generator=g), dim=0)
            if greedy[r]:
                j = int(torch.argmax(w))
                q[r, s] = 0.0
                q[r, s, j] = 1.0
            else:
                q[r, s] = w
                j = int(torch.multinomial(w, 1, generator=g))
            tok[r, s] = ids[j]
    ua = torch.rand((R, S), generator=g)
    ur = torch.rand(R, generator=g)
    temps = 0.5 + torch.rand(R, generator=g)
    return dict(z=z, cand=cand, q=q, tok=tok, ua=ua, ur=ur, temps=temps, greedy=greedy, valid=valid)


def _margins_ok(d, r, got_n):
    """True when request r's differing outcome sits on an fp64 decision edge."""
    z = f64(d["z"][r])
    greedy = bool(d["greedy"][r])
    T = float(d["temps"][r])
    for s in range(z.shape[0]):
        p = O.target_distribution(z[s], d["valid"], T, greedy)
        if s < z.shape[0] - 1:
            x = int(d["tok"][r, s])
            hits = np.flatnonzero(d["cand"][r, s].numpy() == x)
            qx = float(d["q"][r, s, hits[0]]) if len(hits) else 0.0
            px = p[x] if x < d["valid"] else 0.0
            if abs(float(d["ua"][r, s]) * qx - px) <= 1e-9 * max(px, 1e-300):
                return True
        c = np.cumsum(p)
        if np.min(np.abs(c - float(d["ur"][r]) * c[-1])) <= 1e-9 * c[-1]:
            return True
    return False


def _run(R, S, V, K, seed, d=None, **kw):
    require_gpu()
    d = _inputs(R, S, V, K, seed, **kw) if d is None else d
    say(f"dflash_verify R={R} S={S} V={V} K={K} valid={d['valid']} seed={seed}")
    acc, com = D.dflash_verify(d["z"].to(DEV), d["cand"].to(DEV), d["q"].to(DEV), d["tok"].to(DEV),
                               d["ua"].to(DEV), d["ur"].to(DEV), d["temps"].to(DEV), d["greedy"].to(DEV),
                               valid_vocab=d["valid"])
    torch.cuda.synchronize()
    acc, com = acc.cpu().numpy(), com.cpu().numpy()
    ra, rc = O.verify(f64(d["z"]), d["valid"], d["cand"].numpy(), d["q"].double().numpy(), d["tok"].numpy(),
                      d["ua"].double().numpy(), d["ur"].double().numpy(), d["temps"].double().numpy(),
                      d["greedy"].numpy())
    edge = 0
    for r in range(R):
        if acc[r] != ra[r] or not np.array_equal(com[r], rc[r]):
            assert _margins_ok(d, r, acc[r]), (r, acc[r], ra[r], com[r], rc[r])
            edge += 1
    # greedy requests: the committed tokens are the target's argmax decoding
    zf = d["z"].float()
    for r in np.flatnonzero(d["greedy"].numpy()):
        n = int(acc[r])
        want = [int(torch.argmax(zf[r, s, :d["valid"]])) for s in range(n + 1)]
        assert list(com[r, :n + 1]) == want
    for r in range(R):                            # kept tokens, one committed draw, then -1
        n = int(acc[r])
        assert 0 <= n <= S and 0 <= com[r, n] < d["valid"] and np.all(com[r, n + 1:] == -1)
    print(f"[verify] R={R} S={S} V={V}: mean accepted {acc.mean():.2f}, {edge} decisions on an fp64 edge", flush=True)
    return acc, com


@pytest.mark.parametrize("R,S,V,K,seed", [(16, 5, 1000, 8, 1), (8, 3, 37, 4, 2), (5, 1, 300, 1, 3),
                                          (12, 15, 5003, 32, 4), (4, 0, 64, 2, 5), (9, 2, 5, 2, 13)])
def test_verify_matches_the_oracle(R, S, V, K, seed):
    # (V = 5: rows shorter than one 16-byte vector, all single elements)
    _run(R, S, V, K, seed)


def test_verify_fp32_rows_shorter_than_a_vector():
    _run(7, 2, 3, 2, 14, dtype=torch.float32)


def test_verify_fp32_logits_and_padded_vocab():
    _run(10, 4, 700, 8, 6, dtype=torch.float32, valid=650)


def test_verify_bench_shape():
    # 32 requests x 15 slots over the 151936-id vocabulary, K = 8
    _run(32, 15, 151936, 8, 7)


def test_verify_all_greedy_and_all_sampled():
    a, _ = _run(16, 7, 2000, 8, 8, greedy_frac=1.0, match_frac=1.0)
    assert np.all(a == 7)                         # every drafted token is the target's argmax: all kept
    _run(16, 7, 2000, 8, 9, greedy_frac=0.0)


def test_verify_empty_is_a_no_op():
    require_gpu()
    e = torch.zeros((0, 3, 16), dtype=torch.bfloat16, device=DEV)
    acc, com = D.dflash_verify(e, torch.zeros((0, 2, 4), dtype=torch.int64, device=DEV),
                               torch.zeros((0, 2, 4), device=DEV), torch.zeros((0, 2), dtype=torch.int64, device=DEV),
                               torch.zeros((0, 2), device=DEV), torch.zeros(0, device=DEV), torch.zeros(0, device=DEV),
                               torch.zeros(0, dtype=torch.uint8, device=DEV))
    assert acc.shape == (0,) and com.shape == (0, 3)


def test_verify_large_vocab_ragged_rows():
    # sampled requests whose chunk sums span every segment: fp32 rows with a
    # ragged valid vocabulary, and bf16 rows of an odd length (so each row
    # starts at a different offset from a 16-byte boundary)
    _run(4, 3, 151936, 8, 10, dtype=torch.float32, valid=151001, greedy_frac=0.0)
    _run(6, 3, 100003, 8, 11, greedy_frac=0.0)


def test_verify_residual_falls_back_to_p():
    # A sampled request at a temperature that makes p the point mass at the
    # argmax, with q(argmax) = 1 and a drafted token of tiny q: the token is
    # rejected, max(0, p - q) is zero everywhere, and the committed token is
    # drawn from p (the argmax).
    require_gpu()
    R, S, V, K = 3, 2, 5000, 4
    d = _inputs(R, S, V, K, 12, greedy_frac=0.0)
    zf = d["z"].float()
    d["temps"][:] = 1e-7
    for r in range(R):
        top = int(torch.argmax(zf[r, 0]))
        others = [v for v in range(V) if v != top][:K - 1]
        d["cand"][r, 0] = torch.tensor([top] + others)
        d["q"][r, 0] = torch.tensor([1.0] + [1e-3] * (K - 1))
        d["tok"][r, 0] = others[0]
    say(f"dflash_verify residual fallback R={R} S={S} V={V}")
    acc, com = D.dflash_verify(d["z"].to(DEV), d["cand"].to(DEV), d["q"].to(DEV), d["tok"].to(DEV),
                               d["ua"].to(DEV), d["ur"].to(DEV), d["temps"].to(DEV), d["greedy"].to(DEV))
    torch.cuda.synchronize()
    ra, rc = O.verify(f64(d["z"]), V, d["cand"].numpy(), d["q"].double().numpy(), d["tok"].numpy(),
                      d["ua"].double().numpy(), d["ur"].double().numpy(), d["temps"].double().numpy(),
                      d["greedy"].numpy())
    assert np.all(ra == 0)
    assert np.array_equal(acc.cpu().numpy(), ra) and np.array_equal(com.cpu().numpy(), rc)
    for r in range(R):
        assert rc[r, 0] == int(torch.argmax(zf[r, 0]))


def test_verify_long_blocks():
    # 70 slots x K = 16: more slots than the commit kernel keeps row
    # statistics for in LDS (64) and more candidates than it preloads (1024
    # threads), so the committed row and the rejected slot's candidates are
    # fetched after the decisions.  Request 0 keeps every token (greedy, all
    # argmax), request 1 keeps 66 tokens and rejects slot 66 (sampled, p a
    # point mass at the argmax, q(argmax) = 1 before it), request 2 is random.
    R, S, V, K = 3, 70, 400, 16
    d = _inputs(R, S, V, K, 15, greedy_frac=0.0)
    zf = d["z"].float()
    d["greedy"][0], d["greedy"][1], d["greedy"][2] = 1, 0, 0
    d["temps"][1] = 1e-7
    for s in range(S):
        top0 = int(torch.argmax(zf[0, s]))
        d["cand"][0, s, 0] = top0 if not bool((d["cand"][0, s, 1:] == top0).any()) else d["cand"][0, s, 0]
        d["tok"][0, s] = top0
        top1 = int(torch.argmax(zf[1, s]))
        others = [v for v in range(V) if v != top1][:K - 1]
        d["cand"][1, s] = torch.tensor([top1] + others)
        d["q"][1, s] = torch.tensor([1.0] + [1e-3] * (K - 1))
        d["tok"][1, s] = top1 if s < 66 else others[0]
    if not bool((d["cand"][0] == d["tok"][0].unsqueeze(-1)).any(-1).all()):
        d["cand"][0, :, 0] = d["tok"][0]
    a, _ = _run(R, S, V, K, 15, d=d)
    assert a[0] == S and a[1] == 66


def _near_ties(d, S, seed):
    """Sets u_accept so that each request's slot r % S sits 3e-7 (relative)
    from its accept edge (alternately just rejected and just kept; earlier
    slots kept outright), then u_residual so that the committed draw's target
    sits 2e-7 of the total from an interval boundary in the middle of the
    drawn distribution (alternately just inside and just before it)."""
    z = f64(d["z"])
    R = z.shape[0]
    temps = d["temps"].double().numpy()
    cand, tok, valid = d["cand"].numpy(), d["tok"].numpy(), d["valid"]
    for r in range(R):
        n = r % S
        d["ua"][r, :n] = 0.0                      # u q(x) = 0 < p(x): kept
        x = int(tok[r, n])
        p = O.target_distribution(z[r, n], valid, temps[r], False)
        qx = float(d["q"][r, n, np.flatnonzero(cand[r, n] == x)[0]])
        u = p[x] / qx * (1 + (3e-7 if r % 2 == 0 else -3e-7))
        if u >= 1.0:
            u = p[x] / qx * (1 - 3e-7)
        d["ua"][r, n] = float(np.float32(u))
    ra, _ = O.verify(z, valid, cand, d["q"].double().numpy(), tok, d["ua"].double().numpy(),
                     d["ur"].double().numpy(), temps, d["greedy"].numpy())
    for r in range(R):
        n = int(ra[r])
        p = O.target_distribution(z[r, n], valid, temps[r], False)
        w = p
        if n < S:
            w = p.copy()
            for jj, v in enumerate(cand[r, n]):
                w[v] = max(0.0, w[v] - float(d["q"][r, n, jj]))
            if not np.any(w > 0):
                w = p
        c = np.cumsum(w)
        k = int(np.searchsorted(c, 0.5 * c[-1]))
        lo = c[k - 1] if k > 0 else 0.0
        side = 1.0 if (r // 2) % 2 == 0 else -1.0
        d["ur"][r] = float(np.float32((lo + side * 2e-7 * c[-1]) / c[-1]))
    return d


@pytest.mark.parametrize("dtype,V,valid,seed", [(torch.bfloat16, 151936, 151936, 16),
                                                (torch.float32, 5003, 4999, 17)])
def test_verify_near_ties_take_the_exact_path(dtype, V, valid, seed):
    # Decisions and draws a few 1e-7 (relative) from their edges: inside the
    # error bound of the fp32 sums, so the kernels take each near-tie
    # decision from its row's exact fp64 sums inside the commit pass (a draw
    # after a rejection there comes from those sums too), and leave a draw
    # from a later row to the exact-sum and fix-up passes (half the requests
    # here); far outside the comparison's 1e-9 edge allowance, so the outcome
    # must equal the oracle's.
    R, S, K = 12, 3, 8
    d = _near_ties(_inputs(R, S, V, K, seed, dtype=dtype, valid=valid, greedy_frac=0.0), S, seed)
    acc, com = _run(R, S, V, K, seed, d=d)
    ra, rc = O.verify(f64(d["z"]), valid, d["cand"].numpy(), d["q"].double().numpy(), d["tok"].numpy(),
                      d["ua"].double().numpy(), d["ur"].double().numpy(), d["temps"].double().numpy(),
                      d["greedy"].numpy())
    assert np.array_equal(acc, ra) and np.array_equal(com, rc)
    assert 0 < int((ra < np.arange(R) % S + 1).sum()) < R   # both sides of the accept edge occur
