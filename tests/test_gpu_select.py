"""GPU parity of dflash_lattice and dflash_walk against the oracle
("[Spec] DFlash2": executive summary edge formula and lossless-q contract;
walk-kernel excerpt).

Lattice bar (stepwise: the oracle gets the GPU's own ids, unary and hidden
rows, and projects them exactly): every score within
    1e-4 (1 + |unary_c| + sum_k |A_pk u_k B_ck|)
of the exact value -- a bar an fp32 evaluation clears with a wide margin and
a projection rounded to bf16 breaks (pinned on the CPU in
tests/test_parity_bars.py).  The rigorous fp32 worst case is printed beside it.
Walk bar: the oracle walks the GPU's own scores in the pages' fp32 order, so
tokens and q must match bit for bit."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import DEV, f64, require_gpu, sample_indices, say
from oracle import dflash_oracle as O
from parity_bars import fp32_sum_bound, lattice_bar

pytestmark = pytest.mark.gpu
REQ_CHUNK = 64      # requests compared per host pass (bounds host memory)


def _lattice_inputs(w: W.Workload, seed=None):
    inp = W.make_inputs(w, device=DEV, parts=("logits", "selector", "sampling"), seed=seed)
    hid = W.normal((w.n_req, w.slots, w.hidden), 1.0, w.dtype, W.master_seed(w), "hidden", DEV)
    return inp, hid


def _check_lattice(w, inp, hid, req_sample=None):
    say(f"dflash_topk+dflash_lattice {w.name} R={w.n_req} S={w.slots} K={w.top_k} r={w.rank} H={w.hidden}")
    ids, unary = D.dflash_topk(inp["logits"], top_k=w.top_k, valid_vocab=w.valid_vocab, multiplier=w.multiplier,
                               softcap=w.softcap)
    ids = ids.view(w.n_req, w.slots, w.top_k)
    unary = unary.view(w.n_req, w.slots, w.top_k)
    scores = D.dflash_lattice(ids, unary, hid, inp["anchor"], inp["sel_a"], inp["sel_b"], inp["proj"])
    torch.cuda.synchronize()
    reqs = np.arange(w.n_req) if req_sample is None else sample_indices(w.n_req, req_sample, seed=1)
    A, B, P = f64(inp["sel_a"]), f64(inp["sel_b"]), f64(inp["proj"])
    worst, loose_worst = 0.0, 0.0
    for c0 in range(0, len(reqs), REQ_CHUNK):
        ri = torch.from_numpy(reqs[c0:c0 + REQ_CHUNK]).to(DEV)
        ids_h = ids[ri].cpu().numpy()
        un_h = f64(unary[ri])
        h_h = f64(hid[ri])
        anc = inp["anchor"][ri].cpu().numpy()
        u = O.project(h_h, P)
        ref = O.lattice(ids_h, un_h, u, anc, A, B)
        err = np.abs(f64(scores[ri]) - ref)
        ratio = err / lattice_bar(ids_h, un_h, u, anc, A, B)
        worst = max(worst, float(np.max(ratio)))
        assert np.all(ratio <= 1.0), (w.name, int(reqs[c0]), float(np.max(ratio)))
        if c0 == 0:   # the fp32 worst-case bound, printed for comparison only
            loose_worst = float(np.max(err / fp32_sum_bound(ids_h, un_h, h_h, P, anc, A, B)))
    print(f"[lattice] {w.name}: {len(reqs)} of {w.n_req} requests, max err / bar {worst:.3e} "
          f"(err / fp32 worst case {loose_worst:.3e} on the first {min(REQ_CHUNK, len(reqs))})", flush=True)
    # slot 0: every predecessor row is the anchor's, so the rows are identical
    assert torch.equal(scores[:, 0, :1, :].expand_as(scores[:, 0]), scores[:, 0])
    return ids, unary, scores


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_lattice_matches_oracle(name):
    # every request of every workload, at full size
    require_gpu()
    w = W.WORKLOADS[name]
    inp, hid = _lattice_inputs(w)
    _check_lattice(w, inp, hid)


@pytest.mark.parametrize("dtype,H,r,K", [("bf16", 40, 8, 4), ("bf16", 200, 24, 5), ("bf16", 1032, 128, 32),
                                         ("f32", 36, 3, 7), ("bf16", 4096, 16, 1)])
def test_lattice_edge_shapes(dtype, H, r, K):
    # Rank not a multiple of 16, hidden not a multiple of 32, K = 1 and 32,
    # a ragged number of slot rows (R*S = 3*6 = 18, not a multiple of 64).
    require_gpu()
    w = W.Workload(name=f"lat_{dtype}_{H}_{r}_{K}", n_req=3, block_size=7, hidden=H, group_size=H // 4 if H % 4 == 0 else H,
                   taps=2, vocab=3000, valid_vocab=3000, top_k=K, rank=r, dtype=dtype, multiplier=1.0, softcap=30.0)
    inp, hid = _lattice_inputs(w)
    _check_lattice(w, inp, hid)


def test_lattice_strided_hidden_view():
    # hidden given as the slot rows of a [R, B, H] block buffer (position 0
    # dropped), the layout the fused path hands over.
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"].replace(n_req=6, vocab=20000, valid_vocab=20000)
    inp = W.make_inputs(w, device=DEV, parts=("logits", "selector", "sampling"))
    block = W.normal((w.n_req, w.block_size, w.hidden), 1.0, "bf16", 99, "block", DEV)
    _check_lattice(w, inp, block[:, 1:, :])


def test_lattice_out_of_range_id_gives_nan_not_a_fault():
    require_gpu()
    w = W.WORKLOADS["tiny_fp32"]
    inp, hid = _lattice_inputs(w)
    ids = torch.randint(0, w.vocab, (w.n_req, w.slots, w.top_k), device=DEV)
    ids[0, 1, 2] = w.vocab + 5                 # candidate beyond the table
    unary = torch.zeros((w.n_req, w.slots, w.top_k), device=DEV)
    s = D.dflash_lattice(ids, unary, hid, inp["anchor"], inp["sel_a"], inp["sel_b"], inp["proj"])
    torch.cuda.synchronize()
    assert torch.isnan(s[0, 1, :, 2]).all()     # as candidate of slot 1
    assert torch.isnan(s[0, 2, 2, :]).all()     # as predecessor in slot 2
    assert torch.isfinite(s[1]).all()


def _walk_check(scores, ids, uni, temps, greedy, label):
    say(f"dflash_walk {label} R={ids.shape[0]} S={ids.shape[1]} K={ids.shape[2]}")
    tok, q = D.dflash_walk(scores, ids, uni, temps, greedy)
    torch.cuda.synchronize()
    rt, rq, _ = O.walk(scores.cpu().numpy(), ids.cpu().numpy(), uni.cpu().numpy(), temps.cpu().numpy(),
                       greedy.cpu().numpy())
    np.testing.assert_array_equal(tok.cpu().numpy(), rt)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    return tok, q


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_walk_on_gpu_scores_matches_oracle_bitwise(name):
    require_gpu()
    w = W.WORKLOADS[name]
    inp, hid = _lattice_inputs(w)
    ids, unary, scores = _check_lattice(w, inp, hid, req_sample=4)
    tok, q = _walk_check(scores, ids, inp["uniforms"], inp["temperatures"], inp["greedy_mask"], name)
    g = inp["greedy_mask"]
    if g.any():   # greedy rows: point masses
        qg = q[g]
        assert torch.equal(qg.max(-1).values, torch.ones_like(qg.max(-1).values))
        assert torch.equal(qg.sum(-1), torch.ones_like(qg.sum(-1)))
    if (~g).any():
        qs = q[~g].double()
        assert torch.allclose(qs.sum(-1), torch.ones_like(qs.sum(-1)), atol=1e-5)


@pytest.mark.parametrize("K", [1, 2, 3, 8, 17, 32])
def test_walk_synthetic_lattices(K):
    # Random lattices with mixed modes, coarse scores (greedy ties), tiny
    # temperatures (clamped to 1e-5), uniforms at exact CDF values.
    require_gpu()
    g = torch.Generator(device=DEV).manual_seed(K)
    R, S = 67, 9
    scores = (torch.randn((R, S, K, K), generator=g, device=DEV) * 3).round() / 2
    scores[5] = 0.0                                            # all tied
    ids = torch.randint(0, 1 << 20, (R, S, K), generator=g, device=DEV)
    uni = torch.rand((R, S), generator=g, device=DEV)
    uni[5] = torch.tensor([j / max(K, 1) for j in range(S)], device=DEV).clamp(max=0.999)
    temps = torch.rand((R,), generator=g, device=DEV) * 2
    temps[3] = 0.0
    temps[4] = 1e-9
    greedy = torch.rand((R,), generator=g, device=DEV) < 0.4
    greedy[5] = False
    _walk_check(scores.contiguous(), ids, uni, temps, greedy, f"synthetic K={K}")


def test_walk_greedy_rows_are_deterministic_in_a_mixed_batch():
    # The PR's own test name: greedy rows must not depend on the other rows'
    # modes, the uniforms or the temperatures.
    require_gpu()
    g = torch.Generator(device=DEV).manual_seed(0)
    R, S, K = 40, 15, 16
    scores = torch.randn((R, S, K, K), generator=g, device=DEV) * 4
    ids = torch.randint(0, 200000, (R, S, K), generator=g, device=DEV)
    greedy = torch.arange(R, device=DEV) % 3 == 0
    t0, q0 = D.dflash_walk(scores, ids, torch.rand((R, S), generator=g, device=DEV),
                           torch.rand((R,), generator=g, device=DEV) + 0.1, greedy)
    greedy2 = greedy | (torch.arange(R, device=DEV) % 3 == 1)
    t1, q1 = D.dflash_walk(scores, ids, torch.rand((R, S), generator=g, device=DEV),
                           torch.rand((R,), generator=g, device=DEV) * 5, greedy2)
    torch.cuda.synchronize()
    assert torch.equal(t0[greedy], t1[greedy]) and torch.equal(q0[greedy], q1[greedy])
    for r in torch.nonzero(greedy).flatten()[:4].tolist():
        t2, q2 = D.dflash_walk(scores[r:r + 1].contiguous(), ids[r:r + 1].contiguous(),
                               torch.zeros((1, S), device=DEV), torch.ones(1, device=DEV),
                               torch.ones(1, dtype=torch.bool, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(t2[0], t0[r]) and torch.equal(q2[0], q0[r])


@pytest.mark.parametrize("S", [20, 45])
def test_walk_large_lattice_beyond_lds_staging(S):
    # K = 32: S = 20 stages 80 KB of scores in the 1024-thread walk (beyond
    # the 64 KB of earlier parts, within gfx950's 160 KB per workgroup);
    # S = 45 (180 KB) is beyond it, and the serial walk reads rows from memory.
    require_gpu()
    g = torch.Generator(device=DEV).manual_seed(9 + S)
    R, K = 5, 32
    scores = torch.randn((R, S, K, K), generator=g, device=DEV) * 2
    ids = torch.randint(0, 1000, (R, S, K), generator=g, device=DEV)
    uni = torch.rand((R, S), generator=g, device=DEV)
    temps = torch.full((R,), 0.9, device=DEV)
    greedy = torch.tensor([True, False, False, True, False], device=DEV)
    _walk_check(scores, ids, uni, temps, greedy, f"S={S}")
