"""GPU parity of the dense head of compute_candidates ("[Spec] DFlash2",
implementation breakdown and risk notes): dflash_lm_head against the
oracle's exact sums rounded once to bf16.

Rule: a GPU logit equals the oracle's rounding of the exact sum, except
where the exact sum lies within the fp32 accumulation bound
(O.lm_head_sum_bound) of a bf16 rounding midpoint; there either neighbour is
correct, and both candidates are checked.  Such cases are counted.  The top-K
of the GPU logits (dflash_topk) equals the oracle's top-K of those logits
bit for bit."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import DEV, f64, require_gpu, sample_indices, say
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu


def _check_logits(got: np.ndarray, h: np.ndarray, w: np.ndarray) -> int:
    """got [rows, cols] (float64 copies of bf16) vs the exact sums of h @ w.T."""
    exact = h @ w.T
    ref = O.round_to_bf16(exact)
    bound = O.lm_head_sum_bound(h, w)
    lo, hi = O.round_to_bf16(exact - bound), O.round_to_bf16(exact + bound)
    off = got != ref
    assert np.all(~off | ((got >= lo) & (got <= hi))), float(np.max(np.abs(got - ref)))
    return int(off.sum())


def _head(w: W.Workload, rows=None, seed=None):
    d = W.make_head_inputs(w, device=DEV, seed=seed, n_rows=rows)
    return d["hidden"], d["weight"]


@pytest.mark.parametrize("M,H,V", [(70, 96, 1000), (130, 200, 392), (1, 8, 8), (257, 64, 136), (128, 4096, 1024)])
def test_lm_head_small_shapes_match_the_exact_sums(M, H, V):
    # ragged row blocks (70, 130, 257 rows), a hidden size that is not a
    # multiple of the 64-wide stage (96, 200), a vocabulary that ends inside a
    # 128-column tile (1000, 392, 136) and the smallest case
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"].replace(hidden=H, vocab=V, valid_vocab=V, n_req=1)
    hid, wt = _head(w, rows=M, seed=M * 7919 + H)
    say(f"dflash_lm_head M={M} H={H} V={V}")
    out = D.dflash_lm_head(hid, wt)
    torch.cuda.synchronize()
    near = _check_logits(f64(out), f64(hid), f64(wt))
    print(f"[lm_head] {M}x{H}x{V}: {near} logits on the rounding band", flush=True)


def test_lm_head_strided_rows_and_output_stride():
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"].replace(hidden=256, vocab=520, valid_vocab=520, n_req=1)
    hid, wt = _head(w, rows=40, seed=5)
    wide = torch.zeros((40, 256 + 64), dtype=hid.dtype, device=DEV)
    wide[:, 16:16 + 256] = hid
    view = wide[:, 16:16 + 256]                          # row stride 320, 32-byte offset
    out_wide = torch.full((40, 600), 7.0, dtype=hid.dtype, device=DEV)
    say("dflash_lm_head strided")
    D.dflash_lm_head(view, wt, out=out_wide[:, :520])
    torch.cuda.synchronize()
    _check_logits(f64(out_wide[:, :520]), f64(hid), f64(wt))
    assert torch.all(out_wide[:, 520:] == 7.0)            # nothing written past the vocab


def test_lm_head_full_bench_shape_sampled_rows_then_topk():
    # 480 slot rows x 4096 x 151936: sampled rows checked over every column,
    # and the chain head -> dflash_topk equal to the oracle's top-K of the
    # GPU logits
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"]
    hid, wt = _head(w)
    say("dflash_lm_head 480x4096x151936")
    out = D.dflash_lm_head(hid, wt)
    ids, unary = D.dflash_topk(out, top_k=w.top_k, valid_vocab=w.valid_vocab, multiplier=w.multiplier,
                               softcap=w.softcap)
    torch.cuda.synchronize()
    rows = sample_indices(w.n_slot_rows, 6, seed=11)
    wt64 = f64(wt)
    got = f64(out[torch.from_numpy(rows).to(DEV)])
    near = _check_logits(got, f64(hid)[rows], wt64)
    print(f"[lm_head] bench shape, {len(rows)} rows: {near} logits on the rounding band", flush=True)
    ref_ids, ref_unary = O.topk(got, w.valid_vocab, w.top_k, w.multiplier, w.softcap)
    np.testing.assert_array_equal(ids.cpu().numpy()[rows], ref_ids)
    assert np.all(np.abs(f64(unary)[rows] - ref_unary) <= 1e-5 * (1 + np.abs(ref_unary)))


def test_lm_head_rejects_fp32_and_empty_is_a_no_op():
    require_gpu()
    h = torch.zeros((4, 16), dtype=torch.float32, device=DEV)
    wt = torch.zeros((8, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(D.DFlashError):
        D.dflash_lm_head(h, wt)
    e = D.dflash_lm_head(torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV),
                         torch.zeros((8, 16), dtype=torch.bfloat16, device=DEV))
    assert e.shape == (0, 8)


@pytest.mark.parametrize("M,H,V,valid,K,m,cap", [
    (70, 96, 1000, 1000, 8, 1.0, 30.0),       # ragged rows, hidden and vocabulary
    (130, 64, 2056, 2000, 16, 0.5, 30.0),     # logical vocab inside the last tile
    (257, 200, 392, 392, 1, 1.0, 0.0),        # K = 1
    (40, 128, 4096, 4093, 32, 1.0, 30.0),     # K = 32, valid not a multiple of 8
    (5, 64, 136, 40, 40 // 2, 1.0, 0.0),      # few valid ids
])
def test_fused_head_topk_equals_head_then_topk(M, H, V, valid, K, m, cap):
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"].replace(hidden=H, vocab=V, valid_vocab=valid, n_req=1)
    hid, wt = _head(w, rows=M, seed=M * 31 + V)
    say(f"dflash_lm_head_topk M={M} H={H} V={V} valid={valid} K={K}")
    ids, unary = D.dflash_lm_head_topk(hid, wt, top_k=K, valid_vocab=valid, multiplier=m, softcap=cap)
    logits = D.dflash_lm_head(hid, wt)
    ids2, unary2 = D.dflash_topk(logits, top_k=K, valid_vocab=valid, multiplier=m, softcap=cap)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(unary, unary2)
    ref_ids, _ = O.topk(f64(logits), valid, K, m, cap)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)


@pytest.mark.parametrize("M,H,V,valid,K", [
    (4096, 128, 131144, 131000, 32),      # 16 x 513 tiles: groups of 2 tiles, a last group of one
    (4000, 64, 262144, 262144, 8),        # 16 x 1024 tiles: groups of 4, ragged last row block
])
def test_fused_head_topk_multi_tile_groups_equal_chain(M, H, V, valid, K):
    # batches with many tiles walk groups of column tiles per workgroup, the
    # group's list carried in LDS from tile to tile
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"].replace(hidden=H, vocab=V, valid_vocab=valid, n_req=1)
    hid, wt = _head(w, rows=M, seed=M + V)
    say(f"dflash_lm_head_topk groups M={M} H={H} V={V} valid={valid} K={K}")
    ids, unary = D.dflash_lm_head_topk(hid, wt, top_k=K, valid_vocab=valid, multiplier=1.0, softcap=30.0)
    logits = D.dflash_lm_head(hid, wt)
    ids2, unary2 = D.dflash_topk(logits, top_k=K, valid_vocab=valid, multiplier=1.0, softcap=30.0)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(unary, unary2)
    rows = sample_indices(M, 24, seed=5)
    ref_ids, _ = O.topk(f64(logits[torch.from_numpy(rows).to(DEV)]), valid, K, 1.0, 30.0)
    np.testing.assert_array_equal(ids[torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref_ids)


def test_fused_head_topk_ties_go_to_the_lower_id():
    # identical head rows give equal logits in every row: the lower id first
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"].replace(hidden=64, vocab=512, valid_vocab=512, n_req=1)
    hid, wt = _head(w, rows=33, seed=77)
    wt = wt.clone()
    wt[300] = hid[0] * 2                  # a clear winner in row 0 ...
    wt[301] = wt[300]                     # ... and its twin with a larger id
    wt[40:48] = wt[7]                     # a block of equal rows
    say("dflash_lm_head_topk ties")
    ids, _ = D.dflash_lm_head_topk(hid, wt, top_k=12)
    torch.cuda.synchronize()
    assert ids[0, 0].item() == 300 and ids[0, 1].item() == 301
    ref, _ = O.topk(f64(D.dflash_lm_head(hid, wt)), 512, 12, 1.0, 0.0)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref)


def test_fused_head_topk_bench_shape_equals_chain():
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"]
    hid, wt = _head(w)
    say("dflash_lm_head_topk 480x4096x151936")
    ids, unary = D.dflash_lm_head_topk(hid, wt, top_k=w.top_k, valid_vocab=w.valid_vocab, multiplier=w.multiplier,
                                       softcap=w.softcap)
    ids2, unary2 = D.dflash_topk(D.dflash_lm_head(hid, wt), top_k=w.top_k, valid_vocab=w.valid_vocab,
                                 multiplier=w.multiplier, softcap=w.softcap)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(unary, unary2)
