"""GPU parity of dflash_topk against the oracle's top-K ("[Spec] DFlash2",
implementation breakdown: deterministic top-k over transformed unary logits;
"DSpark padded-vocab d2t fix": padded ids never selected).  Bar: ids bit-exact
(ties by lowest id); unary within 1e-5 * (1 + |ref|).  Large batches: the
oracle's full sort on a seeded sample of rows, and every row of the batch
through the sort-free validity check of tests/parity_bars.py, which pins the
selected set and its order exactly."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import DEV, f64, require_gpu, sample_indices, say
from oracle import dflash_oracle as O
from parity_bars import topk_violations

ROW_CHUNK = 256     # rows checked per host pass (bounds host memory)

pytestmark = pytest.mark.gpu


def _check(logits, valid, k, m, cap, rows=None, vocab=None, label=""):
    say(f"dflash_topk {label} rows={logits.shape[0]} V={vocab or logits.shape[1]} valid={valid} K={k}")
    ids, unary = D.dflash_topk(logits, top_k=k, valid_vocab=valid, multiplier=m, softcap=cap, vocab=vocab)
    torch.cuda.synchronize()
    sel = np.arange(logits.shape[0]) if rows is None else rows
    idx = torch.from_numpy(sel).to(DEV)
    V = vocab or logits.shape[1]
    ref_ids, ref_unary = O.topk(f64(logits[idx][:, :V]), valid, k, m, cap)
    got_ids, got_unary = ids[idx].cpu().numpy(), f64(unary[idx])
    np.testing.assert_array_equal(got_ids, ref_ids)
    tol = 1e-5 * (1 + np.abs(np.where(np.isfinite(ref_unary), ref_unary, 0)))
    both_ninf = np.isneginf(got_unary) & np.isneginf(ref_unary)
    assert np.all(both_ninf | (np.abs(got_unary - ref_unary) <= tol))
    return ids, unary


def _check_every_row(logits, ids, unary, valid, m, cap, label):
    """Every row through the sort-free validity check; unary of every row
    against the oracle's transform of the selected logits."""
    n = logits.shape[0]
    bad_rows = 0
    for r0 in range(0, n, ROW_CHUNK):
        z = logits[r0:r0 + ROW_CHUNK].float().cpu().numpy()           # bf16 and fp32 are exact in fp32
        got = ids[r0:r0 + ROW_CHUNK].cpu().numpy()
        bad = topk_violations(z, got, valid)
        bad_rows += bad.size
        assert bad.size == 0, (label, int(r0 + bad[0]))
        ref_u = O.transform(np.take_along_axis(z.astype(np.float64), got, axis=1), m, cap)
        got_u = f64(unary[r0:r0 + ROW_CHUNK])
        fin = np.isfinite(ref_u)
        assert np.array_equal(np.isneginf(got_u), ~fin)
        assert np.all(np.abs(got_u[fin] - ref_u[fin]) <= 1e-5 * (1 + np.abs(ref_u[fin])))
    print(f"[topk] {label}: all {n} rows valid", flush=True)


@pytest.mark.parametrize("name,n_rows", [("tiny_fp32", None), ("bf16_b16_v151936", 48),
                                         ("nonpow2_b10_v151936", 48), ("padded_v201024_k16", 48),
                                         ("stress_r1024_k32", 48)])
def test_topk_workloads(name, n_rows):
    # Full-size launches: the oracle's sort on all (tiny) or a seeded sample
    # of rows, then every row through the validity check.
    require_gpu()
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device=DEV, parts=("logits",))
    rows = None if n_rows is None else sample_indices(w.n_slot_rows, n_rows, seed=3)
    ids, unary = _check(inp["logits"], w.valid_vocab, w.top_k, w.multiplier, w.softcap, rows=rows, label=name)
    _check_every_row(inp["logits"], ids, unary, w.valid_vocab, w.multiplier, w.softcap, name)
    if w.plant_peak:
        assert torch.equal(ids[:, 0].cpu(), inp["planted"].cpu())
    if w.valid_vocab < w.vocab:
        assert int(ids.max()) < w.valid_vocab


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,valid,k", [(16384 * 3 + 77, 16384 * 3 + 77, 8), (40000, 39001, 32), (512, 512, 1),
                                       (100, 100, 32), (33, 33, 32), (70000, 16385, 16)])
def test_topk_ragged_vocab_and_tails(dtype, V, valid, k):
    # Several chunks with a ragged last vector (V not a multiple of 8), a
    # logical vocab ending inside a chunk, K at its maximum, K = 1.
    require_gpu()
    rows = 37
    stride = (V + 7) // 8 * 8
    full = W.normal((rows, stride), 3.0, dtype, 11, f"ragged{V}", DEV)
    logits = full[:, :V]
    _check(logits, valid, k, 1.0, 30.0, vocab=V, label=f"ragged {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_mass_ties_take_lowest_ids(dtype):
    # Constant rows, coarse values and -0/+0 mixes force the exact
    # narrowing path (more tied candidates than LDS holds).
    require_gpu()
    td = W.torch_dtype(dtype)
    V, rows = 50000, 8
    g = torch.Generator(device=DEV).manual_seed(5)
    logits = torch.full((rows, V), 2.5, dtype=td, device=DEV)
    logits[1] = torch.round(torch.randn(V, generator=g, device=DEV) * 2).to(td)          # ~9 distinct values
    logits[2] = torch.where(torch.rand(V, generator=g, device=DEV) < 0.5, 0.0, -0.0).to(td)
    logits[3, ::7] = 7.0                                                                  # 7143 ties at the top
    logits[4] = -1.0
    logits[4, 40000:] = float("-inf")
    logits[5] = float("-inf")
    logits[5, 123] = 1.0
    logits[5, 49999] = 1.0                                                                # rest -inf: ties among -inf
    logits[6] = torch.round(torch.randn(V, generator=g, device=DEV) * 0.5).to(td) - 3.0  # all negative
    logits[7, 16384:16384 + 40] = 9.0                                                    # ties straddle a chunk start
    for k in (1, 8, 32):
        _check(logits, V, k, 1.0, 30.0, label=f"ties {dtype} K={k}")
    _check(logits, 30000, 32, 0.5, 30.0, label=f"ties {dtype} valid=30000")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_largest_vocab(dtype):
    # The largest vocabulary the ids' 24-bit field allows (vocab < 2^24): few
    # rows, so each is split into segments and merged; the row maxima and
    # their ties sit at the top of the id range.
    require_gpu()
    V, rows = (1 << 24) - 1, 3
    stride = (V + 7) // 8 * 8                     # 16-byte aligned rows
    logits = W.normal((rows, stride), 3.0, dtype, 17, "maxvocab", DEV)[:, :V]
    logits[0, V - 1] = 40.0                       # the largest id holds the maximum
    logits[1, V - 1] = 40.0
    logits[1, 7] = 40.0                           # a tie with id 7: id 7 first
    logits[2, V - 40:] = 25.0                     # 40 ties in the last ids; K = 32 takes the lowest 32
    for k in (32, 5):
        say(f"dflash_topk max vocab {dtype} V={V} K={k}")
        ids, unary = D.dflash_topk(logits, top_k=k, valid_vocab=V, multiplier=1.0, softcap=30.0, vocab=V)
        torch.cuda.synchronize()
        # the sort-free validity check pins the selected set and its order
        _check_every_row(logits, ids, unary, V, 1.0, 30.0, f"max vocab {dtype} K={k}")
        got = ids.cpu().numpy()
        assert got[0, 0] == V - 1 and got[1, 0] == 7 and got[1, 1] == V - 1
        assert np.array_equal(got[2], np.arange(V - 40, V - 40 + k))


def test_topk_masked_tail_equals_logical_vocab():
    # Padded ids are never returned, whether they are masked by -inf or by
    # the logical vocabulary bound (config with 200058 of 201024).
    require_gpu()
    w = W.WORKLOADS["padded_v201024_k16"].replace(n_req=8)
    inp = W.make_inputs(w, device=DEV, parts=("logits",))
    a, ua = D.dflash_topk(inp["logits"], top_k=16, valid_vocab=200058, multiplier=0.5, softcap=30.0)
    b, ub = D.dflash_topk(inp["logits"], top_k=16, valid_vocab=201024, multiplier=0.5, softcap=30.0)
    high = inp["logits"].clone()
    high[:, 200058:] = 100.0       # padding holding the largest values must still be ignored
    c, uc = D.dflash_topk(high, top_k=16, valid_vocab=200058, multiplier=0.5, softcap=30.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c) and torch.equal(ua, uc)


def test_topk_unary_transform_values():
    # Known transform values: m = 1, cap = 0 is the identity; cap = 30 gives
    # 30 tanh(z / 30); masked entries stay -inf.
    require_gpu()
    z = torch.tensor([[0.0, 1.0, -2.0, 8.0, 30.0, 60.0, -5.0, float("-inf")]], device=DEV)
    logits = torch.full((1, 64), float("-inf"), device=DEV)
    logits[0, :8] = z[0]
    ids, u0 = D.dflash_topk(logits, top_k=8, multiplier=1.0, softcap=0.0)
    _, u1 = D.dflash_topk(logits, top_k=8, multiplier=1.0, softcap=30.0)
    _, u2 = D.dflash_topk(logits, top_k=8, multiplier=0.5, softcap=30.0)
    torch.cuda.synchronize()
    zs = logits[0, ids[0]].double().cpu().numpy()
    np.testing.assert_array_equal(u0[0].double().cpu().numpy(), zs)
    masked = np.isneginf(zs)
    assert masked.sum() == 1
    want1 = np.where(masked, -np.inf, 30 * np.tanh(np.where(masked, 0, zs) / 30))
    want2 = np.where(masked, -np.inf, 30 * np.tanh(0.5 * np.where(masked, 0, zs) / 30))
    np.testing.assert_allclose(u1[0].double().cpu().numpy(), want1, rtol=2e-6, atol=1e-6)
    np.testing.assert_allclose(u2[0].double().cpu().numpy(), want2, rtol=2e-6, atol=1e-6)


def test_topk_repeat_runs_are_bitwise_identical():
    require_gpu()
    w = W.WORKLOADS["nonpow2_b10_v151936"]
    inp = W.make_inputs(w, device=DEV, parts=("logits",))
    say("dflash_topk repeatability")
    a = D.dflash_topk(inp["logits"], top_k=8, multiplier=1.0, softcap=0.0)
    b = D.dflash_topk(inp["logits"], top_k=8, multiplier=1.0, softcap=0.0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
