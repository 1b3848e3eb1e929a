"""GPU tests of dflash_propose_block, the whole draft block ("[Spec]
DFlash2", draft-sampler excerpt): it must equal the chain of the four entry
points bit for bit, repeat bit for bit, and agree end to end with the oracle
run from the raw inputs (ids exact; every walk decision whose margin clears
the rounding band of the fp32 lattice must match; decisions inside the band
are counted and the oracle continues from the GPU's choice).

End-to-end bars (oracle from the raw inputs, float64):
  * scores: the lattice bar 1e-4 (1 + |unary| + sum_k |A u B|) plus the exact
    effect of conv outputs the two sides rounded to different storage values
    and the unary tolerance;
  * a sampled decision may differ only where the uniform lies within the CDF
    shift that band allows (softmax_shift of the row's band / T), a greedy one
    only where the two maxima lie within their bands;
  * q of a sampled row within 1e-5 of the oracle's softmax, widened only by
    the effect of those legitimately different inputs (conv outputs rounded
    differently, the fp32 transform)."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import CONV_TOL, DEV, conv_rel_err, f64, require_gpu, sample_indices, say
from oracle import dflash_oracle as O
from parity_bars import input_shift_bound, lattice_bar, softmax_shift

pytestmark = pytest.mark.gpu


def _cfg(w: W.Workload):
    return D.make_config(taps=w.taps, group_size=w.group_size, rank=w.rank, top_k=w.top_k,
                         multiplier=w.multiplier, softcap=w.softcap, block_size=w.block_size, hidden=w.hidden)


def _propose(w, inp, keep_scores=True, **kw):
    return D.dflash_propose_block(_cfg(w), x=inp["x"], conv_base=inp["base"][0], conv_delta=inp["delta"][:, 0],
                                  logits=inp["logits"], anchor=inp["anchor"], sel_a=inp["sel_a"],
                                  sel_b=inp["sel_b"], proj=inp["proj"], uniforms=inp["uniforms"],
                                  temperatures=inp["temperatures"], greedy_mask=inp["greedy_mask"],
                                  valid_vocab=w.valid_vocab, keep_scores=keep_scores, **kw)


def _chain(w, inp):
    conv = D.dflash_conv(inp["x"], inp["base"][0], inp["delta"][:, 0], block_size=w.block_size,
                         group_size=w.group_size)
    ids, unary = D.dflash_topk(inp["logits"], top_k=w.top_k, valid_vocab=w.valid_vocab, multiplier=w.multiplier,
                               softcap=w.softcap)
    R, S, K = w.n_req, w.slots, w.top_k
    ids, unary = ids.view(R, S, K), unary.view(R, S, K)
    hid = conv.view(R, w.block_size, w.hidden)[:, 1:, :]
    scores = D.dflash_lattice(ids, unary, hid, inp["anchor"], inp["sel_a"], inp["sel_b"], inp["proj"])
    tok, q = D.dflash_walk(scores, ids, inp["uniforms"], inp["temperatures"], inp["greedy_mask"])
    return dict(conv_out=conv, ids=ids, unary=unary, scores=scores, tokens=tok, q=q)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_fused_equals_chain_and_repeats(name):
    require_gpu()
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device=DEV)
    say(f"dflash_propose_block {name} (fused vs chain)")
    a = _propose(w, inp)
    b = _propose(w, inp)
    c = _chain(w, inp)
    torch.cuda.synchronize()
    for k in ("conv_out", "ids", "unary", "scores", "tokens", "q"):
        assert torch.equal(a[k], b[k]), ("repeat", k)
        assert torch.equal(a[k], c[k]), ("chain", k)
    # the scores-in-workspace variant gives the same tokens and q
    d = _propose(w, inp, keep_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(a["tokens"], d["tokens"]) and torch.equal(a["q"], d["q"])


@pytest.mark.parametrize("B,T,n_req", [(2, 1, 37), (3, 2, 21), (7, 3, 19), (10, 5, 13), (13, 8, 11), (16, 8, 9)])
def test_one_launch_for_every_block_size(B, T, n_req):
    # Blocks of 2 to 16 tokens share the top-K's launch (the block's tokens
    # are the first rows of a 16-row matrix tile, the rest zeros): equal to
    # the chain bit for bit and to the oracle, with a ragged last workgroup.
    require_gpu()
    w = W.WORKLOADS["nonpow2_b10_v151936"].replace(n_req=n_req, block_size=B, taps=T, vocab=4096,
                                                  valid_vocab=4096, hidden=1024)
    assert D.propose_block_schedule(_cfg(w), w.n_req, w.dtype) == D.SCHEDULE_ONE_LAUNCH
    inp = W.make_inputs(w, device=DEV)
    say(f"dflash_propose_block one launch B={B} T={T} n_req={n_req}")
    a = _propose(w, inp)
    c = _chain(w, inp)
    torch.cuda.synchronize()
    for k in ("conv_out", "ids", "unary", "scores", "tokens", "q"):
        assert torch.equal(a[k], c[k]), (B, k)
    ref = O.conv(f64(inp["x"]), f64(inp["base"][0]), f64(inp["delta"][:, 0]), B, w.group_size)
    assert conv_rel_err(f64(a["conv_out"]), ref) <= CONV_TOL["bf16"]


@pytest.mark.parametrize("modes", ["sampled:2.0", "alt:1.5", "greedy"])
def test_fused_walk_follows_nonzero_choices(modes):
    """Lattices that fit the fused kernel, with walks that leave row 0: q of
    slot s must be the row of the index chosen at slot s - 1, tokens the
    candidate chosen at slot s -- equal to the chain of entry points."""
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"].replace(n_req=8, plant_peak=False, modes=modes, vocab=8192,
                                               valid_vocab=8192)
    inp = W.make_inputs(w, device=DEV)
    say(f"dflash_propose_block fused walk, {modes}")
    a = _propose(w, inp)
    c = _chain(w, inp)
    torch.cuda.synchronize()
    for k in ("scores", "tokens", "q"):
        assert torch.equal(a[k], c[k]), k
    # the walk must have left row 0 somewhere, or this test covers nothing
    chosen = (a["ids"] == a["tokens"].unsqueeze(-1)).float().argmax(-1)
    assert int((chosen[:, :-1] != 0).sum()) > 0


def _e2e(w: W.Workload, req_sample):
    inp = W.make_inputs(w, device=DEV)
    say(f"dflash_propose_block {w.name} (end to end vs oracle)")
    out = _propose(w, inp)
    torch.cuda.synchronize()
    R, B, S, K, H = w.n_req, w.block_size, w.slots, w.top_k, w.hidden
    reqs = np.arange(R) if req_sample is None else sample_indices(R, req_sample, seed=2)
    tok_rows = np.concatenate([np.arange(r * B, (r + 1) * B) for r in reqs])
    slot_rows = np.concatenate([np.arange(r * S, (r + 1) * S) for r in reqs])
    ti = torch.from_numpy(tok_rows).to(DEV)
    si = torch.from_numpy(slot_rows).to(DEV)
    ri = torch.from_numpy(reqs).to(DEV)
    host = dict(x=f64(inp["x"][ti]), base=f64(inp["base"]), delta=f64(inp["delta"][ti]),
                logits=f64(inp["logits"][si]), anchor=inp["anchor"][ri].cpu().numpy(),
                sel_a=f64(inp["sel_a"]), sel_b=f64(inp["sel_b"]), proj=f64(inp["proj"]),
                uniforms=inp["uniforms"][ri].cpu().numpy(), temperatures=inp["temperatures"][ri].cpu().numpy(),
                greedy_mask=inp["greedy_mask"][ri].cpu().numpy())
    ref = O.propose_block(host, block_size=B, group_size=w.group_size, valid_vocab=w.valid_vocab, top_k=K,
                          multiplier=w.multiplier, softcap=w.softcap, dtype=w.dtype)
    # conv
    assert conv_rel_err(f64(out["conv_out"][ti]), ref["conv_out"]) <= CONV_TOL[w.dtype]
    # ids exact, unary close
    np.testing.assert_array_equal(out["ids"][ri].cpu().numpy(), ref["ids"])
    assert np.all(np.abs(f64(out["unary"][ri]) - ref["unary"]) <= 1e-5 * (1 + np.abs(ref["unary"])))
    # scores: the oracle's (from its own rounded conv output) vs the GPU's
    got_scores = f64(out["scores"][ri])
    anc, A, Bt, P = host["anchor"], host["sel_a"], host["sel_b"], host["proj"]
    h_gpu = f64(out["conv_out"][ti]).reshape(len(reqs), B, H)[:, 1:, :]
    dh = h_gpu - ref["h"]
    # legitimately different inputs: conv outputs rounded to the other
    # neighbour, and the fp32 transform's unary against the exact one
    du = np.abs(f64(out["unary"][ri]) - ref["unary"])
    du = np.where(np.isfinite(du), du, 0.0)
    shift = input_shift_bound(ref["ids"], dh, P, anc, A, Bt) + du[:, :, None, :]
    band = lattice_bar(ref["ids"], ref["unary"], ref["u"], anc, A, Bt) + shift
    err = np.abs(got_scores - ref["scores"])
    print(f"[e2e] {w.name}: {len(reqs)} requests; conv outputs rounded differently: {int(np.count_nonzero(dh))} "
          f"of {dh.size}; max score err / band {float(np.max(err / band)):.3e}", flush=True)
    assert np.all(err <= band), float(np.max(err / band))
    # walk decisions
    got_tok = out["tokens"][ri].cpu().numpy()
    got_q = out["q"][ri].cpu().numpy()
    greedy = host["greedy_mask"]
    near, q_err = 0, 0.0
    for i, r in enumerate(reqs):
        prev = 0
        ids_r = out["ids"][r].cpu().numpy()
        for s in range(S):
            row_ref = ref["scores"][i, s, prev]
            row_band = band[i, s, prev]
            idx = int(np.flatnonzero(ids_r[s] == got_tok[i, s])[0])
            if greedy[i]:
                best = int(np.argmax(row_ref))
                if idx != best:
                    # allowed only if the two are within their bands
                    assert row_ref[best] - row_ref[idx] <= row_band[best] + row_band[idx], (r, s)
                    near += 1
                assert got_q[i, s, idx] == 1.0 and np.count_nonzero(got_q[i, s]) == 1
            else:
                t = max(float(host["temperatures"][i]), 1e-5)
                x = row_ref / t
                p = np.exp(x - x.max()); p /= p.sum()
                cdf = np.cumsum(p)
                u = float(host["uniforms"][i, s])
                want = min(int(np.count_nonzero(u >= cdf)), K - 1)
                if idx != want:
                    # the CDF values move by at most softmax_shift(max band / T)
                    slack = float(softmax_shift(np.max(row_band) / t))
                    assert abs(u - cdf[min(idx, want)]) <= slack, (r, s, u, cdf[min(idx, want)], slack)
                    near += 1
                e = float(np.max(np.abs(got_q[i, s] - p)))
                q_err = max(q_err, e)
                q_tol = 1e-5 + float(softmax_shift(np.max(shift[i, s, prev]) / t))
                assert e <= q_tol, (r, s, e, q_tol)
            prev = idx
    print(f"[e2e] {w.name}: max sampled |q - q_ref| {q_err:.3e}", flush=True)
    return near


@pytest.mark.parametrize("name,reqs", [("tiny_fp32", None), ("bf16_b16_v151936", None),
                                       ("nonpow2_b10_v151936", None), ("padded_v201024_k16", 32),
                                       ("stress_r1024_k32", 32)])
def test_end_to_end_against_oracle(name, reqs):
    require_gpu()
    near = _e2e(W.WORKLOADS[name], reqs)
    print(f"[e2e] {name}: decisions inside the rounding band: {near}", flush=True)


@pytest.mark.parametrize("name,n_req,schedule", [
    ("bf16_b16_v151936", None, D.SCHEDULE_ONE_LAUNCH),
    ("nonpow2_b10_v151936", None, D.SCHEDULE_ONE_LAUNCH),       # blocks of 10 in the one launch
    ("bf16_b16_v151936", 288, D.SCHEDULE_AUX_STREAM),        # 4320 slot rows: the tiled projection
    ("nonpow2_b10_v151936", 240, D.SCHEDULE_AUX_STREAM),     # blocks of 10, 2160 slot rows
])
def test_stream_ordering_on_either_schedule(name, n_req, schedule):
    """Whichever schedule the call takes (asserted first), its kernels must
    see inputs written on the caller's stream just before the call, and work
    the caller enqueues on that stream after it must see every output: on the
    fork/join schedule the conv and the projection run on the library's
    auxiliary stream.  Outputs start poisoned (NaN, -1) so that a read before
    the write that should precede it shows."""
    require_gpu()
    w = W.WORKLOADS[name]
    if n_req is not None:
        w = w.replace(n_req=n_req)
    assert D.propose_block_schedule(_cfg(w), w.n_req, w.dtype) == schedule
    inp = W.make_inputs(w, device=DEV)
    say(f"stream ordering {name} n_req={w.n_req} schedule={schedule}: chain reference")
    ref = _chain(w, inp)
    x_late = torch.zeros_like(inp["x"])
    outs = {k: torch.full_like(v, -1 if v.dtype == torch.int64 else float("nan")) for k, v in ref.items()}
    busy = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say(f"stream ordering {name}: dflash_propose_block on a side stream after a late input write")
    with torch.cuda.stream(side):
        for _ in range(4):
            busy.fill_(1)                 # keeps the side stream busy before the write
        x_late.copy_(inp["x"])
        out = _propose(w, dict(inp, x=x_late), outputs=outs)
        got = {k: out[k].clone() for k in ref}
    torch.cuda.synchronize()
    for k, v in got.items():
        assert torch.equal(v, ref[k]), k


def test_stage_events_are_recorded():
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"]
    inp = W.make_inputs(w, device=DEV)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    say("dflash_propose_block with stage events")
    out = _propose(w, inp, stage_events=ev)
    torch.cuda.synchronize()
    times = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(4)]
    assert all(t >= 0 for t in times)
    assert times[1] > 0
    assert out["tokens"].shape == (w.n_req, w.slots)
    # NULL entries are skipped: only the top-K pair, through a prepared call
    call = D.ProposeBlock(_cfg(w), x=inp["x"], conv_base=inp["base"][0], conv_delta=inp["delta"][:, 0],
                          logits=inp["logits"], anchor=inp["anchor"], sel_a=inp["sel_a"], sel_b=inp["sel_b"],
                          proj=inp["proj"], uniforms=inp["uniforms"], temperatures=inp["temperatures"],
                          greedy_mask=inp["greedy_mask"], valid_vocab=w.valid_vocab)
    pair = [None, None, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] + [None] * 4
    for e in pair[2:4]:
        e.record()
    torch.cuda.synchronize()
    got = call(stage_events=D.ProposeBlock.event_array(pair))
    got = call(stage_events=D.ProposeBlock.event_array(pair))
    torch.cuda.synchronize()
    assert pair[2].elapsed_time(pair[3]) > 0
    assert torch.equal(got["tokens"], out["tokens"]) and torch.equal(got["q"], out["q"])


def test_zero_requests_is_a_no_op():
    require_gpu()
    w = W.WORKLOADS["tiny_fp32"].replace(n_req=0)
    inp = W.make_inputs(w, device=DEV)
    out = _propose(w, inp)
    torch.cuda.synchronize()
    assert out["tokens"].shape == (0, w.slots)
