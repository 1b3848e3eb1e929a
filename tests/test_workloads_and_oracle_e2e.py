"""Host-side checks of the seeded workload generator and an end-to-end run of
the oracle on the tiny workload (CPU only)."""
import numpy as np
import torch

import workloads as W
from oracle import dflash_oracle as O


def _np(t):
    return t.detach().cpu().to(torch.float64).numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def test_generator_is_seeded_and_substreams_are_independent():
    w = W.WORKLOADS["tiny_fp32"]
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    only_logits = W.make_inputs(w, parts=("logits",))
    assert torch.equal(only_logits["logits"], a["logits"])
    c = W.make_inputs(w, seed=123)
    assert not torch.equal(c["x"], a["x"])


def test_workload_shapes_and_structure():
    w = W.WORKLOADS["tiny_fp32"]
    inp = W.make_inputs(w)
    assert inp["x"].shape == (w.n_tokens, w.hidden) and inp["x"].dtype == torch.float32
    assert inp["delta"].shape == (w.n_tokens, 2, w.taps, w.groups)
    assert inp["logits"].shape == (w.n_slot_rows, w.vocab)
    assert inp["greedy_mask"].tolist() == [True, False]
    u = inp["uniforms"]
    assert torch.all((u >= 0) & (u < 1))
    assert torch.equal(u * 2 ** 24, torch.round(u * 2 ** 24))


def test_padded_and_planted_structure_on_small_copies():
    w = W.WORKLOADS["padded_v201024_k16"].replace(n_req=2, vocab=4000, valid_vocab=3900, hidden=64, rank=8)
    inp = W.make_inputs(w, parts=("logits",))
    assert torch.all(torch.isneginf(inp["logits"][:, 3900:]))
    assert torch.all(torch.isfinite(inp["logits"][:, :3900]))
    w2 = W.WORKLOADS["bf16_b16_v151936"].replace(n_req=2, vocab=3000, valid_vocab=3000)
    inp2 = W.make_inputs(w2, parts=("logits",))
    ids, _ = O.topk(_np(inp2["logits"]), 3000, 8, 1.0, 30.0)
    np.testing.assert_array_equal(ids[:, 0], inp2["planted"].numpy())


def test_oracle_end_to_end_on_tiny_workload():
    w = W.WORKLOADS["tiny_fp32"]
    inp = {k: _np(v) for k, v in W.make_inputs(w).items()}
    res = O.propose_block(inp, block_size=w.block_size, group_size=w.group_size,
                          valid_vocab=w.valid_vocab, top_k=w.top_k, multiplier=w.multiplier,
                          softcap=w.softcap, dtype=w.dtype)
    R, S, K = w.n_req, w.slots, w.top_k
    assert res["tokens"].shape == (R, S) and res["q"].shape == (R, S, K)
    # greedy request 0: one-hot q; sampled request 1: a distribution
    assert np.all(res["q"][0].sum(-1) == 1) and np.all(res["q"][0].max(-1) == 1)
    np.testing.assert_allclose(res["q"][1].astype(np.float64).sum(-1), 1, atol=1e-6)
    # each token is one of its slot's candidates
    for r in range(R):
        for s in range(S):
            assert res["tokens"][r, s] in res["ids"][r, s]
