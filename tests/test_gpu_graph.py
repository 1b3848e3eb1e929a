"""GPU tests of the captured draft step ("[Spec] DFlash2", worker excerpt: one
captured graph serves greedy and sampled requests; the host stages the
temperatures and the greedy mask before each replay; the uniforms are drawn
inside the graph by a counter-based generator).

  * dflash_philox_uniforms equals the oracle's Philox-4x32-10 uniforms bit
    for bit (the oracle's generator is pinned by known-answer vectors).
  * Every replay of a ProposeGraph equals an eager step (dflash_philox_uniforms
    then dflash_propose_block on the same staged values) bit for bit, over
    several replays with different temperatures, greedy masks and counters,
    with eager work and synchronisations between the replays; the same
    counter replayed again gives the same tokens."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import DEV, require_gpu, say
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,offset,n", [(0, 0, 16), (0x0123456789ABCDEF, (1 << 32) - 2, 1003),
                                           ((1 << 64) - 1, 12345, 4097), (42, 7, 1)])
def test_philox_uniforms_match_the_oracle(seed, offset, n):
    require_gpu()
    so = torch.tensor([D.binding._as_i64(seed), D.binding._as_i64(offset)], dtype=torch.int64, device=DEV)
    say(f"dflash_philox_uniforms seed={seed:#x} offset={offset} n={n}")
    got = D.dflash_philox_uniforms(so, n)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().double().numpy(), O.philox_uniforms(seed, offset, n))


def _cfg(w: W.Workload):
    return D.make_config(taps=w.taps, group_size=w.group_size, rank=w.rank, top_k=w.top_k,
                         multiplier=w.multiplier, softcap=w.softcap, block_size=w.block_size, hidden=w.hidden)


@pytest.mark.parametrize("name", ["tiny_fp32", "nonpow2_b10_v151936", "bf16_b16_v151936"])
def test_graph_replays_equal_eager_steps(name):
    require_gpu()
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device=DEV)
    R, S = w.n_req, w.slots
    fixed = dict(x=inp["x"], conv_base=inp["base"][0], conv_delta=inp["delta"][:, 0], logits=inp["logits"],
                 anchor=inp["anchor"], sel_a=inp["sel_a"], sel_b=inp["sel_b"], proj=inp["proj"])
    say(f"ProposeGraph {name}: capture")
    g = D.ProposeGraph(_cfg(w), valid_vocab=w.valid_vocab, **fixed)
    # an eager twin on buffers of its own
    u_e = torch.empty((R, S), dtype=torch.float32, device=DEV)
    t_e = torch.empty(R, dtype=torch.float32, device=DEV)
    m_e = torch.empty(R, dtype=torch.uint8, device=DEV)
    so_e = torch.empty(2, dtype=torch.int64, device=DEV)
    eager = D.ProposeBlock(_cfg(w), uniforms=u_e, temperatures=t_e, greedy_mask=m_e, valid_vocab=w.valid_vocab,
                           **fixed)
    rng = np.random.default_rng(3)
    seen = []
    for step in range(4):
        temps = (0.3 + rng.random(R)).astype(np.float32)
        mask = (rng.random(R) < 0.5).astype(np.uint8)
        seed, offset = int(rng.integers(0, 1 << 62)), step * ((R * S + 3) // 4)
        say(f"ProposeGraph {name}: replay {step}")
        out = {k: v.clone() for k, v in g.replay(temps, mask, seed, offset).items()}
        torch.cuda.synchronize()
        # eager work of the program between replays, then the eager twin
        scratch = torch.randn(1 << 20, device=DEV).sum()
        so_e.copy_(torch.tensor([D.binding._as_i64(seed), D.binding._as_i64(offset)], dtype=torch.int64))
        t_e.copy_(torch.from_numpy(temps))
        m_e.copy_(torch.from_numpy(mask))
        D.dflash_philox_uniforms(so_e, R * S, out=u_e.view(-1))
        ref = eager()
        torch.cuda.synchronize()
        assert bool(torch.isfinite(scratch))
        for k in ("conv_out", "ids", "unary", "tokens", "q"):
            assert torch.equal(out[k], ref[k]), (name, step, k)
        assert np.array_equal(g.uniforms.cpu().double().numpy().ravel(), O.philox_uniforms(seed, offset, R * S))
        seen.append((seed, offset, temps, mask, out["tokens"].clone()))
    # the first counter again: the same draw
    seed, offset, temps, mask, tokens = seen[0]
    again = {k: v.clone() for k, v in g.replay(temps, mask, seed, offset).items()}
    torch.cuda.synchronize()
    assert torch.equal(again["tokens"], tokens)
    # the same step launched without the graph (the sweep's like-for-like row)
    say(f"ProposeGraph {name}: step_eager")
    eager_step = g.step_eager(temps, mask, seed, offset)
    torch.cuda.synchronize()
    for k in ("conv_out", "ids", "unary", "tokens", "q"):
        assert torch.equal(eager_step[k], again[k]), (name, "step_eager", k)
