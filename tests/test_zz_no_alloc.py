"""GPU test of dflash_propose_block_noalloc, the entry point for callers that
cannot allocate: through the C ABI it must return exactly what
dflash_propose_block returns on the same inputs, on two calls in a row, the
second with a smaller batch (the shared scratch then still holds the first
call's data)."""
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import DEV, require_gpu, say

pytestmark = pytest.mark.gpu
KEYS = ("conv_out", "ids", "unary", "tokens", "q", "scores")


def _cfg(w):
    return D.make_config(taps=w.taps, group_size=w.group_size, rank=w.rank, top_k=w.top_k,
                         multiplier=w.multiplier, softcap=w.softcap, block_size=w.block_size, hidden=w.hidden)


def _both(w):
    inp = W.make_inputs(w, device=DEV)
    kw = dict(x=inp["x"], conv_base=inp["base"][0], conv_delta=inp["delta"][:, 0], logits=inp["logits"],
              anchor=inp["anchor"], sel_a=inp["sel_a"], sel_b=inp["sel_b"], proj=inp["proj"],
              uniforms=inp["uniforms"], temperatures=inp["temperatures"], greedy_mask=inp["greedy_mask"],
              valid_vocab=w.valid_vocab, keep_scores=True)
    say(f"dflash_propose_block_noalloc {w.name} (R={w.n_req})")
    got = D.dflash_propose_block_noalloc(_cfg(w), **kw)
    torch.cuda.synchronize()
    ref = D.dflash_propose_block(_cfg(w), **kw)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_equals_propose_block_on_two_calls_the_second_smaller():
    require_gpu()
    for name in ("stress_r1024_k32", "bf16_b16_v151936"):
        got, ref = _both(W.WORKLOADS[name])
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), (name, k)
