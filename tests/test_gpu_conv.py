"""GPU parity of dflash_conv against the oracle's block-causal grouped conv
("[Spec] DFlash2", code excerpt of the grouped conv).  Bar: max relative
error (|got - ref| / max(|ref|, RMS(ref))) <= 1e-2 for bf16 output and 1e-5 for
fp32; the identity initialisation must be reproduced bit for bit.  bf16
outputs must also be the exact sum rounded once to nearest: within half a
bf16 spacing of the exact value, widened only by the fp32 accumulation bound
(a truncating or twice-rounding conversion fails this)."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import CONV_TOL, DEV, conv_rel_err, f64, require_gpu, sample_indices, say
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu


def _run_and_check(w: W.Workload, side: int, blocks=None):
    inp = W.make_inputs(w, device=DEV, parts=("conv",))
    x, base, delta = inp["x"], inp["base"][side], inp["delta"][:, side]
    say(f"dflash_conv {w.name} side={side} N={w.n_tokens} H={w.hidden} T={w.taps} B={w.block_size}")
    out = D.dflash_conv(x, base, delta, block_size=w.block_size, group_size=w.group_size)
    torch.cuda.synchronize()
    B = w.block_size
    nblk = w.n_tokens // B
    blks = np.arange(nblk) if blocks is None else sample_indices(nblk, blocks, seed=side)
    rows = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blks])
    idx = torch.from_numpy(rows).to(DEV)
    ref = O.conv(f64(x[idx]), f64(base), f64(delta[idx]), B, w.group_size)
    got = f64(out[idx])
    err = conv_rel_err(got, ref)
    assert err <= CONV_TOL[w.dtype], (w.name, side, err)
    if w.dtype == "bf16":
        _check_rounded_once(got, ref, f64(x[idx]), f64(base), f64(delta[idx]), B, w.group_size)
    return err


def _check_rounded_once(got, ref, x, base, delta, B, gs):
    """|got - exact| <= half the bf16 spacing at got's magnitude (taken on
    the larger side, 2^(e-8) for 2^e <= |got| < 2^(e+1)) + the fp32
    accumulation bound (T + 2) 2^-24 sum_t |coef_t x_t|."""
    mag = np.abs(O.conv(np.abs(x), np.abs(base), np.abs(delta), B, gs))   # >= sum_t |coef_t x_t|
    e = np.floor(np.log2(np.maximum(np.abs(got), 2.0 ** -126)))
    half = 2.0 ** (e - 8)
    T = base.shape[0]
    bound = half + (T + 2) * 2.0 ** -24 * mag
    ratio = np.abs(got - ref) / bound
    assert np.all(ratio <= 1.0), float(np.max(ratio))


@pytest.mark.parametrize("name", ["tiny_fp32", "bf16_b16_v151936", "nonpow2_b10_v151936"])
@pytest.mark.parametrize("side", [0, 1])
def test_conv_matches_oracle(name, side):
    require_gpu()
    _run_and_check(W.WORKLOADS[name], side)


@pytest.mark.parametrize("name", ["padded_v201024_k16", "stress_r1024_k32"])
def test_conv_full_size_sampled_blocks(name):
    require_gpu()
    _run_and_check(W.WORKLOADS[name], 0, blocks=24)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,T,gs,H", [(1, 4, 8, 64), (7, 3, 4, 40), (10, 5, 64, 320), (16, 9, 16, 96),
                                      (3, 1, 2, 24), (5, 8, 12, 48)])
def test_conv_edge_shapes(dtype, B, T, gs, H):
    # B = 1 (only tap 0), odd block sizes, taps above the register-history
    # limit (9), group sizes that split a 16-byte vector (2, 4, 12), T = 1.
    require_gpu()
    if H % (8 if dtype == "bf16" else 4):
        pytest.skip("hidden not a whole number of 16-byte vectors")
    w = W.Workload(name=f"edge_{dtype}_{B}_{T}_{gs}_{H}", n_req=3, block_size=B, hidden=H, group_size=gs,
                   taps=T, vocab=64, valid_vocab=64, top_k=4, rank=8, dtype=dtype, multiplier=1.0, softcap=0.0)
    _run_and_check(w, 0)
    _run_and_check(w, 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_identity_kernel_is_bitwise(dtype):
    # The module's initialisation (tap 0 = 1, other taps 0, no dynamic part)
    # must return the input unchanged, bit for bit.
    require_gpu()
    td = W.torch_dtype(dtype)
    N, H, T, G, B = 4 * 10, 128, 4, 2, 10
    x = W.normal((N, H), 1.0, dtype, 7, "x", DEV)
    base = torch.zeros((T, H), dtype=td, device=DEV)
    base[0] = 1
    delta = torch.zeros((N, T, G), dtype=td, device=DEV)
    say(f"dflash_conv identity {dtype}")
    out = D.dflash_conv(x, base, delta, block_size=B, group_size=H // G)
    torch.cuda.synchronize()
    assert torch.equal(out, x)


def test_empty_input_is_a_no_op():
    require_gpu()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    out = D.dflash_conv(x, torch.zeros((3, 64), dtype=torch.bfloat16, device=DEV),
                        torch.zeros((0, 3, 8), dtype=torch.bfloat16, device=DEV), block_size=4, group_size=8)
    assert out.shape == (0, 64)


def test_repeat_runs_are_bitwise_identical():
    require_gpu()
    w = W.WORKLOADS["nonpow2_b10_v151936"]
    inp = W.make_inputs(w, device=DEV, parts=("conv",))
    say("dflash_conv repeatability")
    a = D.dflash_conv(inp["x"], inp["base"][0], inp["delta"][:, 0], block_size=w.block_size, group_size=w.group_size)
    b = D.dflash_conv(inp["x"], inp["base"][0], inp["delta"][:, 0], block_size=w.block_size, group_size=w.group_size)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
