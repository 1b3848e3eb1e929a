"""GPU parity of dflash_conv_prepare (the conv module's kernel projection and
its side-0 convolution, "[Spec] DFlash2", code excerpt of the grouped conv
module) and of finish through dflash_conv with side 1.

Bars:
  * coefficients (bf16): each equals the oracle's rounding of the exact sum,
    or the other neighbour where the exact sum lies within the fp32
    accumulation bound H 2^-24 sum_k |x_k||w_k| of a rounding midpoint (both
    checked; counted); fp32: within that bound of the exact sum.
  * out: against the oracle's conv fed the GPU's own side-0 coefficients,
    max relative error <= 1e-2 (bf16) / 1e-5 (fp32), as for dflash_conv; and
    bit for bit equal to dflash_conv run on those coefficients (the chain).
  * finish: dflash_conv with base2[1] and coeff[:, 1] against the oracle's
    conv_finish on the GPU's coefficients."""
import numpy as np
import pytest
import torch

import block_draft_proposal_amd as D
import workloads as W
from gpu_helpers import CONV_TOL, DEV, conv_rel_err, f64, require_gpu, sample_indices, say
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu


def _check_coeff(got: np.ndarray, x: np.ndarray, w: np.ndarray, dtype: str) -> int:
    """got [rows, P] float64 copies of the GPU coefficients of rows x."""
    exact = x @ w.T
    bound = O.lm_head_sum_bound(x, w)
    if dtype == "f32":
        assert np.all(np.abs(got - exact) <= bound + np.abs(exact) * 2.0 ** -24), float(np.max(np.abs(got - exact)))
        return 0
    ref = O.round_to_bf16(exact)
    lo, hi = O.round_to_bf16(exact - bound), O.round_to_bf16(exact + bound)
    off = got != ref
    assert np.all(~off | ((got >= lo) & (got <= hi))), float(np.max(np.abs(got - ref)))
    return int(off.sum())


def _run(w: W.Workload, blocks=None, seed=None):
    d = W.make_conv_module_inputs(w, device=DEV, seed=seed)
    x, y, pw, base2 = d["x"], d["y"], d["proj_weight"], d["base2"]
    N, H, T, gs, B = x.shape[0], w.hidden, w.taps, w.group_size, w.block_size
    G = H // gs
    say(f"dflash_conv_prepare {w.name} N={N} H={H} T={T} G={G} B={B} {w.dtype}")
    out, coeff = D.dflash_conv_prepare(x, pw, base2, block_size=B, group_size=gs)
    chain = D.dflash_conv(x, base2[0], coeff[:, 0], block_size=B, group_size=gs)
    fin = D.dflash_conv(y, base2[1], coeff[:, 1], block_size=B, group_size=gs)
    torch.cuda.synchronize()
    assert torch.equal(out, chain)                       # the conv of prepare is dflash_conv on its coefficients
    nblk = N // B
    blks = np.arange(nblk) if blocks is None else sample_indices(nblk, blocks, seed=7)
    rows = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blks])
    idx = torch.from_numpy(rows).to(DEV)
    c_got = f64(coeff[idx]).reshape(len(rows), 2 * T * G)
    near = _check_coeff(c_got, f64(x[idx]), f64(pw), w.dtype)
    cg = c_got.reshape(len(rows), 2, T, G)
    ref_out = O.conv(f64(x[idx]), f64(base2[0]), cg[:, 0], B, gs)
    ref_fin = O.conv_finish(f64(y[idx]), cg, f64(base2), B, gs)
    e1, e2 = conv_rel_err(f64(out[idx]), ref_out), conv_rel_err(f64(fin[idx]), ref_fin)
    assert e1 <= CONV_TOL[w.dtype] and e2 <= CONV_TOL[w.dtype], (e1, e2)
    print(f"[conv_prepare] {w.name}: {near} coefficients on the rounding band; rel err {e1:.2e} / {e2:.2e}",
          flush=True)


@pytest.mark.parametrize("name", ["tiny_fp32", "bf16_b16_v151936", "nonpow2_b10_v151936"])
def test_prepare_and_finish_match_the_oracle(name):
    require_gpu()
    _run(W.WORKLOADS[name])


@pytest.mark.parametrize("name", ["padded_v201024_k16", "stress_r1024_k32"])
def test_prepare_full_size_sampled_blocks(name):
    require_gpu()
    _run(W.WORKLOADS[name], blocks=12)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("R,B,T,gs,H", [(3, 10, 3, 8, 200), (13, 10, 5, 16, 64), (1, 4, 2, 4, 40),
                                        (40, 4, 4, 8, 1024), (2, 16, 1, 64, 64), (9, 7, 9, 4, 96)])
def test_prepare_edge_shapes(dtype, R, B, T, gs, H):
    # token counts that end inside a 128-row tile, coefficient counts that end
    # inside a tile (2 T G = 150, 40, 20, 1024, 2, 432), hidden sizes
    # that are not a multiple of the 64-deep stage (200, 40, 96), T = 1,
    # T = 9 (the generic conv), a split contraction (H = 1024 with 160 tokens)
    # and the 64 x 64 tile
    require_gpu()
    if H % (8 if dtype == "bf16" else 4):
        pytest.skip("hidden not a whole number of 16-byte vectors")
    w = W.Workload(name=f"prep_{dtype}_{R}_{B}_{T}_{gs}_{H}", n_req=R, block_size=B, hidden=H, group_size=gs,
                   taps=T, vocab=64, valid_vocab=64, top_k=4, rank=8, dtype=dtype, multiplier=1.0, softcap=0.0)
    _run(w, seed=R * 100 + H)


def test_prepare_split_contraction_is_deterministic_and_empty_is_a_no_op():
    # the bench-size call splits the contraction over slices; repeated calls
    # give the same bits
    require_gpu()
    w = W.WORKLOADS["bf16_b16_v151936"]
    assert D.lib().dflash_conv_prepare_workspace_size(w.n_tokens, w.hidden, w.group_size, w.taps, 1) > 0
    d = W.make_conv_module_inputs(w, device=DEV)
    a = D.dflash_conv_prepare(d["x"], d["proj_weight"], d["base2"], block_size=w.block_size, group_size=w.group_size)
    b = D.dflash_conv_prepare(d["x"], d["proj_weight"], d["base2"], block_size=w.block_size, group_size=w.group_size)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    e = torch.zeros((0, w.hidden), dtype=torch.bfloat16, device=DEV)
    out, coeff = D.dflash_conv_prepare(e, d["proj_weight"], d["base2"], block_size=w.block_size,
                                       group_size=w.group_size)
    assert out.shape == (0, w.hidden) and coeff.shape[0] == 0
