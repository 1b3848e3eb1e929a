"""Pins of the oracle's block-causal grouped conv against what the DFlash2
pages fix ("[Spec] DFlash2: local convolution + candidate selector", code
excerpt of the grouped conv and of the conv module): identity initialisation,
the single-tap case, block causality, the impulse response, runtime block
sizes (power of two or not) and a hand-worked example."""
import numpy as np
import pytest

from conftest import load_golden
from oracle import dflash_oracle as O


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def test_golden_hand_example():
    g = load_golden("conv_small.json")
    out = O.conv(np.array(g["x"], float), np.array(g["base"], float), np.array(g["delta"], float),
                 g["block_size"], g["group_size"])
    np.testing.assert_array_equal(out, np.array(g["expected"], float))


@pytest.mark.parametrize("B", [1, 4, 10, 16])
def test_identity_initialisation_is_exact(B):
    # The module initialises tap 0 to 1 and every other tap to 0; with zero
    # dynamic coefficients the conv must return its input unchanged.
    rng = np.random.default_rng(1)
    R, H, gs, T = 3, 24, 4, 5
    x = _rand(rng, R * B, H)
    base = np.zeros((T, H)); base[0] = 1.0
    delta = np.zeros((R * B, T, H // gs))
    np.testing.assert_array_equal(O.conv(x, base, delta, B, gs), x)


def test_single_tap_is_elementwise():
    rng = np.random.default_rng(2)
    N, H, gs, B = 12, 16, 4, 4
    x, base = _rand(rng, N, H), _rand(rng, 1, H)
    delta = _rand(rng, N, 1, H // gs)
    want = (base[0][None, :] + np.repeat(delta[:, 0, :], gs, axis=1)) * x
    np.testing.assert_allclose(O.conv(x, base, delta, B, gs), want, rtol=0, atol=1e-14)


def test_block_size_one_keeps_only_tap_zero():
    rng = np.random.default_rng(3)
    N, H, gs, T = 7, 8, 2, 4
    x, base, delta = _rand(rng, N, H), _rand(rng, T, H), _rand(rng, N, T, H // gs)
    want = (base[0][None, :] + np.repeat(delta[:, 0, :], gs, axis=1)) * x
    np.testing.assert_allclose(O.conv(x, base, delta, 1, gs), want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("B,T", [(4, 3), (10, 5), (16, 4), (3, 6)])
def test_impulse_response(B, T):
    # x = unit impulse at (token j0, channel c0): the output at (i, c0) must be
    # exactly the coefficient of tap i - j0 of OUTPUT token i, for the T - 1
    # tokens after j0 that stay inside j0's block; every other entry is zero.
    rng = np.random.default_rng(4)
    R, H, gs = 2, 12, 3
    N = R * B
    base, delta = _rand(rng, T, H), _rand(rng, N, T, H // gs)
    for j0 in [0, 1, B - 1, B, N - 1]:
        if j0 >= N:
            continue
        for c0 in [0, 5, H - 1]:
            x = np.zeros((N, H)); x[j0, c0] = 1.0
            out = O.conv(x, base, delta, B, gs)
            want = np.zeros((N, H))
            blk_end = (j0 // B + 1) * B
            for i in range(j0, min(j0 + T, blk_end)):
                want[i, c0] = base[i - j0, c0] + delta[i, i - j0, c0 // gs]
            np.testing.assert_array_equal(out, want)


def test_block_causality_by_perturbation():
    # The conv is linear in x; a change of x[j] may only reach out[i] with i
    # in j's block and 0 <= i - j < T.
    rng = np.random.default_rng(5)
    R, B, H, gs, T = 3, 6, 8, 2, 4
    N = R * B
    x, base, delta = _rand(rng, N, H), _rand(rng, T, H), _rand(rng, N, T, H // gs)
    ref = O.conv(x, base, delta, B, gs)
    for j in range(N):
        x2 = x.copy(); x2[j] += 1.0
        changed = np.flatnonzero(np.any(O.conv(x2, base, delta, B, gs) != ref, axis=1))
        allowed = [i for i in range(N) if i // B == j // B and 0 <= i - j < T]
        assert set(changed) <= set(allowed)
        assert j in changed


def test_requests_are_independent():
    # Running R requests together equals running each block alone.
    rng = np.random.default_rng(6)
    R, B, H, gs, T = 4, 10, 8, 4, 5
    N = R * B
    x, base, delta = _rand(rng, N, H), _rand(rng, T, H), _rand(rng, N, T, H // gs)
    whole = O.conv(x, base, delta, B, gs)
    parts = np.concatenate([O.conv(x[r * B:(r + 1) * B], base, delta[r * B:(r + 1) * B], B, gs)
                            for r in range(R)])
    np.testing.assert_array_equal(whole, parts)


@pytest.mark.parametrize("B", [16, 10])
def test_runtime_block_sizes_match_shift_form(B):
    # Shift form of the same conv: tap t adds coeff_t(i) * x[i - t] wherever
    # the in-block position is >= t (position via & for a power-of-two block
    # size, % otherwise); the oracle's per-block loop must agree exactly in
    # value (summation order differs, so compare to rounding).
    rng = np.random.default_rng(7)
    R, H, gs, T = 3, 16, 4, 4
    N = R * B
    x, base, delta = _rand(rng, N, H), _rand(rng, T, H), _rand(rng, N, T, H // gs)
    pos = np.arange(N) & (B - 1) if (B & (B - 1)) == 0 else np.arange(N) % B
    want = np.zeros((N, H))
    for t in range(T):
        coeff = base[t][None, :] + np.repeat(delta[:, t, :], gs, axis=1)
        shifted = np.zeros_like(x); shifted[t:] = x[: N - t]
        want += coeff * shifted * (pos >= t)[:, None]
    np.testing.assert_allclose(O.conv(x, base, delta, B, gs), want, rtol=1e-13, atol=1e-13)


def test_scaling_input_by_two_is_exact():
    rng = np.random.default_rng(8)
    R, B, H, gs, T = 2, 5, 8, 2, 3
    x, base, delta = _rand(rng, R * B, H), _rand(rng, T, H), _rand(rng, R * B, T, H // gs)
    np.testing.assert_array_equal(O.conv(2 * x, base, delta, B, gs), 2 * O.conv(x, base, delta, B, gs))


def test_round_to_bf16_known_values():
    # bf16 keeps 8 significant bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    # and goes to the even one (1); 1 + 3*2^-8 goes up to 1 + 2^-6.
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -3.0, 2.0 ** -133, 2.0 ** -134, 3.5e38, 0.0])
    got = O.round_to_bf16(v)
    np.testing.assert_array_equal(got, [1.0, 1.0, 1 + 2 ** -6, -3.0, 2.0 ** -133, 0.0, np.inf, 0.0])


def test_round_to_bf16_matches_torch_on_fp32_values():
    # For inputs that are already fp32 numbers, one RNE rounding to bf16 is
    # what torch's fp32 -> bf16 conversion does.
    import torch
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(20000) * 10.0).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(v).float().to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.round_to_bf16(v), want)
