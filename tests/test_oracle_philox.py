"""Pins of the oracle's counter-based uniforms: Philox-4x32-10 as published by
Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2,
3", SC 2011), checked against the known-answer vectors distributed with that
paper's reference implementation, and the mapping to uniforms."""
import numpy as np

from oracle import dflash_oracle as O


def test_philox_known_answers():
    cases = [
        ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
         (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
        ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
         (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
        ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
         (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
    ]
    for ctr, key, want in cases:
        assert O.philox4x32_10(ctr, key) == want


def test_uniforms_are_the_top_24_bits_of_each_word_in_counter_order():
    seed, offset = 0x0123456789ABCDEF, (1 << 32) - 1          # the offset carries into the second word
    u = O.philox_uniforms(seed, offset, 10)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    for b in range(3):
        c = offset + b
        words = O.philox4x32_10((c & 0xFFFFFFFF, c >> 32, 0, 0), key)
        for j in range(4):
            if 4 * b + j < 10:
                assert u[4 * b + j] == (words[j] >> 8) / 2.0 ** 24
    assert np.all((u >= 0) & (u < 1)) and np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))


def test_offsets_continue_one_stream():
    # drawing n then m numbers from offset o equals drawing n + m (n a multiple of 4)
    whole = O.philox_uniforms(7, 100, 20)
    assert np.array_equal(whole[:12], O.philox_uniforms(7, 100, 12))
    assert np.array_equal(whole[12:], O.philox_uniforms(7, 103, 8))


def test_uniforms_look_uniform():
    u = O.philox_uniforms(2024, 0, 40000)
    hist = np.histogram(u, bins=20, range=(0, 1))[0]
    chi2 = float(np.sum((hist - 2000) ** 2 / 2000))
    assert chi2 < 43.8                                          # 99.9% point of chi-square(19)
