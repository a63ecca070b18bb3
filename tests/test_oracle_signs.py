"""Pins of the oracle's seeded random-sign generator (SplitMix64).

The generator is the one of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators" (OOPSLA 2014), in the form of Vigna's
public-domain splitmix64.c.  The expected outputs are its first outputs as
published elsewhere: for seed 1234567 the values the Rosetta Code task
"Pseudo-random numbers/Splitmix64" lists, for seed 0 the widely quoted first
three outputs.  A wrong constant, shift or counter offset changes all of them."""
import numpy as np

import oracle as O

PUBLISHED = {
    0: [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F],
    1234567: [6457827717110365317, 3203168211198807973, 9817491932198370423],
}


def test_splitmix64_published_outputs():
    for seed, outs in PUBLISHED.items():
        assert [O.splitmix64(seed, n) for n in range(len(outs))] == outs


def test_seeded_signs_follow_top_bit():
    s = O.seeded_signs(0, 1, 0)
    assert s.dtype == np.int8 and s.shape == (1, 128)
    # outputs 0 and 1 of seed 0 have top bits 1 and 0; output 2 has top bit 0
    assert list(s[0, :3]) == [-1, 1, 1]


def test_seeded_signs_layout_and_balance():
    H = 8
    k = O.seeded_signs(12345, H, 0)
    v = O.seeded_signs(12345, H, 1)
    assert set(np.unique(k)) <= {-1, 1} and set(np.unique(v)) <= {-1, 1}
    # head h is a slice of one counter stream: head 1 of H heads == head 0 shifted by d outputs
    assert np.array_equal(k[1], np.array([-1 if O.splitmix64(12345, 128 + i) >> 63 else 1 for i in range(128)]))
    # D_K and D_V and different seeds are distinct draws
    assert not np.array_equal(k, v)
    assert not np.array_equal(k, O.seeded_signs(12346, H, 0))
    # a fair coin: 2048 draws, |sum| within 5 sigma (sigma = sqrt(2048) ~ 45)
    assert abs(int(k.astype(int).sum()) + int(v.astype(int).sum())) < 5 * 45
