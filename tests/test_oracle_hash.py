"""Pins of the oracle's sortLSH step: sign-bit hash, Gray-code rank, stable sort.

* Gray rank: exhaustive closed-form checks for every r <= 16.
* Hash bits: on integer-valued inputs every fp32 product and partial sum
  is exact, so the bits must equal the signs of exact integer dot products
  (pins the bit order, the sign convention and which projection is which).
* Summation order: a hand-derived fp32 case whose sign depends on the
  order (derivation in the test).
* Sort: Python's ``sorted`` on (rank, index) pairs.
"""

import numpy as np
import pytest

from oracle import gauss, hyperattn


@pytest.mark.parametrize("r", list(range(1, 17)))
def test_gray_inverse_exhaustive(r):
    codes = np.arange(1 << r, dtype=np.uint32)
    rank = hyperattn.gray_inverse(codes, r)
    # bijection on [0, 2^r)
    assert np.array_equal(np.sort(rank), codes)
    # it inverts the reflected-binary Gray code g(k) = k ^ (k >> 1)
    assert np.array_equal(rank ^ (rank >> np.uint32(1)), codes)
    # codes ordered by rank: neighbours differ in exactly one bit
    order = codes[np.argsort(rank)]
    diff = order[1:] ^ order[:-1]
    assert np.all(diff != 0) and np.all((diff & (diff - 1)) == 0)


@pytest.mark.parametrize("d,r", [(64, 7), (128, 8), (128, 16), (64, 1), (8, 3), (4, 5), (32, 12)])
def test_hash_bits_equal_exact_integer_signs(d, r):
    rng = np.random.default_rng(d * 100 + r)
    x = rng.integers(-8, 9, size=(500, d)).astype(np.float32)
    R = rng.integers(-8, 9, size=(r, d)).astype(np.float32)
    x[0] = 0.0                                   # all-zero row: every bit 0
    exact = x.astype(np.int64) @ R.astype(np.int64).T
    code = hyperattn.hash_codes(x, R)
    expect = np.zeros(len(x), dtype=np.uint32)
    for p in range(r):
        expect |= (exact[:, p] > 0).astype(np.uint32) << np.uint32(p)
    assert np.array_equal(code, expect)
    assert code[0] == 0


def test_hash_summation_order_hand_derived():
    # R = all ones, d = 64, one projection.  Nonzero inputs:
    #   x[9] = 1, x[20] = 2^24, x[38] = -2^24, x[39] = -1   (exact sum 0).
    # Defined order: groups of 8 consecutive elements, each summed by
    # halving (pairs 4 apart, 2 apart, 1 apart), then the 8 group sums by
    # halving.
    #   group 1 = 1;  group 2 = 2^24;
    #   group 4: pairs 4 apart give (-2^24, -1) in slots (2, 3), then slots
    #   (0, 1) = (-2^24, -1), then -2^24 - 1 = -16777217 rounds to -2^24
    #   (tie to even);
    #   group sums [0, 1, 2^24, 0, -2^24, 0, 0, 0]: pairs 4 apart
    #   [-2^24, 1, 2^24, 0], pairs 2 apart [0, 1], total +1 > 0 -> bit 1.
    # (Plain halving over 64 gives 0, a running sum -1: both bit 0.)
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, 9], x[0, 20], x[0, 38], x[0, 39] = 1.0, 2.0**24, -(2.0**24), -1.0
    x[1] = -x[0]                                  # mirror: total -1 -> bit 0
    R = np.ones((1, 64), dtype=np.float32)
    t = hyperattn.projection_sums(x, R)
    assert t[0, 0] == 1.0 and t[1, 0] == -1.0
    assert hyperattn.hash_codes(x, R).tolist() == [1, 0]


def test_hash_zero_and_negative_zero_give_bit_zero():
    R = np.ones((2, 64), dtype=np.float32)
    R[1] = -1.0
    x = np.zeros((3, 64), dtype=np.float32)
    x[1, 0] = -0.0
    x[2, 5] = np.nan
    assert hyperattn.hash_codes(x, R).tolist() == [0, 0, 0]


def test_hash_agrees_with_fp64_signs_away_from_zero():
    rng = np.random.default_rng(7)
    R = gauss.projections(3, 128, 8)
    x = rng.standard_normal((4000, 128)).astype(np.float32)
    t64 = x.astype(np.float64) @ R.astype(np.float64).T
    code = hyperattn.hash_codes(x, R)
    bits = (code[:, None] >> np.arange(8, dtype=np.uint32)[None, :]) & 1
    scale = np.linalg.norm(x, axis=1)[:, None] * np.linalg.norm(R, axis=1)[None, :]
    clear = np.abs(t64) > 1e-5 * scale
    assert np.array_equal(bits[clear], (t64[clear] > 0).astype(np.uint32))


@pytest.mark.parametrize("n,r", [(1, 7), (7, 1), (1000, 7), (4096, 8), (3000, 12)])
def test_sort_perm_is_stable_rank_order(n, r):
    rng = np.random.default_rng(n + r)
    rank = rng.integers(0, 1 << r, size=n).astype(np.uint32)
    perm = hyperattn.sort_perm(rank)
    ref = sorted(range(n), key=lambda i: (int(rank[i]), i))
    assert perm.tolist() == ref
