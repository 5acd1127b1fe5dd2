"""Pins of the oracle's sortLSH step: sign-bit hash, Gray-code rank, stable sort.

* Gray rank: exhaustive closed-form checks for every r <= 16.
* Hash bits: on integer-valued inputs the bits must equal the signs of
  exact integer dot products (pins the bit order, the sign convention and
  which projection is which).
* Exact sign: cancelling sums whose fp32 and fp64 evaluations lose the
  sign (hand-derived, in the test), and random fp32 rows against exact
  rational arithmetic (Python fractions).
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


def test_hash_exact_sign_hand_derived():
    # R = all ones, d = 64, one projection; the sign must be that of the
    # exact sum, whatever order a floating-point evaluation would take.
    #   row 0: 2^60 + 1 - 2^60 = 1 > 0 -> bit 1 (fp32 and fp64 running sums
    #          both absorb the 1 and give 0);
    #   row 1: the mirror, -1 -> bit 0;
    #   row 2: 1 + 2^24 - 2^24 - 1 = 0 exactly -> bit 0 (fp32 running sum
    #          gives -1, a halving order can give +1);
    #   row 3: 2^-100 + 2^50 - 2^50 = 2^-100 > 0 -> bit 1.
    x = np.zeros((4, 64), dtype=np.float32)
    x[0, 3], x[0, 17], x[0, 40] = 2.0**60, 1.0, -(2.0**60)
    x[1] = -x[0]
    x[2, 9], x[2, 20], x[2, 38], x[2, 39] = 1.0, 2.0**24, -(2.0**24), -1.0
    x[3, 0], x[3, 1], x[3, 63] = 2.0**-100, 2.0**50, -(2.0**50)
    R = np.ones((1, 64), dtype=np.float32)
    assert hyperattn.hash_codes(x, R).tolist() == [1, 0, 0, 1]


def test_hash_bits_equal_exact_rational_signs():
    from fractions import Fraction
    rng = np.random.default_rng(11)
    d, r = 16, 5
    R = rng.standard_normal((r, d)).astype(np.float32)
    x = rng.standard_normal((300, d)).astype(np.float32)
    # rows built to cancel: pairs x_i R_i = -x_j R_j exactly, plus rows
    # scaled far apart so that fp64 sums lose low-order terms
    x[:40] = 0.0
    for i in range(40):
        a, b = rng.choice(d, size=2, replace=False)
        x[i, a] = np.float32(2.0 ** int(rng.integers(-20, 20)))
        x[i, b] = -x[i, a]
    x[40:80] *= np.float32(2.0 ** 40)
    x[40:80, 0] = np.float32(2.0 ** -60)
    code = hyperattn.hash_codes(x, R)
    for i in range(len(x)):
        for p in range(r):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[i], R[p]))
            assert (int(code[i]) >> p) & 1 == (1 if exact > 0 else 0), (i, p)


def test_hash_zero_and_non_finite_give_bit_zero():
    R = np.ones((2, 64), dtype=np.float32)
    R[1] = -1.0
    x = np.ones((5, 64), dtype=np.float32)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 0] = -0.0
    x[2, 5] = np.nan
    x[3, 7] = np.inf                              # +inf: still bit 0 for both projections
    x[4, 7] = -np.inf
    assert hyperattn.hash_codes(x, R).tolist() == [0, 0, 0, 0, 0]
    R2 = np.ones((2, 64), dtype=np.float32)
    R2[1, 3] = np.nan                             # a non-finite projection gives bit 0 for every row
    assert hyperattn.hash_codes(np.ones((2, 64), dtype=np.float32), R2).tolist() == [1, 1]


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
