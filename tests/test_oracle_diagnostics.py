"""Pins of the oracle diagnostics (CPU only).

* alpha: all scores equal (Q = 0) make P uniform, so every column's
  squared mass is n (1/n)^2 = 1/n; causal with Q = 0 gives the closed form
  c_j = sum_{i >= j} 1/(i+1)^2 = psi'(j+1) - psi'(n+1) (trigamma, scipy);
  a dominant diagonal (P close to I) gives alpha close to 1; skipping
  columns takes the maximum over the rest only;
* kappa: Q = 0 makes every residual row sum n - b_eff, so kappa = 1;
  r_i equals the exact row sum minus the block part's row sum of the
  forward's oracle (independent code path); one block leaves no residual
  (kappa infinite);
* planted mistakes (column norm not squared, rows instead of columns)
  trip the closed forms.
"""

import numpy as np
import pytest
from scipy import special

import oracle
from oracle import diagnostics as dg
from oracle import hyperattn as oh


def test_alpha_uniform_closed_form():
    n, d = 50, 8
    k = np.random.default_rng(1).standard_normal((n, d))
    c = dg.column_sqmass(np.zeros((n, d)), k)
    assert np.max(np.abs(c - 1.0 / n)) < 1e-15
    assert abs(dg.alpha(np.zeros((n, d)), k) - 1.0 / n) < 1e-15


def test_alpha_causal_closed_form():
    n, d = 40, 4
    k = np.random.default_rng(2).standard_normal((n, d))
    c = dg.column_sqmass(np.zeros((n, d)), k, causal=True)
    j = np.arange(n)
    ref = special.polygamma(1, j + 1) - special.polygamma(1, n + 1)
    assert np.max(np.abs(c - ref)) < 1e-13


def test_alpha_dominant_diagonal_and_skip():
    n, d = 30, 30
    q = np.eye(n) * 40.0
    k = np.eye(n)
    assert abs(dg.alpha(q, k) - 1.0) < 1e-12
    g = np.random.default_rng(3)
    q, k = g.standard_normal((n, d)), g.standard_normal((n, d))
    c = dg.column_sqmass(q, k)
    assert dg.alpha(q, k, skip=5) == float(np.max(c[5:]))
    assert dg.alpha(q, k, skip=5) <= dg.alpha(q, k)


def test_kappa_uniform_is_one():
    n, d, block = 64, 8, 16
    g = np.random.default_rng(4)
    k = g.standard_normal((n, d))
    rq = g.integers(0, 8, n)
    rk = g.integers(0, 8, n)
    r = dg.residual_row_sums(np.zeros((n, d)), k, rq, rk, block)
    assert np.max(np.abs(r - (n - block))) < 1e-12
    assert abs(dg.kappa(np.zeros((n, d)), k, rq, rk, block) - 1.0) < 1e-15


def test_residual_is_exact_minus_block_part():
    n, d, block = 96, 8, 16
    g = np.random.default_rng(5)
    q, k, v = g.standard_normal((n, d)) * 0.5, g.standard_normal((n, d)) * 0.5, g.standard_normal((n, d))
    R = oracle.projections(5, d, 4)
    rq, rk = oh.ranks(q.astype(np.float32), R), oh.ranks(k.astype(np.float32), R)
    r = dg.residual_row_sums(q, k, rq, rk, block)
    pq, pk = oh.sort_perm(rq), oh.sort_perm(rk)
    lb, _ = oh.block_part(q[pq], k[pk], v[pk], block)
    D = np.exp(q @ k.T).sum(axis=1)
    ref = np.empty(n)
    ref[pq] = D[pq] - np.exp(lb)
    assert np.max(np.abs(r - ref) / D) < 1e-12
    assert dg.kappa(q, k, rq, rk, n) == float("inf")


_correct = dg.column_sqmass


def _not_squared(q, k, causal=False):
    return np.sqrt(_correct(q, k, causal)) * np.sqrt(q.shape[0])


def _rows_not_columns(q, k, causal=False):
    P = dg._probabilities(q, k, causal)
    return np.sum(P * P, axis=1)


@pytest.mark.parametrize("mutant", [_not_squared, _rows_not_columns])
def test_planted_alpha_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(dg, "column_sqmass", mutant)
    with pytest.raises(AssertionError):
        test_alpha_uniform_closed_form()
        test_alpha_causal_closed_form()


@pytest.mark.parametrize("causal", [False, True])
def test_column_sqmass_cols_equals_dense(causal):
    """The chunked column masses (used at full sizes) equal the dense ones
    on the listed columns, with chunks that do not divide n."""
    g = np.random.default_rng(11)
    n, d = 301, 16
    q = g.standard_normal((n, d))
    k = g.standard_normal((n, d))
    cols = np.array([0, 1, 5, 150, 299, 300])
    want = dg.column_sqmass(q, k, causal)[cols]
    got = dg.column_sqmass_cols(q, k, cols, causal, chunk=64)
    assert np.allclose(got, want, rtol=1e-12, atol=0)
