"""Pins of the oracle's row-norm-sampling variant (CPU only).

* squared row norms: exact on integer-valued rows, and within fp32
  rounding of the fp64 sum otherwise;
* quantised weights: bracketed by exact rational arithmetic, largest in
  [2^39, 2^40);
* draws: the smallest t with c_t > r, against a linear scan; frequencies
  against the exact probabilities (chi-square);
* estimator: the expectation of the one-draw numerator, enumerated over
  every position with its exact probability, equals the exact residual
  product (keys outside the row's block) -- unbiasedness;
* equal-norm values reduce the weights to the uniform seg / m;
* block = n reduces the output to exact attention; the normaliser (lse)
  equals the uniform method's exactly;
* planted mistakes (uniform weight, norm instead of squared norm, wrong
  block in the exclusion) each trip one of these.

Causal variant (every quadrant with its own node's draws):
* the normaliser (lse) equals the uniform causal method's exactly;
* block >= n (every quadrant is one block) and min_seq_len >= n each give
  exact causal attention;
* unbiasedness of the whole causal numerator: with one draw per quadrant,
  the expectation of out e^lse -- each node's draw enumerated over every
  key position of that node with its exact probability -- equals the
  exact causal numerator sum_{j <= i} e^{q_i . k_j} v_j (spans of odd
  length included, so rectangular quadrants are covered);
* each node's weights are the squared norms of its own key rows;
* planted mistakes (weights ignoring the norms, weights of the wrong
  rows, the merge dropping the row-norm part, the wrong key block in the
  exclusion) each trip one of these.
"""

from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import rownorm as rn
from oracle import hyperattn as oh
from oracle.philox import philox_words


def test_row_norms_exact_on_integers():
    g = np.random.default_rng(1)
    v = g.integers(-40, 41, size=(50, 24)).astype(np.float32)
    assert np.array_equal(rn.row_norms_sq(v), np.sum(v.astype(np.int64) ** 2, axis=1).astype(np.float32))


def test_row_norms_close_to_fp64():
    g = np.random.default_rng(2)
    v = g.standard_normal((200, 64)).astype(np.float32)
    ref = np.sum(v.astype(np.float64) ** 2, axis=1)
    assert np.max(np.abs(rn.row_norms_sq(v) - ref) / ref) < 64 * 2.0 ** -24


def test_quantized_weights_bracket():
    g = np.random.default_rng(3)
    w = (g.standard_normal(300) ** 2 * np.exp(g.uniform(-8, 8, 300))).astype(np.float32)
    n = rn.quantized_weights(w)
    mx = max(Fraction(float(x)) for x in w)
    e = 0
    while Fraction(2) ** e <= mx:                       # mx = f 2^e, f in [0.5, 1)
        e += 1
    while Fraction(2) ** (e - 1) > mx:
        e -= 1
    scale = Fraction(2) ** (rn.QBITS - e)
    for wi, ni in zip(w, n):
        x = Fraction(float(wi)) * scale
        assert ni <= x < ni + 1
    assert 2 ** 39 <= int(n.max()) < 2 ** 40


def test_probabilities_follow_squared_norms():
    g = np.random.default_rng(12)
    v = (g.standard_normal((300, 16)) * np.exp(g.uniform(-2, 2, (300, 1)))).astype(np.float32)
    n = rn.quantized_weights(rn.row_norms_sq(v))
    sq = np.sum(v.astype(np.float64) ** 2, axis=1)
    assert np.max(np.abs(n / n.sum() - sq / sq.sum())) < 1e-6 * np.max(sq / sq.sum())


def test_draws_are_the_cdf_inverse():
    g = np.random.default_rng(4)
    n_sorted = g.integers(0, 50, size=37).astype(np.int64)
    n_sorted[[3, 10]] = 0                               # never drawn
    pos, T = rn.rownorm_positions(9, 1, 2, 3, n_sorted, 200)
    x = philox_words(9, 200, c1=3, c2=2, c3=4)
    c = np.cumsum(n_sorted)
    for i in range(200):
        r = (int(x[i]) * T) >> 32
        t = 0
        while c[t] <= r:
            t += 1
        assert pos[i] == t
    assert not np.any(np.isin(pos, [3, 10]))


def test_draw_frequencies():
    n_sorted = np.array([1, 5, 0, 20, 7, 3, 40, 2, 12, 10], dtype=np.int64)
    pos, T = rn.rownorm_positions(11, 0, 0, 1, n_sorted, 20000)
    counts = np.bincount(pos, minlength=len(n_sorted))
    keep = n_sorted > 0
    expected = 20000 * n_sorted[keep] / T
    assert counts[~keep].sum() == 0
    assert stats.chisquare(counts[keep], expected).pvalue > 1e-4


def _problem(ns, d, seed, equal_norms=False):
    g = np.random.default_rng(seed)
    q = g.standard_normal((ns, d)) * 0.4
    k = g.standard_normal((ns, d)) * 0.4
    v = g.standard_normal((ns, d)).astype(np.float32)
    if equal_norms:
        v = (v / np.linalg.norm(v, axis=1, keepdims=True) * 2.0).astype(np.float32)
        v[:, :] = v[0:1, :] * np.sign(g.standard_normal((ns, 1))).astype(np.float32)
    return q, k, v


def _sorted(q, k, v, r, seed):
    R = oracle.projections(seed, q.shape[1], r)
    pq = oh.sort_perm(oh.ranks(q.astype(np.float32), R))
    pk = oh.sort_perm(oh.ranks(k.astype(np.float32), R))
    return q[pq], k[pk], v.astype(np.float64)[pk], pk


@pytest.mark.parametrize("b_eff", [4, 8])
def test_one_draw_estimator_is_unbiased(b_eff):
    ns, d = 32, 6
    q, k, v = _problem(ns, d, 5)
    Qs, Ks, Vs, pk = _sorted(q, k, v, 3, 5)
    n_sorted = rn.quantized_weights(rn.row_norms_sq(v))[pk]
    T = int(n_sorted.sum())
    expect = np.zeros((ns, d))
    for t in range(ns):
        p = float(rn.exact_probability(n_sorted, t))
        if p == 0.0:
            continue
        lr, orr = rn.rownorm_part(Qs, Ks, Vs, np.array([t]), n_sorted, T, b_eff)
        num = np.where(np.isfinite(lr)[:, None], orr * np.exp(np.where(np.isfinite(lr), lr, 0.0))[:, None], 0.0)
        expect += p * num
    A = np.exp(Qs @ Ks.T)
    outside = (np.arange(ns)[:, None] // b_eff) != (np.arange(ns)[None, :] // b_eff)
    exact = (A * outside) @ Vs
    assert np.max(np.abs(expect - exact)) < 1e-12 * max(1.0, np.max(np.abs(exact)))


def test_equal_norms_give_uniform_weights():
    ns, d, m, b_eff = 64, 8, 40, 16
    q, k, v = _problem(ns, d, 6, equal_norms=True)
    Qs, Ks, Vs, pk = _sorted(q, k, v, 4, 6)
    n_sorted = rn.quantized_weights(rn.row_norms_sq(v))[pk]
    assert np.all(n_sorted == n_sorted[0])
    idx = np.random.default_rng(7).integers(0, ns, m)
    lr, orr = rn.rownorm_part(Qs, Ks, Vs, idx, n_sorted, int(n_sorted.sum()), b_eff)
    lu, ou = oh.sample_part(Qs, Ks, Vs, idx, b_eff)
    fin = np.isfinite(lu)
    assert np.array_equal(fin, np.isfinite(lr))
    assert np.max(np.abs(lr[fin] - lu[fin])) < 1e-12
    assert np.max(np.abs(orr[fin] - ou[fin])) < 1e-12


def test_one_block_is_exact_attention_and_lse_is_the_uniform_methods():
    B, H, n, d = 1, 2, 64, 8
    g = np.random.default_rng(8)
    q = (g.standard_normal((B, H, n, d)) * 0.5).astype(np.float32)
    k = (g.standard_normal((B, H, n, d)) * 0.5).astype(np.float32)
    v = g.standard_normal((B, H, n, d)).astype(np.float32)
    cfg = oh.HAConfig(block=n, samples=9, proj_bits=4, seed=3)
    o, l = rn.forward(q, k, v, cfg)
    oe, le = oh.exact_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    assert np.max(np.abs(o - oe)) < 1e-12 and np.max(np.abs(l - le)) < 1e-12
    cfg = oh.HAConfig(block=8, samples=9, proj_bits=4, seed=3)
    _, l1 = rn.forward(q, k, v, cfg)
    _, l2 = oh.forward(q, k, v, cfg)
    assert np.array_equal(l1, l2)


# ---- planted mistakes -------------------------------------------------------------------

_correct_part = rn.rownorm_part
_correct_quant = rn.quantized_weights


def _uniform_weight_part(Qs, Ks, Vs, idx, n_sorted, T, b_eff, positions=None, b_k=None):
    return oh.sample_part(Qs, Ks, Vs, idx, b_eff, positions, b_k)


def _wrong_block_part(Qs, Ks, Vs, idx, n_sorted, T, b_eff, positions=None, b_k=None):
    return _correct_part(Qs, Ks, Vs, idx, n_sorted, T, 1, positions, 1)


def _norm_not_squared(w32):
    return _correct_quant(np.sqrt(np.asarray(w32, dtype=np.float64)).astype(np.float32))


@pytest.mark.parametrize("target,mutant", [("rownorm_part", _uniform_weight_part),
                                           ("rownorm_part", _wrong_block_part)])
def test_planted_estimator_mistakes_are_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(rn, target, mutant)
    with pytest.raises(AssertionError):
        test_one_draw_estimator_is_unbiased(4)


def test_planted_norm_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(rn, "quantized_weights", _norm_not_squared)
    with pytest.raises(AssertionError):
        test_probabilities_follow_squared_norms()


# ---- causal variant -----------------------------------------------------------------------

def _causal_head(n, d, seed):
    g = np.random.default_rng(seed)
    q = (g.standard_normal((n, d)) * 0.5).astype(np.float32)
    k = (g.standard_normal((n, d)) * 0.5).astype(np.float32)
    v = g.standard_normal((n, d)).astype(np.float32)
    return q, k, v


def _causal_run(q, k, v, cfg):
    R = oracle.projections(cfg.seed, q.shape[1], cfg.proj_bits)
    rq, rk = oh.ranks(q, R), oh.ranks(k, R)
    return rn.causal_problem_rownorm(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), rq, rk, v,
                                     cfg.seed, 0, 0, cfg)


@pytest.mark.parametrize("n,s,block", [(64, 8, 4), (45, 6, 3)])
def test_causal_lse_is_the_uniform_methods(n, s, block):
    q, k, v = _causal_head(n, 8, 20 + n)
    cfg = oh.HAConfig(block=block, samples=5, proj_bits=4, causal=True, min_seq_len=s, seed=4)
    _, l1 = _causal_run(q, k, v, cfg)
    _, l2 = oh.forward(q[None, None], k[None, None], v[None, None], cfg)
    assert np.array_equal(l1, l2[0, 0])


@pytest.mark.parametrize("block,s", [(64, 8), (8, 64)])
def test_causal_limits_are_exact_attention(block, s):
    n = 64
    q, k, v = _causal_head(n, 8, 31)
    cfg = oh.HAConfig(block=block, samples=7, proj_bits=4, causal=True, min_seq_len=s, seed=5)
    o, l = _causal_run(q, k, v, cfg)
    oe, le = oh.exact_attention(q[None, None].astype(np.float64), k[None, None].astype(np.float64),
                                v[None, None].astype(np.float64), causal=True)
    assert np.max(np.abs(o - oe[0, 0])) < 1e-12 and np.max(np.abs(l - le[0, 0])) < 1e-12


def test_causal_numerator_is_unbiased(monkeypatch):
    # n = 20, min_seq_len 4: spans 20 -> 10 -> 5 -> (2, 3); the spans of 5
    # split unevenly (3 queries over 2 keys)
    n, d = 20, 6
    q, k, v = _causal_head(n, d, 41)
    cfg = oh.HAConfig(block=2, samples=1, proj_bits=3, causal=True, min_seq_len=4, seed=6)
    real = rn.rownorm_positions
    seen = {}                                          # node -> its sorted n_t

    def record(seed, b, h, node, n_sorted, m):
        seen[node] = np.asarray(n_sorted, dtype=np.int64).copy()
        return real(seed, b, h, node, n_sorted, m)

    monkeypatch.setattr(rn, "rownorm_positions", record)
    _causal_run(q, k, v, cfg)
    assert sorted(seen) == [1, 2, 3, 4, 5, 6, 7]
    # node -> its keys [lo, mid): the node's weights are the squared norms of
    # those value rows (as a multiset: the order is the node's sort)
    keys = {1: (0, 10), 2: (0, 5), 3: (10, 15), 4: (0, 2), 5: (5, 7), 6: (10, 12), 7: (15, 17)}
    for node, (lo, mid) in keys.items():
        sq = np.sum(v[lo:mid].astype(np.float64) ** 2, axis=1)
        got = np.sort(seen[node] / seen[node].sum())
        assert len(got) == mid - lo and np.max(np.abs(got - np.sort(sq / sq.sum()))) < 1e-6
    choice = {node: 0 for node in seen}

    def forced(seed, b, h, node, n_sorted, m):
        assert m == 1 and np.array_equal(n_sorted, seen[node])
        return np.array([choice[node]], dtype=np.int64), int(np.sum(n_sorted))

    monkeypatch.setattr(rn, "rownorm_positions", forced)

    def numerator():
        o, l = _causal_run(q, k, v, cfg)
        return o * np.exp(l)[:, None]

    base = numerator()
    expect = base.copy()
    for node, ns in seen.items():                       # the estimate is linear in each node's draw
        T = int(ns.sum())
        for t in range(len(ns)):
            if ns[t] == 0:
                continue
            choice[node] = t
            expect += (ns[t] / T) * (numerator() - base)
        choice[node] = 0
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    A = np.exp(q64 @ k64.T) * np.tri(n)
    exact = A @ v64
    assert np.max(np.abs(expect - exact)) < 1e-10 * np.max(np.abs(exact))


_correct_merge = rn.merge_variant
_correct_problem = rn.noncausal_problem_rownorm


def _flat_weights(w32):
    # planted: every key equally likely (the node's norms ignored)
    return np.full(np.shape(w32), 2 ** 39, dtype=np.int64)


def _merge_without_rownorm(lb, ob, lu, lr, orr):
    return _correct_merge(lb, ob, lu, lr, orr * 0.0)


def _query_rows_weights(q, k, v, rank_q, rank_k, v32, *args, **kw):
    # planted: the weights taken from rows other than the node's keys (the
    # head's last rows)
    return _correct_problem(q, k, v, rank_q, rank_k, _QUERY_V[0][-len(v32):], *args, **kw)


_QUERY_V = [None]


@pytest.mark.parametrize("target,mutant", [("quantized_weights", _flat_weights),
                                           ("merge_variant", _merge_without_rownorm),
                                           ("rownorm_part", _wrong_block_part),
                                           ("noncausal_problem_rownorm", _query_rows_weights)])
def test_planted_causal_mistakes_are_caught(monkeypatch, target, mutant):
    _QUERY_V[0] = _causal_head(20, 6, 41)[2]
    monkeypatch.setattr(rn, target, mutant)
    with pytest.raises(AssertionError):
        test_causal_numerator_is_unbiased(monkeypatch)
