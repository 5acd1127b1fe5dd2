"""Pins of the oracle backward (CPU only).

* the weight matrix W, fed to a plain weighted softmax, reproduces the
  step-by-step forward of ``oracle.hyperattn`` (non-causal and causal);
* central finite differences of that step-by-step forward (ranks and
  samples held fixed) match the analytic gradients;
* W = 1 (block >= n, or min_seq_len >= n causal) reduces to exact attention,
  whose gradients torch autograd computes in fp64;
* grouped heads: dK, dV of a KV head are the sums over its query heads;
* planted mistakes in the backward formula are caught by the finite
  differences;
* rectangular problems (n_q != n_k): the weights reproduce
  ``forward_rect`` and ``backward_rect`` matches finite differences;
* ``round_bf16`` (the bf16 output that D is formed from, reading R14b)
  equals torch's float32 -> bfloat16 conversion, ties included.
"""

import numpy as np
import pytest
import torch

from oracle import backward as ob
from oracle import hyperattn as oh
from oracle.gauss import projections

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(n, d, seed, scale=0.5):
    g = np.random.default_rng(seed)
    q = g.standard_normal((n, d)) * scale
    k = g.standard_normal((n, d)) * scale
    v = g.standard_normal((n, d))
    return q, k, v


def _ranks(q, k, r, seed):
    R = projections(seed, q.shape[1], r)
    return oh.ranks(q.astype(np.float32), R), oh.ranks(k.astype(np.float32), R)


def _fwd(q, k, v, rq, rk, cfg):
    """Step-by-step forward of one head with ranks held fixed."""
    if cfg.causal:
        return oh.causal_problem(q, k, v, rq, rk, cfg.seed, 0, 0, cfg)
    return oh.noncausal_problem(q, k, v, rq, rk, cfg.seed, 0, 0, 1, cfg.block, cfg.samples)


CASES = [
    oh.HAConfig(block=16, samples=12, proj_bits=4, seed=3),
    oh.HAConfig(block=8, samples=40, proj_bits=5, seed=4),                  # many duplicate samples
    oh.HAConfig(block=16, samples=10, proj_bits=4, causal=True, min_seq_len=16, seed=5),
    oh.HAConfig(block=4, samples=6, proj_bits=3, causal=True, min_seq_len=8, seed=6),
    oh.HAConfig(block=12, samples=10, proj_bits=4, seed=7),                 # ragged last block
    oh.HAConfig(block=12, samples=8, proj_bits=4, causal=True, min_seq_len=16, seed=8),  # ragged quadrants
]


def _weights(rq, rk, cfg):
    if cfg.causal:
        return ob.causal_weights(rq, rk, cfg.seed, 0, 0, cfg)
    return ob.noncausal_weights(rq, rk, cfg.seed, 0, 0, 1, cfg.block, cfg.samples)


@pytest.mark.parametrize("n", [64, 45])                                   # 45: odd causal splits
@pytest.mark.parametrize("cfg", CASES)
def test_weights_reproduce_the_forward(cfg, n):
    q, k, v = _inputs(n, 8, cfg.seed)
    rq, rk = _ranks(q, k, cfg.proj_bits, cfg.seed)
    o, lse = _fwd(q, k, v, rq, rk, cfg)
    W = _weights(rq, rk, cfg)
    o2, lse2 = ob.weighted_attention(q, k, v, W)
    assert np.max(np.abs(o - o2)) < 1e-12
    assert np.max(np.abs(lse - lse2)) < 1e-12


@pytest.mark.parametrize("cfg", CASES)
def test_gradients_match_finite_differences(cfg):
    n, d = 64, 8
    q, k, v = _inputs(n, d, cfg.seed + 10)
    rq, rk = _ranks(q, k, cfg.proj_bits, cfg.seed)
    do = np.random.default_rng(cfg.seed + 20).standard_normal((n, d))
    W = _weights(rq, rk, cfg)
    dq, dk, dv = ob.weighted_backward(q, k, v, W, do)

    def loss(q_, k_, v_):
        return float(np.sum(do * _fwd(q_, k_, v_, rq, rk, cfg)[0]))

    g = np.random.default_rng(cfg.seed + 30)
    h = 1e-5
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            i, j = int(g.integers(n)), int(g.integers(d))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][i, j] += h
            lp = loss(args["q"], args["k"], args["v"])
            args[name][i, j] -= 2 * h
            lm = loss(args["q"], args["k"], args["v"])
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i, j]) <= 1e-6 * max(1.0, abs(fd)), (name, i, j, fd, grad[i, j])


@pytest.mark.parametrize("causal", [False, True])
def test_exact_case_matches_autograd(causal):
    n, d = 48, 8
    q, k, v = _inputs(n, d, 7)
    do = np.random.default_rng(8).standard_normal((n, d))
    cfg = oh.HAConfig(block=n, samples=5, proj_bits=4, causal=causal, min_seq_len=n, seed=1)
    rq, rk = _ranks(q, k, cfg.proj_bits, cfg.seed)
    W = _weights(rq, rk, cfg)
    assert np.all(W == (np.tril(np.ones((n, n))) if causal else 1.0))
    dq, dk, dv = ob.weighted_backward(q, k, v, W, do)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    S = tq @ tk.T
    if causal:
        S = S.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    out = torch.softmax(S, dim=-1) @ tv
    out.backward(torch.tensor(do))
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(got - ref.numpy())) < 1e-12


def test_grouped_heads_sum_over_the_group():
    B, H, Hkv, n, d = 1, 4, 2, 32, 8
    g = np.random.default_rng(9)
    q = (g.standard_normal((B, H, n, d)) * 0.5).astype(np.float32)
    k = (g.standard_normal((B, Hkv, n, d)) * 0.5).astype(np.float32)
    v = g.standard_normal((B, Hkv, n, d)).astype(np.float32)
    do = g.standard_normal((B, H, n, d))
    cfg = oh.HAConfig(block=8, samples=6, proj_bits=4, seed=2)
    dq, dk, dv = ob.backward(q, k, v, do, cfg)
    R = projections(cfg.seed, d, cfg.proj_bits)
    for kv in range(Hkv):
        sk = np.zeros((n, d))
        sv = np.zeros((n, d))
        for h in (2 * kv, 2 * kv + 1):
            rq, rk = oh.ranks(q[0, h], R), oh.ranks(k[0, kv], R)
            W = ob.noncausal_weights(rq, rk, cfg.seed, 0, h, 1, cfg.block, cfg.samples)
            gq, gk, gv = ob.weighted_backward(q[0, h].astype(np.float64), k[0, kv].astype(np.float64),
                                              v[0, kv].astype(np.float64), W, do[0, h])
            assert np.array_equal(dq[0, h], gq)
            sk += gk
            sv += gv
        assert np.max(np.abs(dk[0, kv] - sk)) < 1e-12
        assert np.max(np.abs(dv[0, kv] - sv)) < 1e-12


_correct_backward = ob.weighted_backward


def _drop_d(q, k, v, W, do):           # forgets the row term D
    O, lse = ob.weighted_attention(q, k, v, W)
    P = np.where(W > 0, W * np.exp(q @ k.T - lse[:, None]), 0.0)
    dS = P * (do @ v.T)
    return dS @ k, dS.T @ q, P.T @ do


def _unweighted_p(q, k, v, W, do):     # drops the sample weight from P
    O, lse = ob.weighted_attention(q, k, v, W)
    P = np.where(W > 0, np.exp(q @ k.T - lse[:, None]), 0.0)
    dS = P * (do @ v.T - np.sum(do * O, axis=1)[:, None])
    return dS @ k, dS.T @ q, P.T @ do


def _transposed_dk(q, k, v, W, do):    # dK from dS instead of dS^T
    dq, dk, dv = _correct_backward(q, k, v, W, do)
    O, lse = ob.weighted_attention(q, k, v, W)
    P = np.where(W > 0, W * np.exp(q @ k.T - lse[:, None]), 0.0)
    dS = P * (do @ v.T - np.sum(do * O, axis=1)[:, None])
    return dq, dS @ q, dv


@pytest.mark.parametrize("mutant", [_drop_d, _unweighted_p, _transposed_dk])
def test_planted_backward_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(ob, "weighted_backward", mutant)
    with pytest.raises(AssertionError):
        test_gradients_match_finite_differences(CASES[0])


@pytest.mark.parametrize("nq,nk,block,m", [(12, 20, 4, 5), (21, 9, 5, 4)])
def test_rect_backward(nq, nk, block, m):
    from oracle import HAConfig
    rng = np.random.default_rng(nq * nk)
    q = (rng.standard_normal((1, 2, nq, 6)) * 0.7).astype(np.float32)
    k = (rng.standard_normal((1, 1, nk, 6)) * 0.7).astype(np.float32)
    v = rng.standard_normal((1, 1, nk, 6)).astype(np.float32)
    do = rng.standard_normal((1, 2, nq, 6))
    cfg = HAConfig(block=block, samples=m, proj_bits=3, seed=2)
    dq, dk, dv = ob.backward_rect(q, k, v, do, cfg)
    R = projections(2, 6, 3)
    Ws = [ob.noncausal_weights(oh.ranks(q[0, h], R), oh.ranks(k[0, 0], R), 2, 0, h, 1, block, m) for h in range(2)]
    q64, k64, v64 = (a.astype(np.float64) for a in (q, k, v))
    # the weights reproduce the rectangular forward
    o, l = oh.forward_rect(q, k, v, cfg)
    for h in range(2):
        O, L = ob.weighted_attention(q64[0, h], k64[0, 0], v64[0, 0], Ws[h])
        assert np.max(np.abs(O - o[0, h])) < 1e-12 and np.max(np.abs(L - l[0, h])) < 1e-12

    def f(qq, kk, vv):
        return sum(np.sum(do[0, h] * ob.weighted_attention(qq[0, h], kk[0, 0], vv[0, 0], Ws[h])[0])
                   for h in range(2))

    eps = 1e-6
    for arr, grad, idx in ((q64, dq, (0, 1, nq // 2, 2)), (k64, dk, (0, 0, nk // 2, 1)), (v64, dv, (0, 0, 1, 4))):
        plus, minus = arr.copy(), arr.copy()
        plus[idx] += eps
        minus[idx] -= eps
        args_p = [plus if a is arr else a for a in (q64, k64, v64)]
        args_m = [minus if a is arr else a for a in (q64, k64, v64)]
        fd = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd))


@pytest.mark.parametrize("n,block,m,seed", [
    (300, 64, 40, 1),      # ragged last block (300 = 4 x 64 + 44)
    (257, 50, 100, 2),     # many duplicate draws, ragged
    (256, 64, 0, 3),       # no samples: block part only
    (200, 256, 30, 4),     # one block holds every row: every draw excluded
    (512, 32, 16, 5),      # many small blocks
])
def test_block_backward_equals_dense(n, block, m, seed):
    """The block-wise backward (used at full sizes, where an n x n W does not
    fit) gives the dense-W backward's gradients for the same ranks and
    draws."""
    g = np.random.default_rng(seed)
    d = 16
    q = g.standard_normal((n, d)) * 0.5
    k = g.standard_normal((n, d)) * 0.5
    v = g.standard_normal((n, d))
    do = g.standard_normal((n, d))
    R = projections(seed, d, 5)
    rq, rk = oh.ranks(q.astype(np.float32), R), oh.ranks(k.astype(np.float32), R)
    W = ob.noncausal_weights(rq, rk, seed, 0, 3, 1, block, m)
    want = ob.weighted_backward(q, k, v, W, do)
    got = ob.noncausal_backward_blocks(q, k, v, do, rq, rk, seed, 0, 3, 1, block, m)
    for a, b, what in zip(got, want, ("dq", "dk", "dv")):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-12), what


@pytest.mark.parametrize("n,block,m,s,seed", [
    (512, 32, 16, 64, 6),     # three levels, even splits
    (301, 24, 10, 40, 7),     # odd splits at several levels, ragged blocks
    (256, 64, 0, 32, 8),      # no samples
    (200, 16, 40, 200, 9),    # one leaf: exact causal attention
])
@pytest.mark.parametrize("out_round", [None, ob.round_bf16], ids=["fp64_out", "bf16_out"])
def test_causal_dq_rows_equal_dense(n, block, m, s, seed, out_round):
    """Row-wise causal dq (used at full sizes) equals the dense-W backward's
    dq on every row, for the same ranks and draws (D from the exact or the
    bf16-rounded output)."""
    g = np.random.default_rng(seed)
    d = 16
    q = g.standard_normal((n, d)) * 0.5
    k = g.standard_normal((n, d)) * 0.5
    v = g.standard_normal((n, d))
    do = g.standard_normal((n, d))
    R = projections(seed, d, 5)
    rq, rk = oh.ranks(q.astype(np.float32), R), oh.ranks(k.astype(np.float32), R)
    cfg = oh.HAConfig(block=block, samples=m, proj_bits=5, causal=True, min_seq_len=s, seed=seed)
    W = ob.causal_weights(rq, rk, seed, 0, 2, cfg)
    want = ob.weighted_backward(q, k, v, W, do, out_round)[0]
    rows = np.arange(n)
    got = ob.causal_dq_rows(q, k, v, do, rq, rk, seed, 0, 2, cfg, rows, out_round=out_round)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)
    if out_round is not None:             # the rounding reaches dq
        assert not np.allclose(got, ob.weighted_backward(q, k, v, W, do)[0], rtol=1e-6, atol=1e-9)


def test_round_bf16_matches_torch():
    """round_bf16 equals torch's float32 -> bfloat16 conversion (nearest,
    ties to even) on fp32 values over a wide range, on exact ties (a bf16
    value plus half its last place, both signs, odd and even last bits)
    and on zero; a rounding to 7 or 9 bits, or one that breaks ties away
    from zero, fails it."""
    g = np.random.default_rng(3)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-20, 20, 20000))).astype(np.float32)
    b = torch.from_numpy(x[:4000]).to(torch.bfloat16).double().numpy()
    _, e = np.frexp(b)
    ties = (b + np.ldexp(1.0, e - 9)).astype(np.float32)     # half of 2^(e-8), the last place of 8 bits
    x = np.concatenate([x, ties, -ties, np.float32([0.0, 1.0, -2.5, 3.0])])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ob.round_bf16(x.astype(np.float64)), want)
