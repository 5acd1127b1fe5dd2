"""Pins of the oracle's rectangular problems (n_q queries, n_k keys; CPU only).

* brute force from A = exp(Q K^T) and an explicit n_q x n_k block mask
  (query block t = sorted positions [t b, (t+1) b), key block t = sorted
  key positions [t b_k, (t+1) b_k), sample weight n_k / m) at 1e-12;
* n_k = n_q reproduces the square forward exactly; b >= n_q puts every key
  in the one block (exact attention over all keys);
* the one-sample estimate of the residual mass, averaged over every key
  position, equals the exact residual row sum (unbiasedness);
* b_k reduces to b for square problems and never makes more nonempty key
  blocks than query blocks.
"""

import numpy as np
import pytest

import oracle
from oracle import HAConfig
from oracle import hyperattn as oh


def _rand(rng, B, H, Hkv, nq, nk, d, scale=0.7):
    q = (rng.standard_normal((B, H, nq, d)) * scale).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, nk, d)) * scale).astype(np.float32)
    v = rng.standard_normal((B, Hkv, nk, d)).astype(np.float32)
    return q, k, v


def _brute(q, k, v, rq, rk, idx, b, b_k):
    nq, nk = q.shape[0], k.shape[0]
    A = np.exp(q @ k.T)
    pq = sorted(range(nq), key=lambda i: (int(rq[i]), i))
    pk = sorted(range(nk), key=lambda j: (int(rk[j]), j))
    qblk = np.empty(nq, dtype=np.int64)
    kblk = np.empty(nk, dtype=np.int64)
    for pos, i in enumerate(pq):
        qblk[i] = pos // b
    for pos, j in enumerate(pk):
        kblk[j] = pos // b_k
    M = (qblk[:, None] == kblk[None, :]).astype(np.float64)
    D = (A * M).sum(1)
    N = (A * M) @ v
    for s in idx:
        j = pk[s]
        w = (nk / len(idx)) * A[:, j] * (1.0 - M[:, j])
        D = D + w
        N = N + w[:, None] * v[j][None, :]
    return N / D[:, None], np.log(D)


@pytest.mark.parametrize("nq,nk,block,m", [(48, 20, 8, 11), (20, 52, 6, 9), (33, 70, 10, 25), (64, 16, 16, 5)])
def test_rect_brute_force(nq, nk, block, m):
    rng = np.random.default_rng(nq * nk + block)
    q, k, v = _rand(rng, 1, 1, 1, nq, nk, 6)
    cfg = HAConfig(block=block, samples=m, proj_bits=3, seed=2)
    out, lse = oh.forward_rect(q, k, v, cfg)
    R = oracle.projections(2, 6, 3)
    rq, rk = oh.ranks(q[0, 0], R), oh.ranks(k[0, 0], R)
    b = min(block, nq)
    b_k = -(-b * nk // nq)
    idx = oh.sample_positions(2, 0, 0, 1, nk, m)
    o_ref, l_ref = _brute(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64),
                          rq, rk, idx, b, b_k)
    assert np.max(np.abs(out[0, 0] - o_ref)) < 1e-12
    assert np.max(np.abs(lse[0, 0] - l_ref)) < 1e-12


def test_square_reduces_to_forward():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 2, 2, 1, 40, 40, 8)
    cfg = HAConfig(block=12, samples=7, proj_bits=4, seed=5)
    a = oh.forward_rect(q, k, v, cfg)
    b = oh.forward(q, k, v, cfg)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_one_block_is_exact_attention():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 1, 2, 2, 30, 75, 8)
    out, lse = oh.forward_rect(q, k, v, HAConfig(block=30, samples=9, proj_bits=4, seed=6))
    for h in range(2):
        S = q[0, h].astype(np.float64) @ k[0, h].astype(np.float64).T
        P = np.exp(S - S.max(1, keepdims=True))
        ref = (P / P.sum(1, keepdims=True)) @ v[0, h]
        assert np.max(np.abs(out[0, h] - ref)) < 1e-12


@pytest.mark.parametrize("nq,nk,block", [(40, 17, 8), (17, 40, 5)])
def test_one_sample_estimate_is_unbiased(nq, nk, block):
    rng = np.random.default_rng(nq + nk)
    q, k, v = _rand(rng, 1, 1, 1, nq, nk, 6)
    q, k, v = (a[0, 0].astype(np.float64) for a in (q, k, v))
    R = oracle.projections(7, 6, 3)
    rq, rk = oh.ranks(q.astype(np.float32), R), oh.ranks(k.astype(np.float32), R)
    pq, pk = oh.sort_perm(rq), oh.sort_perm(rk)
    Qs, Ks, Vs = q[pq], k[pk], v[pk]
    b = min(block, nq)
    b_k = oh.key_block(b, nq, nk)
    mean = np.zeros(nq)
    for t in range(nk):
        l, _ = oh.sample_part(Qs, Ks, Vs, np.array([t]), b, b_k=b_k)
        mean += np.where(np.isfinite(l), np.exp(l), 0.0) / nk
    A = np.exp(Qs @ Ks.T)
    outside = (np.arange(nq)[:, None] // b) != (np.arange(nk)[None, :] // b_k)
    assert np.max(np.abs(mean - (A * outside).sum(1)) / A.sum(1)) < 1e-12


def test_key_block_properties():
    for nq in range(1, 60):
        for b in range(1, nq + 1):
            assert oh.key_block(b, nq, nq) == b
            for nk in (1, 7, 64, 200):
                bk = oh.key_block(b, nq, nk)
                assert -(-nk // bk) <= -(-nq // b)
