"""Pins of the oracle's attention steps against textbook definitions.

* block >= segment: every row's block is the whole segment and every sample
  is excluded, so the method reduces to exact softmax attention, checked
  against ``scipy.special.softmax`` at 1e-12 (non-causal; and causal with
  min_seq_len >= n, or block >= n/2 so that every quadrant is one block).
* tiny n: A = exp(Q K^T) enumerated in full, the block mask M^H built
  explicitly from the permutations, the sampled columns enumerated, and the
  normaliser D, its block and sampled parts and the output compared with
  the oracle at 1e-12.
* unbiasedness: averaging the one-sample estimate over all ns positions
  gives exactly the out-of-block mass, so E[D_hat] = D.
* mass invariant: exp(lse) = exp(lse_blk) + exp(lse_smp) per row.
* merge: the log-sum-exp merge equals the direct quotient
  (N1 + N2) / (D1 + D2).
* planted mistakes: plausible bugs put into the oracle (on the CPU) make
  these pins fail.
"""

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import hyperattn
from oracle.hyperattn import HAConfig


def _rand_qkv(rng, B, H, Hkv, n, d, scale=None):
    s = d ** -0.25 if scale is None else scale
    q = (rng.standard_normal((B, H, n, d)) * s).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, n, d)) * s).astype(np.float32)
    v = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    return q, k, v


def _textbook(q, k, v, causal):
    B, H, n, d = q.shape
    G = H // k.shape[1]
    out = np.zeros((B, H, n, d))
    for b in range(B):
        for h in range(H):
            S = q[b, h].astype(np.float64) @ k[b, h // G].astype(np.float64).T
            if causal:
                S = np.where(np.tril(np.ones((n, n), bool)), S, -np.inf)
            out[b, h] = softmax(S, axis=1) @ v[b, h // G].astype(np.float64)
    return out


@pytest.mark.parametrize("n,block,m", [(64, 64, 0), (64, 1000, 16), (96, 96, 50), (1, 1, 3)])
def test_full_block_is_exact_attention(n, block, m):
    rng = np.random.default_rng(n + m)
    q, k, v = _rand_qkv(rng, 2, 4, 2, n, 16, scale=0.7)
    out, lse = oracle.forward(q, k, v, HAConfig(block=block, samples=m, proj_bits=5, seed=11))
    assert np.max(np.abs(out - _textbook(q, k, v, False))) < 1e-12
    ex_out, ex_lse = oracle.exact_attention(q, k, v)
    assert np.max(np.abs(lse - ex_lse)) < 1e-12


@pytest.mark.parametrize("n,s,block", [(64, 64, 8), (64, 100, 8), (128, 16, 64), (96, 12, 48),
                                       (45, 6, 64), (101, 10, 51)])    # odd splits (R19)
def test_causal_special_cases_are_exact_causal(n, s, block):
    rng = np.random.default_rng(n + s + block)
    q, k, v = _rand_qkv(rng, 1, 2, 1, n, 8, scale=0.8)
    out, _ = oracle.forward(q, k, v, HAConfig(block=block, samples=7, proj_bits=4,
                                              causal=True, min_seq_len=s, seed=3))
    assert np.max(np.abs(out - _textbook(q, k, v, True))) < 1e-12


def _brute_force_problem(q, k, v, rank_q, rank_k, idx, block):
    """Everything built from A = exp(Q K^T) and an explicit n x n mask."""
    n = q.shape[0]
    b_eff = min(block, n)
    A = np.exp(q @ k.T)
    pq = sorted(range(n), key=lambda i: (int(rank_q[i]), i))
    pk = sorted(range(n), key=lambda i: (int(rank_k[i]), i))
    qblk = np.empty(n, dtype=np.int64)
    kblk = np.empty(n, dtype=np.int64)
    for pos, i in enumerate(pq):
        qblk[i] = pos // b_eff
    for pos, j in enumerate(pk):
        kblk[j] = pos // b_eff
    M = (qblk[:, None] == kblk[None, :]).astype(np.float64)        # M^H
    D_blk = (A * M).sum(1)
    N_blk = (A * M) @ v
    m = len(idx)
    D_smp = np.zeros(n)
    N_smp = np.zeros_like(v)
    for s in idx:                       # sorted key position s -> key pk[s]
        j = pk[s]
        w = (n / m) * A[:, j] * (1.0 - M[:, j])
        D_smp += w
        N_smp += w[:, None] * v[j][None, :]
    return D_blk, D_smp, (N_blk + N_smp) / (D_blk + D_smp)[:, None], pq


@pytest.mark.parametrize("n,d,block,m,r", [(64, 4, 8, 16, 3), (48, 8, 16, 9, 4), (32, 8, 4, 40, 2), (64, 8, 64, 5, 3),
                                           (50, 4, 16, 12, 3), (40, 8, 12, 30, 3)])     # ragged last block
def test_tiny_n_brute_force(n, d, block, m, r):
    rng = np.random.default_rng(1000 + n + d + m)
    q = rng.standard_normal((n, d)) * 0.9
    k = rng.standard_normal((n, d)) * 0.9
    v = rng.standard_normal((n, d))
    R = oracle.projections(5, d, r)
    rq = oracle.ranks(q.astype(np.float32), R)
    rk = oracle.ranks(k.astype(np.float32), R)
    parts = {}
    out, lse = hyperattn.noncausal_problem(q.astype(np.float32).astype(np.float64),
                                           k.astype(np.float32).astype(np.float64),
                                           v.astype(np.float32).astype(np.float64),
                                           rq, rk, 5, 0, 2, 1, block, m, parts=parts)
    qf, kf, vf = (a.astype(np.float32).astype(np.float64) for a in (q, k, v))
    D_blk, D_smp, o_ref, pq = _brute_force_problem(qf, kf, vf, rq, rk, parts["idx"], block)
    # oracle parts are in sorted order; brute force in original order
    inv = np.empty(n, dtype=np.int64)
    inv[np.array(pq)] = np.arange(n)
    assert np.allclose(np.exp(parts["lse_blk"][inv]), D_blk, rtol=1e-12, atol=0)
    got_smp = np.exp(parts["lse_smp"][inv])
    assert np.allclose(got_smp, D_smp, rtol=1e-12, atol=1e-300)
    assert np.allclose(np.exp(lse), D_blk + D_smp, rtol=1e-12, atol=0)
    assert np.max(np.abs(out - o_ref)) < 1e-12


@pytest.mark.parametrize("n,block", [(32, 8), (48, 16), (40, 40)])
def test_sample_estimate_is_unbiased(n, block):
    rng = np.random.default_rng(n * block)
    d = 8
    Qs = rng.standard_normal((n, d)) * 0.8
    Ks = rng.standard_normal((n, d)) * 0.8
    Vs = rng.standard_normal((n, d))
    A = np.exp(Qs @ Ks.T)
    b_eff = min(block, n)
    out_mass = np.zeros(n)
    out_num = np.zeros((n, d))
    for p in range(n):
        for j in range(n):
            if j // b_eff != p // b_eff:
                out_mass[p] += A[p, j]
                out_num[p] += A[p, j] * Vs[j]
    acc_D = np.zeros(n)
    acc_N = np.zeros((n, d))
    for j in range(n):                     # one sample at each position in turn
        l, o = hyperattn.sample_part(Qs, Ks, Vs, np.array([j]), b_eff)
        D = np.exp(l)
        acc_D += D
        acc_N += o * D[:, None]
    assert np.allclose(acc_D / n, out_mass, rtol=1e-12, atol=0)
    assert np.allclose(acc_N / n, out_num, rtol=1e-12, atol=1e-14)
    lb, _ = hyperattn.block_part(Qs, Ks, Vs, b_eff)
    assert np.allclose(np.exp(lb) + acc_D / n, A.sum(1), rtol=1e-12)


def test_mass_invariant_and_merge_closed_form():
    rng = np.random.default_rng(5)
    n, d = 256, 16
    q, k, v = (rng.standard_normal((n, d)) * 0.7 for _ in range(3))
    R = oracle.projections(1, d, 6)
    parts = {}
    out, lse = hyperattn.noncausal_problem(q, k, v, oracle.ranks(q.astype(np.float32), R),
                                           oracle.ranks(k.astype(np.float32), R), 1, 0, 0, 1,
                                           32, 64, parts=parts)
    lb, ob, ls, osm = parts["lse_blk"], parts["o_blk"], parts["lse_smp"], parts["o_smp"]
    pq = parts["perm_q"]
    assert np.allclose(np.exp(lse[pq]), np.exp(lb) + np.exp(ls), rtol=1e-12)
    Db, Ds = np.exp(lb), np.exp(ls)
    direct = (ob * Db[:, None] + osm * Ds[:, None]) / (Db + Ds)[:, None]
    assert np.max(np.abs(out[pq] - direct)) < 1e-12
    # -inf part: merge returns the other part unchanged
    l, o = hyperattn.lse_merge(lb, ob, np.full(n, -np.inf), np.zeros_like(ob))
    assert np.array_equal(l, lb) and np.max(np.abs(o - ob)) == 0


def test_rows_subset_matches_full():
    rng = np.random.default_rng(9)
    q, k, v = _rand_qkv(rng, 1, 4, 2, 256, 16)
    for cfg in (HAConfig(block=32, samples=20, proj_bits=5, seed=4),
                HAConfig(block=16, samples=24, proj_bits=6, causal=True, min_seq_len=32, seed=4)):
        full, full_lse = oracle.forward(q, k, v, cfg)
        rows = np.array([0, 5, 31, 32, 100, 129, 200, 255])
        sub, sub_lse = oracle.forward_rows(q, k, v, cfg, heads=[(0, 1), (0, 3)], rows=rows)
        assert np.max(np.abs(sub[0] - full[0, 1][rows])) < 1e-12
        assert np.max(np.abs(sub[1] - full[0, 3][rows])) < 1e-12
        assert np.max(np.abs(sub_lse[1] - full_lse[0, 3][rows])) < 1e-12


def test_causal_recursion_structure():
    # one level (n = 2 s): rows < s are pure leaf attention; rows >= s merge
    # the second leaf with the quadrant (queries [s, n), keys [0, s)).
    rng = np.random.default_rng(21)
    n, s, d = 64, 32, 8
    q, k, v = _rand_qkv(rng, 1, 1, 1, n, d)
    cfg = HAConfig(block=8, samples=6, proj_bits=3, causal=True, min_seq_len=s, seed=2)
    out, lse = oracle.forward(q, k, v, cfg)
    qd, kd, vd = (a[0, 0].astype(np.float64) for a in (q, k, v))
    lower = _textbook(q[:, :, :s], k[:, :, :s], v[:, :, :s], True)[0, 0]
    assert np.max(np.abs(out[0, 0, :s] - lower)) < 1e-12
    R = oracle.projections(2, d, 3)
    rq = oracle.ranks(q[0, 0], R)
    rk = oracle.ranks(k[0, 0], R)
    oq, lq = hyperattn.noncausal_problem(qd[s:], kd[:s], vd[:s], rq[s:], rk[:s], 2, 0, 0, 1, 8, 6)
    S = qd[s:] @ kd[s:].T
    S = np.where(np.tril(np.ones((s, s), bool)), S, -np.inf)
    leaf_l = np.log(np.exp(S).sum(1))
    leaf_o = softmax(S, axis=1) @ vd[s:]
    D = np.exp(leaf_l) + np.exp(lq)
    expect = (leaf_o * np.exp(leaf_l)[:, None] + oq * np.exp(lq)[:, None]) / D[:, None]
    assert np.max(np.abs(out[0, 0, s:] - expect)) < 1e-12
    assert np.max(np.abs(lse[0, 0, s:] - np.log(D))) < 1e-12
    assert oracle.causal_levels(131072, 4096) == 5 and oracle.causal_levels(4096, 4096) == 0


def test_argument_errors():
    rng = np.random.default_rng(0)
    q, k, v = _rand_qkv(rng, 1, 3, 2, 64, 8)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, HAConfig(block=8, samples=1, proj_bits=3))
    q, k, v = _rand_qkv(rng, 1, 2, 1, 60, 8)
    oracle.forward(q, k, v, HAConfig(block=8, samples=1, proj_bits=3))       # ragged last block: valid
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, HAConfig(block=4, samples=1, proj_bits=17))
    q, k, v = _rand_qkv(rng, 1, 2, 1, 48, 8)
    # 48 -> 24 -> 12 -> 6 -> 3 -> (1, 2): odd splits are valid (R19)
    oracle.forward(q, k, v, HAConfig(block=3, samples=1, proj_bits=3, causal=True, min_seq_len=2))


def test_empty_sequence():
    q = np.zeros((1, 2, 0, 8), np.float32)
    k = np.zeros((1, 1, 0, 8), np.float32)
    out, lse = oracle.forward(q, k, k, HAConfig(block=8, samples=4, proj_bits=3))
    assert out.shape == (1, 2, 0, 8) and lse.shape == (1, 2, 0)


# ----------------------------------------------------------------------------
# Planted mistakes: each plausible bug in the oracle must trip a pin above.
# ----------------------------------------------------------------------------

def _bruteforce_error():
    rng = np.random.default_rng(77)
    n, d, block, m, r = 64, 8, 8, 24, 4
    q = rng.standard_normal((n, d)) * 0.9
    k = rng.standard_normal((n, d)) * 0.9
    v = rng.standard_normal((n, d))
    R = oracle.projections(5, d, r)
    rq = oracle.ranks(q.astype(np.float32), R)
    rk = oracle.ranks(k.astype(np.float32), R)
    parts = {}
    out, _ = hyperattn.noncausal_problem(q, k, v, rq, rk, 5, 0, 2, 1, block, m, parts=parts)
    _, _, o_ref, _ = _brute_force_problem(q, k, v, rq, rk, parts["idx"], block)
    return np.max(np.abs(out - o_ref))


def _wrong_sample_part(Qs, Ks, Vs, idx, b_eff, positions=None, b_k=None):  # (almost) no in-block exclusion
    return _orig_sample_part(Qs, Ks, Vs, idx, 1, positions, 1 << 40)


def _wrong_weight_sample_part(Qs, Ks, Vs, idx, b_eff, positions=None, b_k=None):  # weight 1 instead of ns/m
    l, o = _orig_sample_part(Qs, Ks, Vs, idx, b_eff, positions, b_k)
    return l - np.log(Qs.shape[0] / len(idx)), o


def _wrong_sort(rank):                                   # ties in reverse index order
    rank = np.asarray(rank)
    return np.lexsort((-np.arange(len(rank)), rank))


_orig_sample_part = hyperattn.sample_part


@pytest.mark.parametrize("mutant", ["no_exclusion", "no_weight", "sort_order", "transposed_kv"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    assert _bruteforce_error() < 1e-12
    if mutant == "no_exclusion":
        monkeypatch.setattr(hyperattn, "sample_part", _wrong_sample_part)
    elif mutant == "no_weight":
        monkeypatch.setattr(hyperattn, "sample_part", _wrong_weight_sample_part)
    elif mutant == "sort_order":
        monkeypatch.setattr(hyperattn, "sort_perm", _wrong_sort)
    elif mutant == "transposed_kv":
        orig = hyperattn.block_part
        monkeypatch.setattr(hyperattn, "block_part",
                            lambda Qs, Ks, Vs, b, positions=None, b_k=None: orig(Qs, Vs, Ks, b, positions, b_k))
    assert _bruteforce_error() > 1e-6


def test_planted_gray_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(hyperattn, "gray_inverse", lambda code, r: np.asarray(code, np.uint32))
    codes = np.arange(1 << 6, dtype=np.uint32)
    rank = hyperattn.gray_inverse(codes, 6)
    order = codes[np.argsort(rank)]
    diff = order[1:] ^ order[:-1]
    assert not np.all((diff & (diff - 1)) == 0)


@pytest.mark.parametrize("n,s,block,m,H,Hkv", [(256, 32, 12, 8, 2, 1), (300, 40, 16, 5, 1, 1), (128, 200, 8, 4, 1, 1)])
def test_causal_parts_rebuild_the_forward(n, s, block, m, H, Hkv):
    """causal_parts lists every leaf and quadrant of the recursion with its
    intermediates: leaves partition the rows, the quadrants of one depth
    have disjoint query and key ranges with node ids in [2^depth,
    2^(depth+1)), and the total mass of a row -- leaf plus the block and
    sample parts of every quadrant holding it, as plain sums e^lse -- with
    the matching weighted outputs gives the forward's output and lse."""
    rng = np.random.default_rng(n + s)
    d = 16
    q, k, v = _rand_qkv(rng, 1, H, Hkv, n, d)
    cfg = HAConfig(block=block, samples=m, proj_bits=5, causal=True, min_seq_len=s, seed=9)
    out, lse = oracle.forward(q, k, v, cfg)
    R = oracle.projections(9, d, 5)
    for h in range(H):
        g = h // (H // Hkv)
        qd, kd, vd = q[0, h].astype(np.float64), k[0, g].astype(np.float64), v[0, g].astype(np.float64)
        leaves, quads = hyperattn.causal_parts(qd, kd, vd, oracle.ranks(q[0, h], R), oracle.ranks(k[0, g], R),
                                               9, 0, h, cfg)
        covered = np.concatenate([np.arange(lf["lo"], lf["hi"]) for lf in leaves])
        assert np.array_equal(np.sort(covered), np.arange(n))
        depths = [qd_["depth"] for qd_ in quads]
        assert (max(depths) + 1 if quads else 0) == oracle.causal_levels(n, s)
        for dep in set(depths):
            at = [x for x in quads if x["depth"] == dep]
            qr = np.concatenate([np.arange(x["mid"], x["hi"]) for x in at])
            kr = np.concatenate([np.arange(x["lo"], x["mid"]) for x in at])
            assert len(np.unique(qr)) == len(qr) and len(np.unique(kr)) == len(kr)
            assert all(2 ** dep <= x["node"] < 2 ** (dep + 1) for x in at)
        D = np.zeros(n)
        N = np.zeros((n, d))
        for lf in leaves:
            w = np.exp(lf["lse"])
            D[lf["lo"]:lf["hi"]] += w
            N[lf["lo"]:lf["hi"]] += w[:, None] * lf["o"]
        for x in quads:
            rows = x["mid"] + x["perm_q"]                 # sorted position -> row
            assert np.array_equal(np.sort(x["perm_k"]), np.arange(x["mid"] - x["lo"]))
            for lk, ok in (("lse_blk", "o_blk"), ("lse_smp", "o_smp")):
                w = np.exp(x[lk])
                D[rows] += w
                N[rows] += w[:, None] * x[ok]
        assert np.max(np.abs(N / D[:, None] - out[0, h])) < 1e-12
        assert np.max(np.abs(np.log(D) - lse[0, h])) < 1e-12
