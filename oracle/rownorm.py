"""Row-norm-sampling variant of the product with V (CPU, fp64 except where
a precision is fixed).  Test infrastructure only (see the package
docstring).

[S] "Approach" estimates the normaliser D from exact block row sums plus
uniform column samples, and names row-norm sampling for the product with
V; "Builds on" lists approximate matrix multiplication via row norm
sampling.  The pages print no formula.  Reading R15 (the plainest
approximate-matrix-multiplication reading that the rest supports):

* D is unchanged: exact block row sums + uniform samples of weight ns/m.
* The numerator N_i = sum_j A_ij v_j is the exact block part plus an
  estimate of the residual product (keys outside row i's block) from m
  key positions drawn iid with p_t proportional to ||v_t||^2 over the
  problem's sorted keys; a kept draw t contributes A_it v_t / (m p_t), a
  draw inside the row's block contributes nothing; duplicates count each
  time.
* out_i = (N_blk + N_rn) / (D_blk + D_unif), lse_i = ln(D_blk + D_unif).
* Causal (reading R20): the leaves stay exact; every quadrant of the
  recursion (queries [mid, hi), keys [lo, mid), node id `node`) is such a
  problem with that node's draws -- the largest weight, the CDF and the
  Philox counters (i // 4, node, head, 2 batch + 2) all over the node's
  keys -- and its (out, lse) merges with the rest of the row by the usual
  log-sum-exp merge, so a row's result is
  (N_leaf + sum over its quadrants of (N_blk + N_rn)) /
  (D_leaf + sum over its quadrants of (D_blk + D_unif)).  A rectangular
  quadrant (odd span) takes the key blocks of reading R18 for both the
  uniform and the row-norm exclusions.

Exact probabilities, so that the draws are reproducible bit for bit:
w_t = ||v_t||^2 in fp32 (each square rounded, groups of 8 consecutive
squares summed by halving, group sums by halving);
with max_t w_t = f 2^e (f in [0.5, 1)), n_t = floor(w_t 2^(40 - e)), an
integer below 2^40 (keys whose weight is below 2^-40 of the largest get
n_t = 0 and are never drawn); c_t = n_0 + ... + n_t in exact integers,
T = c_last; draw i takes word x_i of the Philox stream with counters
(i // 4, node, head, 2 * batch + 2) -- even last word, so it meets neither
the projections (0) nor the uniform samples (odd) -- sets
r = floor(x_i T / 2^32) and picks the smallest t with c_t > r.  Then
p_t = n_t / T exactly and the weight of a draw is T / (m n_t).  T = 0 (all
value rows zero) means no draws.
"""

from fractions import Fraction

import numpy as np

from .hyperattn import (block_part, causal_problem, key_block, sample_part, sample_positions, sort_perm, _check,
                        ranks)
from .gauss import projections
from .philox import philox_words

QBITS = 40


def _padded_dim(d):
    """Smallest 8 * 2^k >= d."""
    g = 1
    while 8 * g < d:
        g *= 2
    return 8 * g


def _halving_sum_last(v):
    """Sum over the last axis by repeated halving: v <- v[:h] + v[h:]."""
    while v.shape[-1] > 1:
        h = v.shape[-1] // 2
        v = v[..., :h] + v[..., h:]
    return v[..., 0]


def row_norms_sq(v32):
    """w_t = ||v_t||^2 in fp32 with the fixed order above."""
    v32 = np.asarray(v32, dtype=np.float32)
    rows, d = v32.shape
    dp = _padded_dim(d)
    vp = np.zeros((rows, dp), dtype=np.float32)
    vp[:, :d] = v32
    sq = vp * vp                                            # fp32 squares
    groups = _halving_sum_last(sq.reshape(rows, dp // 8, 8))
    return _halving_sum_last(groups).astype(np.float32)


def quantized_weights(w32):
    """n_t = floor(w_t 2^(40 - e)) as Python-exact int64, e from max w."""
    w = np.asarray(w32, dtype=np.float64)
    mx = float(np.max(w)) if w.size else 0.0
    if not mx > 0.0:
        return np.zeros(w.shape, dtype=np.int64)
    _, e = np.frexp(mx)                                     # mx = f 2^e, f in [0.5, 1)
    return np.floor(np.ldexp(w, QBITS - int(e))).astype(np.int64)


def rownorm_positions(seed, batch_idx, head, node, n_sorted, m):
    """m sorted key positions drawn with p_t = n_t / T (n_sorted: n_t in
    sorted key order).  Returns (positions int64 [m], T)."""
    n_sorted = np.asarray(n_sorted, dtype=np.int64)
    T = int(n_sorted.sum())
    if m == 0 or T == 0:
        return np.zeros(0, dtype=np.int64), T
    c = np.cumsum(n_sorted)                                 # exact: T < 2^57
    x = philox_words(seed, m, c1=node, c2=head, c3=2 * batch_idx + 2)
    pos = np.empty(m, dtype=np.int64)
    for i in range(m):
        r = (int(x[i]) * T) >> 32
        pos[i] = int(np.searchsorted(c, r, side="right"))   # smallest t with c_t > r
    return pos, T


def rownorm_part(Qs, Ks, Vs, idx, n_sorted, T, b_eff, positions=None, b_k=None):
    """Residual numerator estimate as (lse_r, o_r):
    e^{lse_r} = sum_{kept s} A_{p, idx_s} T / (m n_{idx_s}) and
    o_r e^{lse_r} = sum_{kept s} A_{p, idx_s} T / (m n_{idx_s}) v_{idx_s};
    draw s is kept unless idx_s // b_k == p // b_eff (b_k = b_eff for
    square problems)."""
    ns, d = Qs.shape
    b_k = b_eff if b_k is None else b_k
    if positions is None:
        positions = np.arange(ns)
    positions = np.asarray(positions, dtype=np.int64)
    m = len(idx)
    if m == 0:
        return np.full(len(positions), -np.inf), np.zeros((len(positions), d))
    idx = np.asarray(idx, dtype=np.int64)
    n_s = np.asarray(n_sorted, dtype=np.int64)[idx]
    logw = np.log(float(T)) - np.log(float(m)) - np.log(n_s.astype(np.float64))
    Ksm, Vsm = Ks[idx], Vs[idx]
    col_blk = idx // b_k
    lse = np.empty(len(positions))
    o = np.empty((len(positions), d))
    for c in range(0, len(positions), 4096):
        p = positions[c:c + 4096]
        S = Qs[p] @ Ksm.T + logw[None, :]
        keep = (p // b_eff)[:, None] != col_blk[None, :]
        S = np.where(keep, S, -np.inf)
        mx = np.max(S, axis=1, keepdims=True)
        ok = np.isfinite(mx)
        E = np.where(np.isfinite(S), np.exp(S - np.where(ok, mx, 0.0)), 0.0)
        ssum = E.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            oo = (E @ Vsm) / ssum[:, None]
            ll = np.where(ok[:, 0], mx[:, 0], 0.0) + np.log(ssum)
        o[c:c + 4096] = np.where((ssum > 0)[:, None], oo, 0.0)
        lse[c:c + 4096] = np.where(ssum > 0, ll, -np.inf)
    return lse, o


def merge_variant(lb, ob, lu, lr, orr):
    """out = (ob e^lb + orr e^lr) / (e^lb + e^lu), lse = ln(e^lb + e^lu)."""
    lse = np.logaddexp(lb, lu)
    with np.errstate(invalid="ignore"):
        wb = np.where(np.isfinite(lb), np.exp(lb - lse), 0.0)
        wr = np.where(np.isfinite(lr), np.exp(lr - lse), 0.0)
    return lse, ob * wb[..., None] + orr * wr[..., None]


def noncausal_problem_rownorm(q, k, v, rank_q, rank_k, v32, seed, batch_idx, head, node, block,
                              samples, rows=None, parts=None):
    """One non-causal problem of ns queries and n_k keys with the row-norm
    product (reading R15; n_k != ns for a rectangular causal quadrant,
    reading R18).  v32: the value rows as fp32 (for the exact weights).
    Returns (o, lse) in original row order (``rows``: local indices, all
    if None)."""
    ns, d = q.shape
    n_k = k.shape[0]
    if ns == 0:
        return np.zeros((0, d)), np.zeros(0)
    if n_k == 0:
        raise ValueError("a problem with queries needs keys")
    b_eff = min(block, ns)
    if b_eff < 1:
        raise ValueError("block must be >= 1")
    b_k = key_block(b_eff, ns, n_k)
    pq = sort_perm(rank_q)
    pk = sort_perm(rank_k)
    Qs, Ks, Vs = q[pq], k[pk], v[pk]
    n_sorted = quantized_weights(row_norms_sq(v32))[pk]
    idx_u = sample_positions(seed, batch_idx, head, node, n_k, samples)
    idx_r, T = rownorm_positions(seed, batch_idx, head, node, n_sorted, samples)
    if rows is None:
        positions = None
    else:
        inv = np.empty(ns, dtype=np.int64)
        inv[pq] = np.arange(ns)
        positions = inv[np.asarray(rows, dtype=np.int64)]
    lb, ob = block_part(Qs, Ks, Vs, b_eff, positions, b_k)
    lu, _ = sample_part(Qs, Ks, Vs, idx_u, b_eff, positions, b_k)
    lr, orr = rownorm_part(Qs, Ks, Vs, idx_r, n_sorted, T, b_eff, positions, b_k)
    lse, o = merge_variant(lb, ob, lu, lr, orr)
    if parts is not None:
        parts.update(perm_q=pq, perm_k=pk, idx_u=idx_u, idx_r=idx_r, n_sorted=n_sorted, T=T,
                     lse_blk=lb, o_blk=ob, lse_u=lu, lse_r=lr, o_r=orr)
    if rows is None:
        out = np.empty_like(o)
        out[pq] = o
        lse_out = np.empty_like(lse)
        lse_out[pq] = lse
        return out, lse_out
    return o, lse


def causal_problem_rownorm(q, k, v, rank_q, rank_k, v32, seed, batch_idx, head, cfg, rows=None):
    """Causal forward of one head with the row-norm product in every
    quadrant (reading R20): the recursion of ``causal_problem`` with each
    node's quadrant solved by ``noncausal_problem_rownorm`` under that
    node's id.  q, k, v fp64 [n, d]; v32 the value rows as fp32."""
    def quadrant(lo, mid, hi, node, local_rows):
        return noncausal_problem_rownorm(q[mid:hi], k[lo:mid], v[lo:mid], rank_q[mid:hi], rank_k[lo:mid],
                                         v32[lo:mid], seed, batch_idx, head, node, cfg.block, cfg.samples,
                                         rows=local_rows)
    return causal_problem(q, k, v, rank_q, rank_k, seed, batch_idx, head, cfg, rows=rows, quadrant=quadrant)


def forward_rows(q, k, v, cfg, heads=None, rows=None):
    """Forward with the row-norm product for the listed (batch, head) pairs
    and rows; arguments as ``oracle.hyperattn.forward_rows``."""
    B, H, Hkv, n, d = _check(q, k, v, cfg)
    G = H // Hkv
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    if rows is not None:
        rows = np.sort(np.asarray(rows, dtype=np.int64))
    nr = n if rows is None else len(rows)
    R = projections(cfg.seed, d, cfg.proj_bits)
    out = np.zeros((len(heads), nr, d))
    lse = np.zeros((len(heads), nr))
    for i, (b, h) in enumerate(heads):
        g = h // G
        rq, rk = ranks(q[b, h], R), ranks(k[b, g], R)
        q64, k64, v64 = q[b, h].astype(np.float64), k[b, g].astype(np.float64), v[b, g].astype(np.float64)
        if cfg.causal:
            o, l = causal_problem_rownorm(q64, k64, v64, rq, rk, v[b, g], cfg.seed, b, h, cfg, rows=rows)
        else:
            o, l = noncausal_problem_rownorm(q64, k64, v64, rq, rk, v[b, g], cfg.seed, b, h, 1,
                                             cfg.block, cfg.samples, rows=rows)
        out[i] = o
        lse[i] = l
    return out, lse


def forward(q, k, v, cfg):
    """Full forward with the row-norm product:
    (out [B, H, n, d], lse [B, H, n]) in fp64."""
    B, H, n, d = q.shape
    out, lse = forward_rows(q, k, v, cfg)
    return out.reshape(B, H, n, d), lse.reshape(B, H, n)


def exact_probability(n_sorted, t):
    """p_t = n_t / T as an exact fraction (for the tests)."""
    n_sorted = [int(x) for x in n_sorted]
    return Fraction(n_sorted[t], sum(n_sorted))
