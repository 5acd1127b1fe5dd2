"""The method's fine-grained parameters as diagnostics (CPU, fp64).  Test
infrastructure only (see the package docstring).

[S] "Approach": the guarantee rests on two parameters instead of bounded
entries -- the largest column norm of the normalised attention matrix
D^-1 A, and the ratio of row norms of the unnormalised matrix after the
large entries are detected and removed.  [S] "Limitations": alpha is the
largest squared column norm of the softmax matrix, assumed n^{o(1)} and
checked only empirically.  [S] "Surprising findings": for chatglm2 the
first columns of D^-1 A hold heavy entries, so alpha was taken without
the first 32 columns.

Readings:

* R16: alpha = max_{j >= skip} sum_i P_ij^2 with P = D^-1 A of exact
  attention (A = exp(Q K^T), causal calls masked to j <= i); skip = 32 for
  the chatglm2-like inputs.
* R17: kappa = max_i r_i / min_i r_i with r_i = sum_{j outside row i's
  block} A_ij, the row sums (1-norms, A >= 0) of A after the entries the
  sortLSH blocks find are removed (non-causal problems; a row with r_i = 0
  makes kappa infinite).
"""

import numpy as np

from .hyperattn import sort_perm


def _probabilities(q, k, causal):
    S = np.asarray(q, np.float64) @ np.asarray(k, np.float64).T
    if causal:
        n = S.shape[0]
        S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    S = S - np.max(S, axis=1, keepdims=True)
    E = np.exp(S)
    return E / E.sum(axis=1, keepdims=True)


def column_sqmass(q, k, causal=False):
    """c_j = sum_i P_ij^2 for one head (q, k: [n, d])."""
    P = _probabilities(q, k, causal)
    return np.sum(P * P, axis=0)


def alpha(q, k, causal=False, skip=0):
    """alpha = max_{j >= skip} c_j (R16)."""
    return float(np.max(column_sqmass(q, k, causal)[skip:]))


def residual_row_sums(q, k, rank_q, rank_k, block):
    """r_i = sum of A_ij over keys j outside row i's block of the sorted
    matrix (blocks of b_eff = min(block, n) sorted positions), original
    row order."""
    n = q.shape[0]
    b_eff = min(block, n)
    pq, pk = sort_perm(rank_q), sort_perm(rank_k)
    blk_q = np.empty(n, dtype=np.int64)
    blk_q[pq] = np.arange(n) // b_eff
    blk_k = np.empty(n, dtype=np.int64)
    blk_k[pk] = np.arange(n) // b_eff
    A = np.exp(np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    outside = blk_q[:, None] != blk_k[None, :]
    return np.sum(A * outside, axis=1)


def kappa(q, k, rank_q, rank_k, block):
    """kappa = max_i r_i / min_i r_i (R17); inf if some r_i = 0."""
    r = residual_row_sums(q, k, rank_q, rank_k, block)
    mn = float(np.min(r))
    return float(np.max(r)) / mn if mn > 0 else float("inf")


def column_sqmass_cols(q, k, cols, causal=False, chunk=2048):
    """c_j = sum_i P_ij^2 for the listed columns j only, the row
    normalisers taken chunk by chunk of rows, so that an n of tens of
    thousands needs no n x n matrix (q, k: [n, d])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    cols = np.asarray(cols, dtype=np.int64)
    n = q.shape[0]
    out = np.zeros(len(cols))
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        S = q[r0:r1] @ k.T
        if causal:
            S = np.where(np.arange(r0, r1)[:, None] >= np.arange(n)[None, :], S, -np.inf)
        mx = np.max(S, axis=1, keepdims=True)
        lse = mx + np.log(np.sum(np.exp(S - mx), axis=1, keepdims=True))
        out += np.sum(np.exp(2.0 * (S[:, cols] - lse)), axis=0)
    return out
