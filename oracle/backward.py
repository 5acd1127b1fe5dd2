"""Backward pass of the HyperAttention forward (dQ, dK, dV) on the CPU in fp64.

Test infrastructure only (see the package docstring).

Reading (the pages print no backward formulas; [S] "Key results" times the
method forward and backward): hashing, sorting and sampling do
not depend continuously on the inputs, so for fixed ranks and samples the
forward of ``oracle.hyperattn`` is, row by row, a softmax over key rows with
fixed multiplicities W_ij:

    O_i = sum_j W_ij e^{s_ij} v_j / sum_j W_ij e^{s_ij},   s_ij = q_i . k_j,

where, for one non-causal problem, W_ij = [j is in row i's block] + (ns/m)
times the number of kept samples at j's sorted position (kept: outside row
i's block); for the causal recursion W is the sum of the exact leaves'
lower triangles and every level's quadrant weights -- the log-sum-exp merge
of the parts is exactly the joint weighted softmax.  For an upstream dO its
gradient is the weighted-softmax backward:

    P = W o exp(S - lse),  dV = P^T dO,  dP = dO V^T,
    D_i = sum_j P_ij dP_ij = dO_i . O_i,  dS = P o (dP - D),
    dQ = dS K,  dK = dS^T Q,

with dK and dV of a KV head summed over its query heads (grouped heads).
The weights are built here from the same ranks, permutations and samples as
the forward; the tests pin them against the step-by-step forward and the
gradients against finite differences of it and, for W = 1, against autograd.
"""

import numpy as np

from .gauss import projections
from .hyperattn import (_check, causal_levels, key_block, ranks, sample_positions, sort_perm)


def noncausal_weights(rank_q, rank_k, seed, batch_idx, head, node, block, samples):
    """W [n_q, n_k] (rows: queries, columns: keys, both in original local
    order) of one non-causal problem: 1 inside the row's diagonal block of
    the sorted matrix (query blocks of b, key blocks of b_k, reading R18),
    plus n_k/m per sample at the key's sorted position when that position
    lies outside the row's block."""
    ns, n_k = len(rank_q), len(rank_k)
    if ns == 0 or n_k == 0:
        return np.zeros((ns, n_k))
    b_eff = min(block, ns)
    b_k = key_block(b_eff, ns, n_k)
    pq = sort_perm(rank_q)
    pk = sort_perm(rank_k)
    spos_q = np.empty(ns, dtype=np.int64)
    spos_q[pq] = np.arange(ns)                      # sorted position of each query row
    spos_k = np.empty(n_k, dtype=np.int64)
    spos_k[pk] = np.arange(n_k)
    blk_q = spos_q // b_eff
    blk_k = spos_k // b_k
    same = blk_q[:, None] == blk_k[None, :]
    W = same.astype(np.float64)
    if samples > 0:
        idx = sample_positions(seed, batch_idx, head, node, n_k, samples)
        count = np.bincount(idx, minlength=n_k)[spos_k]   # samples on each key row
        W += np.where(same, 0.0, (n_k / samples) * count[None, :])
    return W


def causal_weights(rank_q, rank_k, seed, batch_idx, head, cfg):
    """W [n, n] of the causal recursion: every leaf of length <= min_seq_len
    contributes its causal lower triangle (weight 1), every split
    [lo, mid, hi) with node id contributes the non-causal weights of queries
    [mid, hi) over keys [lo, mid)."""
    n = len(rank_q)
    causal_levels(n, cfg.min_seq_len)
    W = np.zeros((n, n))

    def rec(lo, hi, node):
        ns = hi - lo
        if ns <= cfg.min_seq_len:
            W[lo:hi, lo:hi] += np.tril(np.ones((ns, ns)))
            return
        mid = lo + ns // 2
        rec(lo, mid, 2 * node)
        rec(mid, hi, 2 * node + 1)
        W[mid:hi, lo:mid] += noncausal_weights(rank_q[mid:hi], rank_k[lo:mid], seed, batch_idx,
                                               head, node, cfg.block, cfg.samples)

    rec(0, n, 1)
    return W


def weighted_attention(q, k, v, W):
    """(O, lse) of the weighted softmax sum_j W_ij e^{q_i.k_j} v_j / (its row
    sum); rows with no positive weight give O = 0, lse = -inf."""
    S = q @ k.T
    with np.errstate(divide="ignore"):
        logits = np.where(W > 0, S + np.log(np.where(W > 0, W, 1.0)), -np.inf)
    mx = np.max(logits, axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    E = np.exp(logits - mx)
    den = E.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(den > 0, (E @ v) / np.where(den > 0, den, 1.0), 0.0)
        lse = np.where(den[:, 0] > 0, np.log(np.where(den[:, 0] > 0, den[:, 0], 1.0)) + mx[:, 0], -np.inf)
    return O, lse


def round_bf16(x):
    """x (fp64 array, normal range) rounded to the nearest bfloat16 value,
    ties to even: 8 significant bits (frexp gives x = m 2^e, m in [0.5, 1))."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def weighted_backward(q, k, v, W, do, out_round=None):
    """(dq, dk, dv) of sum(do * O) for O = weighted_attention(q, k, v, W).

    out_round: None, or a rounding applied to O before D = rowsum(do * O)
    (reading R14b: a backward handed the forward's output in the input
    dtype forms D from that output; ``round_bf16`` models a bf16 one)."""
    O, lse = weighted_attention(q, k, v, W)
    S = q @ k.T
    with np.errstate(invalid="ignore", over="ignore"):
        P = np.where(W > 0, W * np.exp(S - np.where(np.isfinite(lse), lse, 0.0)[:, None]), 0.0)
    dv = P.T @ do
    dP = do @ v.T
    D = np.sum(do * (O if out_round is None else out_round(O)), axis=1)
    dS = P * (dP - D[:, None])
    dq = dS @ k
    dk = dS.T @ q
    return dq, dk, dv


def head_weights(q32, k32, cfg, b, h, G, R):
    """W of query head h of batch entry b (KV head h // G)."""
    rq = ranks(q32[b, h], R)
    rk = ranks(k32[b, h // G], R)
    if cfg.causal:
        return causal_weights(rq, rk, cfg.seed, b, h, cfg)
    return noncausal_weights(rq, rk, cfg.seed, b, h, 1, cfg.block, cfg.samples)


def backward(q, k, v, do, cfg):
    """Full backward: (dq [B, H, n, d], dk, dv [B, Hkv, n, d]) in fp64 for
    the forward of ``oracle.hyperattn.forward`` with config ``cfg``.

    q, k, v: float32 arrays holding the input values exactly (bf16 widened);
    do: the upstream gradient of the output (any float array)."""
    B, H, Hkv, n, d = _check(q, k, v, cfg)
    G = H // Hkv
    R = projections(cfg.seed, d, cfg.proj_bits)
    dq = np.zeros((B, H, n, d))
    dk = np.zeros((B, Hkv, n, d))
    dv = np.zeros((B, Hkv, n, d))
    for b in range(B):
        for h in range(H):
            W = head_weights(q, k, cfg, b, h, G, R)
            g = h // G
            gq, gk, gv = weighted_backward(q[b, h].astype(np.float64), k[b, g].astype(np.float64),
                                           v[b, g].astype(np.float64), W, np.asarray(do[b, h], np.float64))
            dq[b, h] = gq
            dk[b, g] += gk
            dv[b, g] += gv
    return dq, dk, dv


def backward_rect(q, k, v, do, cfg):
    """Backward of ``oracle.hyperattn.forward_rect`` (reading R18): q, do
    [B, H, n_q, d], k, v [B, Hkv, n_k, d] float32 arrays holding the input
    values exactly.  Returns (dq [B, H, n_q, d], dk, dv [B, Hkv, n_k, d]) in
    fp64; W is the rectangular problem's weights (noncausal_weights with
    n_q queries and n_k keys)."""
    if cfg.causal:
        raise ValueError("rectangular problems are non-causal")
    B, H, n_q, d = q.shape
    Hkv, n_k = k.shape[1], k.shape[2]
    G = H // Hkv
    R = projections(cfg.seed, d, cfg.proj_bits)
    dq = np.zeros((B, H, n_q, d))
    dk = np.zeros((B, Hkv, n_k, d))
    dv = np.zeros((B, Hkv, n_k, d))
    for b in range(B):
        for h in range(H):
            g = h // G
            W = noncausal_weights(ranks(q[b, h], R), ranks(k[b, g], R), cfg.seed, b, h, 1, cfg.block,
                                  cfg.samples)
            gq, gk, gv = weighted_backward(q[b, h].astype(np.float64), k[b, g].astype(np.float64),
                                           v[b, g].astype(np.float64), W, np.asarray(do[b, h], np.float64))
            dq[b, h] = gq
            dk[b, g] += gk
            dv[b, g] += gv
    return dq, dk, dv


def noncausal_backward_blocks(q, k, v, do, rank_q, rank_k, seed, batch_idx, head, node, block, samples):
    """(dq, dk, dv) of one square non-causal problem, query block by query
    block: the same W as ``noncausal_weights`` (block keys at weight 1,
    kept samples at n/m per draw), but only the non-zero columns of each
    block's rows are formed, so a 131072-row head takes seconds instead of
    an n x n matrix.  q, do [n, d], k, v [n, d] fp64; the weighted-softmax
    backward of the module docstring is applied to each block's rows."""
    n, d = q.shape
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    if n == 0:
        return dq, dk, dv
    b_eff = min(block, n)
    b_k = key_block(b_eff, n, n)
    pq = sort_perm(rank_q)
    pk = sort_perm(rank_k)
    if samples > 0:
        idx = sample_positions(seed, batch_idx, head, node, n, samples)
        pos, count = np.unique(idx, return_counts=True)  # sampled sorted key positions, draws at each
    else:
        pos = count = np.zeros(0, dtype=np.int64)
    for t in range((n + b_eff - 1) // b_eff):
        qrows = pq[t * b_eff:min((t + 1) * b_eff, n)]
        bpos = np.arange(min(t * b_k, n), min((t + 1) * b_k, n))
        kept = (pos // b_k) != t
        kpos = np.concatenate([bpos, pos[kept]])
        wts = np.concatenate([np.ones(len(bpos)), (n / samples) * count[kept] if samples > 0 else np.zeros(0)])
        krows = pk[kpos]
        Wt = np.broadcast_to(wts, (len(qrows), len(krows)))
        gq, gk, gv = weighted_backward(q[qrows], k[krows], v[krows], Wt, do[qrows])
        dq[qrows] = gq
        np.add.at(dk, krows, gk)
        np.add.at(dv, krows, gv)
    return dq, dk, dv


def backward_head_blocks(q, k, v, do, cfg, b, h):
    """Non-causal (dq of query head h, dk and dv of its KV head restricted to
    that query head's contribution) by ``noncausal_backward_blocks``; arrays
    as for ``backward``."""
    if cfg.causal:
        raise ValueError("block-wise backward: non-causal problems only")
    B, H, Hkv, n, d = _check(q, k, v, cfg)
    g = h // (H // Hkv)
    R = projections(cfg.seed, d, cfg.proj_bits)
    return noncausal_backward_blocks(q[b, h].astype(np.float64), k[b, g].astype(np.float64),
                                     v[b, g].astype(np.float64), np.asarray(do[b, h], np.float64),
                                     ranks(q[b, h], R), ranks(k[b, g], R), cfg.seed, b, h, 1, cfg.block,
                                     cfg.samples)


def causal_dq_rows(q, k, v, do, rank_q, rank_k, seed, batch_idx, head, cfg, rows, out_round=None):
    """dq of the listed rows of one causal problem, each from its own row of
    ``causal_weights`` (the leaf's keys up to the row at weight 1, plus, at
    every split whose upper half holds the row, the quadrant's block keys
    and kept draws), so full sizes need no n x n matrix.  q, k, v, do
    [n, d] fp64; returns [len(rows), d].  out_round as for
    ``weighted_backward``."""
    n = len(rank_q)
    causal_levels(n, cfg.min_seq_len)
    perms = {}

    def quadrant_row(lo, mid, hi, node, iq):
        # row iq (local to [mid, hi)) of noncausal_weights(rank_q[mid:hi], rank_k[lo:mid], ...)
        if (lo, hi) not in perms:
            pq = sort_perm(rank_q[mid:hi])
            spos = np.empty(hi - mid, dtype=np.int64)
            spos[pq] = np.arange(hi - mid)
            perms[(lo, hi)] = (spos, sort_perm(rank_k[lo:mid]))
        spos, pk = perms[(lo, hi)]
        ns, nk = hi - mid, mid - lo
        b_eff = min(cfg.block, ns)
        b_k = key_block(b_eff, ns, nk)
        t = spos[iq] // b_eff
        bpos = np.arange(min(t * b_k, nk), min((t + 1) * b_k, nk))
        cols, wts = [pk[bpos]], [np.ones(len(bpos))]
        if cfg.samples > 0:
            pos, count = np.unique(sample_positions(seed, batch_idx, head, node, nk, cfg.samples),
                                   return_counts=True)
            kept = (pos // b_k) != t
            cols.append(pk[pos[kept]])
            wts.append((nk / cfg.samples) * count[kept])
        return lo + np.concatenate(cols), np.concatenate(wts)

    out = np.zeros((len(rows), q.shape[1]))
    for r, i in enumerate(rows):
        cols, wts = [], []
        lo, hi, node = 0, n, 1
        while hi - lo > cfg.min_seq_len:
            mid = lo + (hi - lo) // 2
            if i >= mid:
                c, w = quadrant_row(lo, mid, hi, node, i - mid)
                cols.append(c)
                wts.append(w)
                lo, node = mid, 2 * node + 1
            else:
                hi, node = mid, 2 * node
        cols.append(np.arange(lo, i + 1))
        wts.append(np.ones(i + 1 - lo))
        kc = np.concatenate(cols)
        Wr = np.concatenate(wts)[None, :]
        gq, _, _ = weighted_backward(q[i:i + 1], k[kc], v[kc], Wr, do[i:i + 1], out_round)
        out[r] = gq[0]
    return out
