"""HyperAttention forward pass, step by step, on the CPU in fp64.

Test infrastructure only (see the package docstring).

The method ([S] "Approach"; [A] "Abstract") approximates softmax attention
D^-1 A V, with A = exp(Q K^T) and D the diagonal of row sums of A:

  1. sortLSH: hash the rows of Q and K, sort each by bucket in
     Hamming (Gray-code) order and keep the equal-size diagonal blocks of
     the sorted matrix -- the entries found to be large;
  2. the normaliser D is the exact masked row sum over the row's block plus
     an estimate of the rest from uniformly sampled key columns;
  3. the product with V uses the same split: exact inside the block, the
     sampled columns outside it (reading below);
  4. causal masking by recursion ([S] summary line and "Limitations": a
     recursive causal-masking extension whose partitioning and merging cost
     shrinks the causal speed-up): both diagonal halves recurse causally,
     the off-diagonal quadrant (later queries, earlier keys) is unmasked
     and handled by steps 1-3, and the halves fall back to exact causal
     attention once they are short.

Readings taken where the pages are silent or garbled (each is repeated at
the function that uses it):

  * the product with V re-uses the uniform column samples of the
    normaliser; [S] "Approach" names row-norm sampling for the product,
    which is a different estimator and not built here;
  * a hash bit is the sign of the exact real dot product with the
    projection (no rounding);
  * A = exp(Q K^T) with no softmax scale (callers pre-scale Q and K);
  * no clipping or threshold constants (none are printed);
  * samples are iid uniform *with replacement* over the sorted key
    positions of the (sub)problem, shared by all its rows, and excluded for
    a row when they fall inside that row's block; each kept sample carries
    weight ns/m, so the out-of-block estimate is unbiased;
  * causal leaves: a span of length <= min_seq_len is computed exactly;
    a longer span must split into two even halves;
  * the non-causal call is one problem (node 1) and ignores min_seq_len.
"""

import math
from dataclasses import dataclass

import numpy as np

from .gauss import projections
from .philox import philox_words


@dataclass
class HAConfig:
    block: int
    samples: int
    proj_bits: int
    causal: bool = False
    min_seq_len: int = 0
    seed: int = 0


# ----------------------------------------------------------------------------
# Step 1: sortLSH -- hash, Gray-code rank, stable sort  ([S] "Approach",
# "Builds on": Hamming sorted LSH)
# ----------------------------------------------------------------------------

def hash_codes(x32, R):
    """Sign-bit code: bit p is 1 iff the exact real dot product <x, R_p> is
    positive (so an exact zero gives 0); projection 0 is the least
    significant bit.  A row or projection holding a non-finite value gives
    bit 0.

    Reading R3: the pages define the hash by the sign of the projection and
    give no arithmetic, so the sign is that of the exact sum.  Computed here
    as follows.  x (bf16 or fp32 values) and R (fp32) widen to fp64 exactly,
    and each product x_k R_pk is exact in fp64 (two 24-bit significands).
    Their fp64 sum t, in any order, is within (d - 1) u / (1 - (d - 1) u)
    of S = sum_k |x_k R_pk| (u = 2^-53, no underflow or overflow over this
    range), so |t| > 2 d u S fixes the sign.  The remaining cases take
    math.fsum, whose correctly rounded result has the sign of the exact
    sum."""
    x = np.asarray(x32, dtype=np.float64)
    Rd = np.asarray(R, dtype=np.float64)
    rows, d = x.shape
    code = np.zeros(rows, dtype=np.uint32)
    finite_x = np.all(np.isfinite(x), axis=1)
    for p in range(Rd.shape[0]):
        if not np.all(np.isfinite(Rd[p])):
            continue                                   # bit p is 0 for every row
        with np.errstate(invalid="ignore", over="ignore"):
            prod = x * Rd[p]                           # exact products
            t = prod.sum(axis=1)
            S = np.abs(prod).sum(axis=1)
        sure = np.abs(t) > 2.0 * d * 2.0 ** -53 * S
        bit = np.zeros(rows, dtype=bool)
        bit[sure] = t[sure] > 0
        for i in np.nonzero(~sure & finite_x)[0]:
            bit[i] = math.fsum(prod[i]) > 0
        bit &= finite_x
        code |= bit.astype(np.uint32) << np.uint32(p)
    return code


def gray_inverse(code, r):
    """Position of ``code`` in the reflected-binary Gray sequence g(k) = k ^ (k>>1):
    the prefix xor code ^ code>>1 ^ code>>2 ^ ... ^ code>>(r-1).

    Reading of "Hamming sorted": buckets are ordered by this position, so
    consecutive buckets differ in exactly one hash bit."""
    x = np.asarray(code, dtype=np.uint32).copy()
    shift = 1
    while shift < r:
        x ^= x >> np.uint32(shift)
        shift *= 2
    return x


def ranks(x32, R):
    """Bucket rank of each row: Gray position of its sign code."""
    return gray_inverse(hash_codes(x32, R), R.shape[0])


def sort_perm(rank):
    """Sorted position -> original index, ordered by (rank, index): the
    sort is stable, ties keep their original order."""
    return np.argsort(np.asarray(rank), kind="stable")


# ----------------------------------------------------------------------------
# Steps 2-3: exact block part + sampled part ([S] "Approach": exact masked
# row sums + uniform column sampling)
# ----------------------------------------------------------------------------

def sample_positions(seed, batch_idx, head, node, ns, m):
    """m sorted-key positions in [0, ns), iid uniform with replacement.

    Reading: word i of the Philox stream with counters
    (i // 4, node, head, 2*batch_idx + 1) under the seed (word i % 4 of that
    counter) becomes floor(word * ns / 2^32).  The last counter word is odd
    here and 0 for the projections, so the two streams never meet."""
    if m == 0:
        return np.zeros(0, dtype=np.int64)
    w = philox_words(seed, m, c1=node, c2=head, c3=2 * batch_idx + 1)
    return ((w * np.uint64(ns)) >> np.uint64(32)).astype(np.int64)


def _softmax_stats(S, V):
    """lse and softmax(S) V row by row, fp64 with max shift; rows whose
    scores are all -inf give lse = -inf and o = 0."""
    mx = np.max(S, axis=-1, keepdims=True)
    finite = np.isfinite(mx)
    mx_safe = np.where(finite, mx, 0.0)
    E = np.where(np.isfinite(S), np.exp(S - mx_safe), 0.0)
    ssum = E.sum(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.matmul(E, V) / ssum[..., None]
        lse = mx_safe[..., 0] + np.log(ssum)
    o = np.where((ssum > 0)[..., None], o, 0.0)
    lse = np.where(ssum > 0, lse, -np.inf)
    return lse, o


def key_block(b_eff, n_q, n_k):
    """Key block size b_k of a problem with n_q queries, n_k keys and query
    blocks of b_eff (reading R18): ceil(b_eff n_k / n_q), so that query
    block t pairs with key block t and b_k = b_eff when n_k = n_q."""
    return -(-b_eff * n_k // n_q)


def block_part(Qs, Ks, Vs, b_eff, positions=None, b_k=None):
    """Exact attention of sorted query p over the sorted keys of its own
    diagonal block t = p // b_eff, i.e. keys [t b_k, min((t+1) b_k, n_k))
    (reading R9: consecutive runs of b_eff sorted positions, the last run
    holding what remains; b_k = b_eff for square problems, R18 otherwise).
    Returns (lse_blk, o_blk) for ``positions`` (all if None):
    exp(lse_blk) = sum_{j in blk} e^{S_pj},  o_blk = that softmax times V."""
    ns, d = Qs.shape
    n_k = Ks.shape[0]
    b_k = b_eff if b_k is None else b_k
    if positions is None:
        positions = np.arange(ns)
    positions = np.asarray(positions, dtype=np.int64)
    lse = np.empty(len(positions))
    o = np.empty((len(positions), d))
    blk = positions // b_eff
    for t in np.unique(blk):
        rows = np.nonzero(blk == t)[0]
        lo, hi = min(t * b_k, n_k), min((t + 1) * b_k, n_k)
        if hi <= lo:                        # a rectangular problem's query block past the keys
            lse[rows] = -np.inf
            o[rows] = 0.0
            continue
        S = Qs[positions[rows]] @ Ks[lo:hi].T
        l, oo = _softmax_stats(S, Vs[lo:hi])
        lse[rows] = l
        o[rows] = oo
    return lse, o


def sample_part(Qs, Ks, Vs, idx, b_eff, positions=None, b_k=None):
    """Sampled estimate of the mass outside the row's block:
    D_smp = (n_k/m) sum_{i: idx_i // b_k != p // b_eff} e^{S_{p, idx_i}}
    and the matching weighted sum of value rows; duplicates count each time
    (b_k = b_eff for square problems).  Returns (lse_smp, o_smp) with
    exp(lse_smp) = D_smp; an empty sum gives lse = -inf, o = 0."""
    ns, d = Qs.shape
    n_k = Ks.shape[0]
    b_k = b_eff if b_k is None else b_k
    if positions is None:
        positions = np.arange(ns)
    positions = np.asarray(positions, dtype=np.int64)
    m = len(idx)
    if m == 0:
        return np.full(len(positions), -np.inf), np.zeros((len(positions), d))
    idx = np.asarray(idx, dtype=np.int64)
    Ksm = Ks[idx]
    Vsm = Vs[idx]
    col_blk = idx // b_k
    lse = np.empty(len(positions))
    o = np.empty((len(positions), d))
    for c in range(0, len(positions), 4096):
        p = positions[c:c + 4096]
        S = Qs[p] @ Ksm.T
        keep = (p // b_eff)[:, None] != col_blk[None, :]
        S = np.where(keep, S, -np.inf)
        l, oo = _softmax_stats(S, Vsm)
        lse[c:c + 4096] = l + np.log(n_k / m)
        o[c:c + 4096] = oo
    return lse, o


def lse_merge(l1, o1, l2, o2):
    """Merge two parts given as (lse, normalised output):
    lse = ln(e^l1 + e^l2), o = o1 e^{l1 - lse} + o2 e^{l2 - lse}."""
    l = np.logaddexp(l1, l2)
    with np.errstate(invalid="ignore"):
        w1 = np.where(np.isfinite(l1), np.exp(l1 - l), 0.0)
        w2 = np.where(np.isfinite(l2), np.exp(l2 - l), 0.0)
    return l, o1 * w1[..., None] + o2 * w2[..., None]


def noncausal_problem(q, k, v, rank_q, rank_k, seed, batch_idx, head, node,
                      block, samples, rows=None, parts=None):
    """One non-causal (sub)problem of ns queries and n_k keys (n_k = ns
    unless the problem is rectangular, reading R18).

    q: fp64 [ns, d], k, v: fp64 [n_k, d] rows in original order; rank_q,
    rank_k: bucket ranks of those rows.  Returns (o, lse) for ``rows``
    (local indices, all if None) in original row order.  If ``parts`` is a
    dict it receives the intermediates (perms, samples, per-part lse/o in
    sorted order)."""
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
    idx = sample_positions(seed, batch_idx, head, node, n_k, samples)
    if rows is None:
        positions = None
    else:
        inv = np.empty(ns, dtype=np.int64)
        inv[pq] = np.arange(ns)
        positions = inv[np.asarray(rows, dtype=np.int64)]
    lb, ob = block_part(Qs, Ks, Vs, b_eff, positions, b_k)
    ls, osm = sample_part(Qs, Ks, Vs, idx, b_eff, positions, b_k)
    lse, o = lse_merge(lb, ob, ls, osm)
    if parts is not None:
        parts.update(perm_q=pq, perm_k=pk, idx=idx, lse_blk=lb, o_blk=ob,
                     lse_smp=ls, o_smp=osm, b_eff=b_eff, b_k=b_k)
    if rows is None:
        out = np.empty_like(o)
        out[pq] = o                                # unsort
        lse_out = np.empty_like(lse)
        lse_out[pq] = lse
        return out, lse_out
    return o, lse


# ----------------------------------------------------------------------------
# Step 4: causal recursion ([S] summary and "Limitations")
# ----------------------------------------------------------------------------

def _exact_causal_rows(q, k, v, rows):
    """Exact causal softmax attention: local row i attends keys 0..i."""
    rows = np.asarray(rows, dtype=np.int64)
    S = q[rows] @ k.T
    S = np.where(np.arange(k.shape[0])[None, :] <= rows[:, None], S, -np.inf)
    lse, o = _softmax_stats(S, v)
    return o, lse


def causal_levels(n, min_seq_len):
    """Depth of the recursion: splits until every span is <= min_seq_len
    (the longest span at each depth has ceil(ns / 2) rows)."""
    L, ns = 0, n
    while ns > min_seq_len:
        ns = ns - ns // 2
        L += 1
    return L


def causal_problem(q, k, v, rank_q, rank_k, seed, batch_idx, head, cfg, rows=None, quadrant=None):
    """Causal HyperAttention of one head.  causal(lo, hi, node): a span of
    length <= min_seq_len is exact causal attention; otherwise, with
    mid = lo + (hi - lo) // 2 (reading R19: an odd span gives its right
    half the extra row), causal(lo, mid, 2 node) and causal(mid, hi,
    2 node + 1) recurse, and rows [mid, hi) are merged (deepest level
    first) with the non-causal problem of queries [mid, hi) over keys
    [lo, mid) (rectangular when the span is odd, reading R18), with this
    node's samples.  Ranks come from the one hash of the whole sequence
    (one projection matrix for all nodes).

    ``quadrant(lo, mid, hi, node, local_rows) -> (o, lse)`` solves one
    quadrant (rows local to [mid, hi)); None: ``noncausal_problem``."""
    n, d = q.shape
    s = cfg.min_seq_len
    all_rows = np.arange(n) if rows is None else np.sort(np.asarray(rows, dtype=np.int64))
    o_out = np.zeros((len(all_rows), d))
    l_out = np.zeros(len(all_rows))
    pos_of = {int(r): i for i, r in enumerate(all_rows)}

    def rec(lo, hi, node, want):
        ns = hi - lo
        if len(want) == 0:
            return
        if ns <= s:
            o, l = _exact_causal_rows(q[lo:hi], k[lo:hi], v[lo:hi], want - lo)
            for j, r in enumerate(want):
                o_out[pos_of[int(r)]] = o[j]
                l_out[pos_of[int(r)]] = l[j]
            return
        mid = lo + ns // 2
        rec(lo, mid, 2 * node, want[want < mid])
        upper = want[want >= mid]
        rec(mid, hi, 2 * node + 1, upper)
        if len(upper) == 0:
            return
        if quadrant is None:
            oq, lq = noncausal_problem(q[mid:hi], k[lo:mid], v[lo:mid], rank_q[mid:hi],
                                       rank_k[lo:mid], seed, batch_idx, head, node,
                                       cfg.block, cfg.samples, rows=upper - mid)
        else:
            oq, lq = quadrant(lo, mid, hi, node, upper - mid)
        sel = np.array([pos_of[int(r)] for r in upper])
        l_new, o_new = lse_merge(l_out[sel], o_out[sel], lq, oq)
        l_out[sel] = l_new
        o_out[sel] = o_new

    rec(0, n, 1, all_rows)
    return o_out, l_out


def causal_parts(q, k, v, rank_q, rank_k, seed, batch_idx, head, cfg):
    """The intermediates of the causal recursion of one head, problem by
    problem (the same split as ``causal_problem``): returns (leaves, quads).

    leaves: list of dicts (lo, hi, o, lse) -- exact causal attention of
    rows [lo, hi) over keys lo..row, in row order.
    quads: list of dicts (lo, mid, hi, node, depth) plus the ``parts`` of
    the non-causal problem of queries [mid, hi) over keys [lo, mid): perm_q
    and perm_k (sorted position -> row within the problem), idx (this
    node's sample positions), lse_blk, o_blk, lse_smp, o_smp (sorted query
    order), listed parents before children.  A row's result is the log-sum-
    exp merge of its leaf with the quadrants holding it, deepest first."""
    n, d = q.shape
    s = cfg.min_seq_len
    leaves, quads = [], []

    def rec(lo, hi, node, depth):
        ns = hi - lo
        if ns <= s:
            o, l = _exact_causal_rows(q[lo:hi], k[lo:hi], v[lo:hi], np.arange(ns))
            leaves.append(dict(lo=lo, hi=hi, o=o, lse=l))
            return
        mid = lo + ns // 2
        parts = {}
        noncausal_problem(q[mid:hi], k[lo:mid], v[lo:mid], rank_q[mid:hi], rank_k[lo:mid], seed,
                          batch_idx, head, node, cfg.block, cfg.samples, parts=parts)
        quads.append(dict(lo=lo, mid=mid, hi=hi, node=node, depth=depth, **parts))
        rec(lo, mid, 2 * node, depth + 1)
        rec(mid, hi, 2 * node + 1, depth + 1)

    rec(0, n, 1, 0)
    return leaves, quads


# ----------------------------------------------------------------------------
# Whole forward and exact attention
# ----------------------------------------------------------------------------

def _check(q, k, v, cfg):
    B, H, n, d = q.shape
    if k.shape[0] != B or k.shape[2] != n or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    Hkv = k.shape[1]
    if Hkv < 1 or H % Hkv:
        raise ValueError("heads must be a multiple of kv_heads")
    if not 1 <= cfg.proj_bits <= 16:
        raise ValueError("proj_bits must be in [1, 16]")
    if cfg.block < 1 or cfg.samples < 0:
        raise ValueError("block >= 1 and samples >= 0 required")
    if cfg.causal:
        causal_levels(n, cfg.min_seq_len)
    return B, H, Hkv, n, d


def forward_rows(q, k, v, cfg, heads=None, rows=None):
    """HyperAttention forward for the listed (batch, head) pairs and
    original row indices (all if None).

    q: [B, H, n, d], k, v: [B, Hkv, n, d] float32 arrays holding the input
    values exactly (bf16 inputs widened); query head h uses KV head
    h // (H / Hkv).  Returns (out, lse) in fp64 with shapes
    [len(heads), len(rows), d] and [len(heads), len(rows)]."""
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
    rank_cache = {}
    for i, (b, h) in enumerate(heads):
        g = h // G
        if (b, g) not in rank_cache:
            rank_cache[(b, g)] = ranks(k[b, g], R)
        rk = rank_cache[(b, g)]
        rq = ranks(q[b, h], R)
        qh = q[b, h].astype(np.float64)
        kh = k[b, g].astype(np.float64)
        vh = v[b, g].astype(np.float64)
        if cfg.causal:
            o, l = causal_problem(qh, kh, vh, rq, rk, cfg.seed, b, h, cfg, rows=rows)
        else:
            o, l = noncausal_problem(qh, kh, vh, rq, rk, cfg.seed, b, h, 1,
                                     cfg.block, cfg.samples, rows=rows)
        out[i] = o
        lse[i] = l
    return out, lse


def forward(q, k, v, cfg):
    """Full forward: (out [B, H, n, d], lse [B, H, n]) in fp64."""
    B, H = q.shape[:2]
    out, lse = forward_rows(q, k, v, cfg)
    return out.reshape(B, H, q.shape[2], q.shape[3]), lse.reshape(B, H, q.shape[2])


def forward_rect(q, k, v, cfg):
    """Non-causal forward of a rectangular problem (reading R18): q
    [B, H, n_q, d], k, v [B, Hkv, n_k, d] float32 arrays holding the input
    values exactly.  Returns (out [B, H, n_q, d], lse [B, H, n_q]) in fp64."""
    if cfg.causal:
        raise ValueError("rectangular problems are non-causal")
    B, H, n_q, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    Hkv, n_k = k.shape[1], k.shape[2]
    if Hkv < 1 or H % Hkv:
        raise ValueError("heads must be a multiple of kv_heads")
    if cfg.block < 1 or cfg.samples < 0 or not 1 <= cfg.proj_bits <= 16:
        raise ValueError("bad method arguments")
    G = H // Hkv
    R = projections(cfg.seed, d, cfg.proj_bits)
    out = np.zeros((B, H, n_q, d))
    lse = np.zeros((B, H, n_q))
    for b in range(B):
        for h in range(H):
            g = h // G
            o, l = noncausal_problem(q[b, h].astype(np.float64), k[b, g].astype(np.float64),
                                     v[b, g].astype(np.float64), ranks(q[b, h], R), ranks(k[b, g], R),
                                     cfg.seed, b, h, 1, cfg.block, cfg.samples)
            out[b, h] = o
            lse[b, h] = l
    return out, lse


def exact_attention(q, k, v, causal=False):
    """softmax(Q K^T) V per head (no scale), fp64, GQA by h // (H / Hkv).
    Returns (out, lse)."""
    B, H, n, d = q.shape
    G = H // k.shape[1]
    out = np.zeros((B, H, n, d))
    lse = np.zeros((B, H, n))
    for b in range(B):
        for h in range(H):
            qh = q[b, h].astype(np.float64)
            kh = k[b, h // G].astype(np.float64)
            vh = v[b, h // G].astype(np.float64)
            S = qh @ kh.T
            if causal:
                S = np.where(np.tri(n, dtype=bool), S, -np.inf)
            lse[b, h], out[b, h] = _softmax_stats(S, vh)
    return out, lse
