"""GPU parity of the individual stages against the oracle, through the C ABI.

Bit-exact: projection matrix, hash ranks, sort permutations (stable), sample
positions, gather.  Tolerance: block part, sampled part, fused parts,
merge+unsort and exact causal leaves.
"""

import numpy as np
import pytest
import torch

import approximate_long_context_amd as ha
import oracle
from oracle import hyperattn as oh

from _util import TOL, compare, compare_lse, np32

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("d,r", [(64, 7), (128, 8), (64, 16), (128, 1), (8, 3), (100, 5)])
def test_projections_device_bit_exact(d, r):
    for seed in [0, 1, 7, 2**40 + 3, 2**64 - 1]:
        got = ha.projections(seed, d, r, DEV).cpu().numpy()
        assert np.array_equal(got, oracle.projections(seed, d, r)), (seed, d, r)


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("r", [1, 7, 8, 16])
def test_hash_bit_exact(dtype, d, r):
    rows = 4099                                   # ragged against rows per wave
    x = _rand((rows, d), dtype, 100 + d + r)
    x[5] = 0                                      # zero row -> code 0
    x[6, 3] = float("nan") if dtype == torch.float32 else x[6, 3]
    R = ha.projections(r, d, r, DEV)
    got = ha.hash_rows(x.to(DEV), R).cpu().numpy().astype(np.uint32)
    ref = oracle.ranks(np32(x), R.cpu().numpy())
    assert np.array_equal(got, ref), int((got != ref).sum())


def _adversarial_rows(d, dtype, seed):
    """Rows whose dot products with R (see _adversarial_R) cancel exactly,
    lose low-order terms in fp32 and fp64, sit near the subnormal range or
    hold non-finite values; plus random rows."""
    rng = np.random.default_rng(seed)
    rows = []
    for a in (1.0, 2.0**-20, 2.0**20, 3.0):
        x = np.zeros(d, np.float64)
        x[0], x[1] = a, -a                                # R_0 = R_1: exact zero for every projection
        rows.append(x)
        y = x.copy()
        y[5] = 2.0**-30                                   # tiny term decides the sign
        rows.append(y)
    x = np.zeros(d, np.float64)
    x[2], x[3], x[4] = 1.0, 2.0**100, -(2.0**100)         # R_2 + 2^100 R_3 - 2^100 R_3: sign of R_2,
    rows.append(x)                                        # lost by fp32 and fp64 sums in any order
    rows.append(-x)
    x = np.zeros(d, np.float64)
    x[3:9] = 2.0**-126 if dtype == torch.float32 else 2.0**-120   # tiny magnitudes
    rows.append(x)
    x = np.ones(d, np.float64)
    x[7] = np.inf
    rows.append(x)
    x = np.ones(d, np.float64)
    x[9] = np.nan
    rows.append(x)
    rows.append(np.zeros(d, np.float64))
    for _ in range(200):
        rows.append(rng.standard_normal(d))
    return torch.tensor(np.stack(rows), dtype=torch.float64).to(dtype)


def _adversarial_R(d, r, seed):
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((r, d)).astype(np.float32)
    R[:, 1] = R[:, 0]
    R[:, 4] = R[:, 3]
    R[:, 2] = np.abs(R[:, 2]) * np.where(np.arange(r) % 2 == 0, 1, -1)   # sign of R_2 alternates
    return R


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_hash_exact_sign_adversarial(dtype, d):
    r = 8
    x = _adversarial_rows(d, dtype, 5 + d)
    R = _adversarial_R(d, r, 9 + d)
    Rn = R.copy()
    Rn[3, 4] = np.inf                                     # a non-finite projection: bit 3 is 0 everywhere
    for Rm in (R, Rn):
        got = ha.hash_rows(x.to(DEV), torch.from_numpy(Rm).to(DEV)).cpu().numpy().astype(np.uint32)
        ref = oracle.ranks(np32(x), Rm)
        assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:10]
    codes = oracle.hash_codes(np32(x), R)
    assert all(codes[i] == 0 for i in range(0, 8, 2))    # exact zeros
    assert codes[8] == sum(1 << p for p in range(r) if p % 2 == 0)   # sign of R_2
    assert codes[9] == sum(1 << p for p in range(r) if p % 2 == 1)
    assert codes[11] == 0 and codes[12] == 0 and codes[13] == 0       # inf, NaN, zero rows


@pytest.mark.parametrize("heads,n,length,first,stride,pieces,r", [
    (3, 5000, 5000, 0, 5000, 1, 7),       # two tiles, ragged
    (2, 20000, 20000, 0, 20000, 1, 8),    # five tiles
    (4, 4096, 1024, 1024, 2048, 2, 7),    # causal-level layout (odd halves)
    (4, 4096, 1024, 0, 2048, 2, 7),       # even halves
    (2, 9000, 4500, 4500, 9000, 1, 7),
    (3, 3000, 3000, 0, 3000, 1, 12),      # two passes
    (2, 70000, 35000, 0, 35000, 2, 16),   # two passes, many tiles
    (1, 1, 1, 0, 1, 1, 3),
    (5, 100, 37, 3, 40, 2, 2),
])
def test_sort_bit_exact(heads, n, length, first, stride, pieces, r):
    g = np.random.default_rng(heads * n + r)
    rank = g.integers(0, 1 << r, size=(heads, n)).astype(np.uint16)
    perm = ha.sort_ranks(torch.from_numpy(rank.view(np.int16)).view(torch.uint16).to(DEV), r,
                         length=length, first=first, stride=stride, pieces=pieces).cpu().numpy()
    for hd in range(heads):
        for i in range(pieces):
            lo = first + i * stride
            ref = lo + oracle.sort_perm(rank[hd, lo:lo + length])
            assert np.array_equal(perm[hd, i], ref), (hd, i)


@pytest.mark.parametrize("batch,heads,node_first,node_count,ns,m", [
    (1, 1, 1, 1, 1024, 64), (2, 3, 4, 4, 4096, 256), (1, 32, 1, 1, 131072, 256),
    (1, 2, 16, 16, 1000, 7), (1, 1, 1, 1, 1, 5)])
def test_sample_indices_bit_exact(batch, heads, node_first, node_count, ns, m):
    got = ha.sample_indices(11, batch, heads, ns, m, node_first, node_count, DEV).cpu().numpy()
    for b in range(batch):
        for h in range(heads):
            for j in range(node_count):
                ref = oracle.sample_positions(11, b, h, node_first + j, ns, m)
                assert np.array_equal(got[b, h, j], ref)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.float32, 128)])
def test_gather_bit_exact(dtype, d):
    src = _rand((3, 777, d), dtype, 5).to(DEV)
    g = np.random.default_rng(1)
    perm = torch.from_numpy(np.stack([g.permutation(777) for _ in range(3)]).astype(np.int32)).to(DEV)
    got = ha.gather_rows(src, perm)
    ref = torch.stack([src[h][perm[h].long()] for h in range(3)])
    assert torch.equal(got, ref)


def _problem(dtype, B, H, Hkv, n, d, block, m, seed=3, scale=None):
    g = torch.Generator(device="cpu").manual_seed(seed)
    s = d ** -0.25 if scale is None else scale
    q = (torch.randn(B, H, n, d, generator=g) * s).to(dtype)
    k = (torch.randn(B, Hkv, n, d, generator=g) * s).to(dtype)
    v = torch.randn(B, Hkv, n, d, generator=g).to(dtype)
    return q, k, v


@pytest.mark.parametrize("dtype,n,d,block,m,H,Hkv", [
    (torch.bfloat16, 1024, 64, 256, 128, 2, 1),
    (torch.bfloat16, 1000, 128, 40, 50, 2, 2),      # blocks smaller than a tile, ragged
    (torch.float32, 1024, 64, 64, 64, 1, 1),
    (torch.bfloat16, 768, 64, 768, 30, 1, 1),       # one block = the whole segment
])
def test_attend_parts_match_oracle(dtype, n, d, block, m, H, Hkv):
    q, k, v = _problem(dtype, 1, H, Hkv, n, d, block, m)
    seed = 5
    R = oracle.projections(seed, d, 7)
    G = H // Hkv
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    Rd = torch.from_numpy(R).to(DEV)
    perm_q = ha.sort_ranks(ha.hash_rows(qd.view(-1, n, d), Rd), 7).view(H, n)
    perm_k = ha.sort_ranks(ha.hash_rows(kd.view(-1, n, d), Rd), 7).view(Hkv, n)
    idx = ha.sample_indices(seed, 1, H, n, m, device=DEV)
    res = {p: ha.attend(qd, kd, vd, perm_q, perm_k, idx, block=block, samples=m, parts=p) for p in (1, 2, 3)}
    for h in range(H):
        parts = {}
        q64 = np32(q[0, h]).astype(np.float64)
        k64 = np32(k[0, h // G]).astype(np.float64)
        v64 = np32(v[0, h // G]).astype(np.float64)
        oh.noncausal_problem(q64, k64, v64, oracle.ranks(np32(q[0, h]), R), oracle.ranks(np32(k[0, h // G]), R),
                             seed, 0, h, 1, block, m, parts=parts)
        assert np.array_equal(perm_q[h].cpu().numpy(), parts["perm_q"])
        assert np.array_equal(perm_k[h // G].cpu().numpy(), parts["perm_k"])
        assert np.array_equal(idx[0, h, 0].cpu().numpy(), parts["idx"])
        tol = TOL[torch.float32] if dtype == torch.float32 else dict(max_abs=2e-2)
        o1, l1 = res[1]
        compare(np32(o1[0, h]), parts["o_blk"], dtype, "block part")
        compare_lse(np32(l1[0, h]), parts["lse_blk"], dtype, "block lse")
        o2, l2 = res[2]
        ls = parts["lse_smp"]
        fin = np.isfinite(ls)
        compare(np32(o2[0, h])[fin], parts["o_smp"][fin], dtype, "sample part")
        compare_lse(np32(l2[0, h]), ls, dtype, "sample lse")
        o3, l3 = res[3]
        lse_t, o_t = oh.lse_merge(parts["lse_blk"], parts["o_blk"], ls, parts["o_smp"])
        compare(np32(o3[0, h]), o_t, dtype, "fused parts")
        compare_lse(np32(l3[0, h]), lse_t, dtype, "fused lse")
        # mass invariant on the GPU: exp(lse) = exp(lse_blk) + exp(lse_smp).
        # bf16: the kernel sums the bf16-rounded P it multiplies V with, so
        # each of the three lse values carries up to 2^-9 relative error.
        gl = np.logaddexp(np32(l1[0, h]).astype(np.float64), np32(l2[0, h]).astype(np.float64))
        assert np.max(np.abs(gl - np32(l3[0, h]))) < (1e-5 if dtype == torch.float32 else 3 * 2.0**-9)
        del tol
    # merge + unsort kernel reproduces the fused result
    out, lse = ha.merge_unsort(res[1][0].view(H, n, d), res[1][1].view(H, n), res[2][0].view(H, n, d),
                               res[2][1].view(H, n), perm_q, dtype=dtype)
    for h in range(H):
        p = perm_q[h].long().cpu()
        compare(np32(out[h])[p.numpy()], np32(res[3][0][0, h]), dtype, "merge_unsort")


@pytest.mark.parametrize("dtype,n,d,leaf,H,Hkv", [
    (torch.bfloat16, 1024, 64, 512, 2, 1),
    (torch.bfloat16, 600, 128, 200, 1, 1),     # leaves not a multiple of the tile
    (torch.float32, 256, 64, 256, 1, 1),
])
def test_causal_leaves_match_exact(dtype, n, d, leaf, H, Hkv):
    q, k, v = _problem(dtype, 1, H, Hkv, n, d, 1, 0, seed=8)
    o, lse = ha.causal_leaves(q.to(DEV), k.to(DEV), v.to(DEV), leaf)
    G = H // Hkv
    for h in range(H):
        for a in range(0, n, leaf):
            sl = slice(a, a + leaf)
            ref_o, ref_l = oracle.exact_attention(np32(q[:, h:h + 1, sl]), np32(k[:, h // G:h // G + 1, sl]),
                                                  np32(v[:, h // G:h // G + 1, sl]), causal=True)
            compare(np32(o[0, h, sl]), ref_o[0, 0], dtype, "leaf")
            compare_lse(np32(lse[0, h, sl]), ref_l[0, 0], dtype, "leaf lse")
