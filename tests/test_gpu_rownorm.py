"""GPU parity of the row-norm-sampling variant (HA_FLAG_ROWNORM) against
``oracle.rownorm``, non-causal and causal (every quadrant of the
recursion with its node's draws; even splits and odd, rectangular ones).

* squared value-row norms: bit-exact (bf16 and fp32, d 64 and 128);
* integer CDF and draws: bit-exact (the draws decide integers, both sides
  use the same exact integer arithmetic);
* forward outputs: the block and uniform parts as in the fused forward,
  the row-norm part from a per-head copy of the drawn V rows carrying the
  draw weight T / (m n_t), rounded to the input dtype (bf16: 2^-9 relative
  per term) -- so the per-element bound is the forward's, scaled by the
  largest reference magnitude for bf16 (draws of small-norm rows carry
  large weights and lift outputs above 1 -- 2 to 5 here even with unit
  normal values -- where one bf16 rounding alone approaches 2e-2):
  max-abs <= 2e-2 max(1, max|ref|) and relative Frobenius <= 1e-2; fp32
  keeps the forward's unscaled bound, 1e-4 both; lse as the forward's (the
  normaliser is the uniform method's, and is asserted bit-identical to it).
"""

import numpy as np
import pytest
import torch

import approximate_long_context_amd as ha
from oracle import HAConfig
from oracle import rownorm as rn
from oracle import hyperattn as oh

from approximate_long_context_amd.workloads import WORKLOADS, make_inputs
from _util import np32, compare_lse, TOL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, H, Hkv, n, d, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(seed)
    s = d ** -0.25
    q = (torch.randn(B, H, n, d, generator=g) * s).to(dtype)
    k = (torch.randn(B, Hkv, n, d, generator=g) * s).to(dtype)
    scale = torch.exp(0.7 * torch.randn(B, Hkv, n, 1, generator=g))      # varied row norms
    v = (torch.randn(B, Hkv, n, d, generator=g) * scale).to(dtype)
    return q, k, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_row_sqnorms_bit_exact(dtype, d):
    _, _, v = _inputs(1, 1, 2, 700, d, 1, dtype)
    w = ha.row_sqnorms(v.to(DEV)).cpu().numpy()
    ref = rn.row_norms_sq(np32(v).reshape(-1, d)).reshape(w.shape)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("B,H,Hkv,n,d,m,seed", [(1, 2, 1, 1000, 64, 300, 2), (2, 4, 2, 4096, 128, 64, 3)])
def test_rownorm_draws_bit_exact(B, H, Hkv, n, d, m, seed):
    _, k, v = _inputs(B, H, Hkv, n, d, seed)
    R = oh.projections(seed, d, 6)
    perm = np.stack([np.stack([oh.sort_perm(oh.ranks(np32(k)[b, g], R)) for g in range(Hkv)])
                     for b in range(B)]).astype(np.int32)
    w = ha.row_sqnorms(v.to(DEV))
    cum, sidx = ha.rownorm_samples(w, torch.from_numpy(perm).to(DEV), H, m, seed)
    cum, sidx = cum.cpu().numpy(), sidx.cpu().numpy()
    G = H // Hkv
    for b in range(B):
        for g in range(Hkv):
            n_sorted = rn.quantized_weights(rn.row_norms_sq(np32(v)[b, g]))[perm[b, g]]
            assert np.array_equal(cum[b, g], np.cumsum(n_sorted))
        for h in range(H):
            n_sorted = rn.quantized_weights(rn.row_norms_sq(np32(v)[b, h // G]))[perm[b, h // G]]
            pos, _ = rn.rownorm_positions(seed, b, h, 1, n_sorted, m)
            assert np.array_equal(sidx[b, h], pos), (b, h)


CASES = [
    # B, H, Hkv, n, d, block, samples, r, seed, dtype
    (1, 2, 1, 1024, 64, 64, 128, 7, 4, torch.bfloat16),       # grouped heads
    (1, 2, 2, 1000, 128, 40, 50, 6, 5, torch.bfloat16),       # block not a multiple of 64, ragged tail
    (2, 1, 1, 512, 64, 512, 40, 5, 6, torch.bfloat16),        # one block: every draw excluded -> exact
    (1, 2, 2, 768, 64, 128, 0, 6, 7, torch.bfloat16),         # no samples: block part only
    (1, 1, 1, 1024, 64, 64, 64, 7, 8, torch.float32),         # fp32
    (1, 2, 1, 1000, 64, 128, 96, 7, 9, torch.bfloat16),       # ragged last block
    (1, 2, 2, 4096, 64, 256, 256, 7, 10, torch.bfloat16),     # many workgroups, one block each
    (1, 1, 1, 3000, 128, 24, 300, 6, 11, torch.bfloat16),     # small blocks: several per workgroup
    (2, 4, 2, 1500, 128, 96, 200, 7, 12, torch.float32),      # fp32, d = 128, batch 2, grouped heads
    (1, 2, 1, 65, 64, 16, 8, 4, 13, torch.bfloat16),          # tiny n: one partial tile, ragged blocks
]


@pytest.mark.parametrize("B,H,Hkv,n,d,block,m,r,seed,dtype", CASES)
def test_rownorm_forward_matches_oracle(B, H, Hkv, n, d, block, m, r, seed, dtype):
    q, k, v = _inputs(B, H, Hkv, n, d, 10 + seed, dtype)
    args = dict(block=block, samples=m, proj_bits=r, seed=seed)
    out, lse = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), flags=ha.HA_FLAG_ROWNORM, **args)
    torch.cuda.synchronize()
    ro, rl = rn.forward(np32(q), np32(k), np32(v), HAConfig(**args))
    got = np32(out).astype(np.float64)
    tol = TOL[dtype]
    scale = max(1.0, float(np.max(np.abs(ro)))) if dtype == torch.bfloat16 else 1.0
    err = float(np.max(np.abs(got - ro)))
    rel = float(np.linalg.norm(got - ro) / np.linalg.norm(ro))
    assert np.all(np.isfinite(got))
    assert err <= tol["max_abs"] * scale, f"max-abs {err:.3e} > {tol['max_abs']} x {scale:.2f}"
    assert rel <= tol["rel_fro"], f"rel-Frobenius {rel:.3e}"
    compare_lse(lse.cpu().numpy(), rl, dtype, "lse")
    # the normaliser is the uniform method's, computed by the same kernel
    # arithmetic (the first pass is its lse-only mode): identical bits
    _, l0 = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), **args)
    assert torch.equal(lse, l0)


def test_rownorm_rejects_other_flags():
    q, k, v = (t.to(DEV) for t in _inputs(1, 1, 1, 256, 64, 30))
    with pytest.raises(ha.HyperAttnError):
        ha.forward(q, k, v, block=64, samples=16, proj_bits=5, flags=ha.HA_FLAG_ROWNORM | ha.HA_FLAG_UNFUSED)
    with pytest.raises(ha.HyperAttnError):
        ha.forward(q, k, v, block=64, samples=16, proj_bits=5, causal=True, min_seq_len=64,
                   flags=ha.HA_FLAG_ROWNORM | ha.HA_FLAG_MATERIALIZE)


# ---- causal: every quadrant with its own node's draws ----------------------------------

CAUSAL_CASES = [
    # B, H, Hkv, n, d, block, samples, r, min_seq_len, seed, dtype
    (1, 2, 1, 2048, 64, 128, 64, 7, 256, 21, torch.bfloat16),     # even splits: one launch per level
    (1, 2, 2, 1000, 128, 64, 50, 6, 100, 22, torch.bfloat16),     # odd spans: node by node, rectangular
    (1, 1, 1, 1024, 64, 64, 64, 7, 128, 23, torch.float32),       # fp32
    (2, 4, 2, 1536, 128, 96, 200, 7, 192, 24, torch.float32),     # fp32, d = 128, batch 2, grouped heads
    (1, 2, 1, 4096, 64, 256, 256, 7, 512, 25, torch.bfloat16),    # several pieces per level
    (1, 2, 1, 777, 64, 32, 40, 5, 64, 26, torch.bfloat16),        # odd spans, small blocks, ragged tails
    (1, 1, 1, 512, 64, 512, 30, 5, 64, 27, torch.bfloat16),       # block >= every quadrant: exact
]


def _check_against(got, ro, lse, rl, dtype, what):
    got = got.astype(np.float64)
    tol = TOL[dtype]
    scale = max(1.0, float(np.max(np.abs(ro)))) if dtype == torch.bfloat16 else 1.0
    err = float(np.max(np.abs(got - ro)))
    rel = float(np.linalg.norm(got - ro) / np.linalg.norm(ro))
    assert np.all(np.isfinite(got)), what
    assert err <= tol["max_abs"] * scale, f"{what}: max-abs {err:.3e} > {tol['max_abs']} x {scale:.2f}"
    assert rel <= tol["rel_fro"], f"{what}: rel-Frobenius {rel:.3e}"
    compare_lse(lse, rl, dtype, f"{what} lse")


@pytest.mark.parametrize("B,H,Hkv,n,d,block,m,r,s,seed,dtype", CAUSAL_CASES)
def test_rownorm_causal_matches_oracle(B, H, Hkv, n, d, block, m, r, s, seed, dtype):
    print(f"[rownorm causal] n {n} d {d} block {block} samples {m} min_seq_len {s} {dtype}", flush=True)
    q, k, v = _inputs(B, H, Hkv, n, d, 40 + seed, dtype)
    args = dict(block=block, samples=m, proj_bits=r, seed=seed, causal=True, min_seq_len=s)
    out, lse = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), flags=ha.HA_FLAG_ROWNORM, **args)
    torch.cuda.synchronize()
    ro, rl = rn.forward(np32(q), np32(k), np32(v), HAConfig(**args))
    _check_against(np32(out), ro, lse.cpu().numpy(), rl, dtype, "causal row-norm")
    # the normaliser is the plain method's: the first pass of every level is
    # the quadrant kernel's lse-only mode and the merges see the same lse
    _, l0 = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), **args)
    assert torch.equal(lse, l0)


@pytest.mark.parametrize("causal", [False, True])
def test_rownorm_degenerate_value_rows(causal):
    """Degenerate weights: KV head 0 has all-zero value rows (T = 0: no
    draws, the numerator is the block part alone) and KV head 1 a single
    nonzero value row (every draw lands on it)."""
    B, H, Hkv, n, d = 1, 4, 2, 1024, 64
    q, k, v = _inputs(B, H, Hkv, n, d, 50)
    v[:, 0] = 0
    keep = v[:, 1, 333].clone()
    v[:, 1] = 0
    v[:, 1, 333] = keep
    args = dict(block=64, samples=96, proj_bits=6, seed=9, causal=causal, min_seq_len=128 if causal else 0)
    out, lse = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), flags=ha.HA_FLAG_ROWNORM, **args)
    torch.cuda.synchronize()
    ro, rl = rn.forward(np32(q), np32(k), np32(v), HAConfig(**args))
    _check_against(np32(out), ro, lse.cpu().numpy(), rl, torch.bfloat16, "degenerate values")
    assert not np.any(np32(out)[0, :2])                # heads of KV head 0: zero output


@pytest.mark.parametrize("n", [1, 3, 33])
@pytest.mark.parametrize("causal", [False, True])
def test_rownorm_tiny_n(n, causal):
    q, k, v = _inputs(1, 2, 1, n, 64, 70 + n)
    args = dict(block=2, samples=5, proj_bits=5, seed=4, causal=causal, min_seq_len=1 if causal else 0)
    out, lse = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), flags=ha.HA_FLAG_ROWNORM, **args)
    torch.cuda.synchronize()
    ro, rl = rn.forward(np32(q), np32(k), np32(v), HAConfig(**args))
    _check_against(np32(out), ro, lse.cpu().numpy(), rl, torch.bfloat16, f"tiny {n}")


def test_rownorm_causal_without_samples_is_the_plain_method():
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 1, 1000, 64, 32))
    args = dict(block=64, samples=0, proj_bits=6, seed=5, causal=True, min_seq_len=100)
    o1, l1 = ha.forward(q, k, v, flags=ha.HA_FLAG_ROWNORM, **args)
    o0, l0 = ha.forward(q, k, v, **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_rownorm_causal_repeatable():
    """Two calls give identical bits (no atomics; the draws are fixed by the seed)."""
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 1, 2048, 64, 33))
    args = dict(block=128, samples=64, proj_bits=7, seed=8, causal=True, min_seq_len=256)
    o1, l1 = ha.forward(q, k, v, flags=ha.HA_FLAG_ROWNORM, **args)
    o2, l2 = ha.forward(q, k, v, flags=ha.HA_FLAG_ROWNORM, **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_rownorm_without_lse_output():
    """A null lse pointer: the variant keeps its normaliser in the workspace
    and the output equals the one computed with an lse buffer."""
    import ctypes
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 1, 1024, 64, 31, torch.bfloat16))
    args = dict(block=128, samples=64, proj_bits=6, seed=3)
    ref, _ = ha.forward(q, k, v, flags=ha.HA_FLAG_ROWNORM, **args)
    out = torch.empty_like(q)
    wsb = ha.lib().hyperattn_workspace_bytes(1, 1024, 64, 2, 1, 128, 64, 6, 0, 0, ha.HA_BF16, ha.HA_FLAG_ROWNORM)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    ha._call("hyperattn_forward_ex", ha._ptr(q), ha._ptr(k), ha._ptr(v), ha.HA_BF16, 1, 1024, 64, 2, 1, 128, 64, 6,
             0, 0, ctypes.c_uint64(3), ha.HA_FLAG_ROWNORM, ha._ptr(out), None, ha._ptr(ws), ws.numel(),
             ha._stream(q.device))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.slow
def test_rownorm_full_workload_sampled_rows():
    """The non-causal long131k pass (32 heads, n = 131072, d = 64, block
    256, 256 samples) that the benchmark times the variant on: rows sampled
    from three heads (first, middle, last; all KV heads distinct) against
    the oracle computed one row at a time."""
    w = WORKLOADS["long131k"]
    assert not w.causal
    print("[rownorm long131k] generating inputs", flush=True)
    q, k, v = make_inputs(w, DEV)
    out, lse = ha.forward(q, k, v, flags=ha.HA_FLAG_ROWNORM, **w.method_args())
    torch.cuda.synchronize()
    g = np.random.default_rng(131)
    rows = np.array(sorted(set(g.choice(w.n, size=40, replace=False).tolist()) | {0, w.n // 2, w.n - 1}))
    heads = [(0, 0), (0, w.heads // 2), (0, w.heads - 1)]
    cfg = HAConfig(block=w.block, samples=w.samples, proj_bits=w.proj_bits, seed=w.seed)
    qc, kc, vc = np32(q), np32(k), np32(v)
    tol = TOL[w.dtype]
    for b, h in heads:
        print(f"[rownorm long131k] oracle rows of head {h}", flush=True)
        ro, rl = rn.forward_rows(qc, kc, vc, cfg, heads=[(b, h)], rows=rows)
        got = np32(out[b, h])[rows].astype(np.float64)
        ref = ro[0]
        scale = max(1.0, float(np.max(np.abs(ref))))
        err = float(np.max(np.abs(got - ref)))
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        assert np.all(np.isfinite(got))
        assert err <= tol["max_abs"] * scale, f"head {h}: max-abs {err:.3e} > {tol['max_abs']} x {scale:.2f}"
        assert rel <= tol["rel_fro"], f"head {h}: rel-Frobenius {rel:.3e}"
        compare_lse(np32(lse[b, h])[rows], rl[0], w.dtype, f"head {h} lse")


@pytest.mark.slow
def test_rownorm_causal_full_workload_sampled_rows():
    """The causal long131k forward (32 heads, n = 131072, d = 64, block 256,
    256 samples, min_seq_len 4096: five levels of quadrants) with the
    variant: rows sampled from two heads against the oracle one row at a
    time."""
    w = WORKLOADS["long131k_causal"]
    assert w.causal
    print("[rownorm long131k_causal] generating inputs", flush=True)
    q, k, v = make_inputs(w, DEV)
    out, lse = ha.forward(q, k, v, flags=ha.HA_FLAG_ROWNORM, **w.method_args())
    torch.cuda.synchronize()
    g = np.random.default_rng(137)
    rows = np.array(sorted(set(g.choice(w.n, size=40, replace=False).tolist()) | {0, 4095, 4096, w.n - 1}))
    cfg = HAConfig(block=w.block, samples=w.samples, proj_bits=w.proj_bits, causal=True,
                   min_seq_len=w.min_seq_len, seed=w.seed)
    qc, kc, vc = np32(q), np32(k), np32(v)
    for b, h in [(0, 0), (0, w.heads - 1)]:
        print(f"[rownorm long131k_causal] oracle rows of head {h}", flush=True)
        ro, rl = rn.forward_rows(qc, kc, vc, cfg, heads=[(b, h)], rows=rows)
        _check_against(np32(out[b, h])[rows], ro[0], np32(lse[b, h])[rows], rl[0], w.dtype, f"head {h}")
