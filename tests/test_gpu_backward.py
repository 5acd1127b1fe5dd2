"""GPU parity of the backward (bf16 and fp32, non-causal and causal) against the fp64 oracle.

The library's forward gives (out, lse); its backward then gives dq, dk, dv
in fp32, compared with ``oracle.backward.backward`` on the same bf16 inputs
and upstream gradient.  Tolerance (derived from the arithmetic): the
kernels round P to bf16 before the P^T dO product and dS = P (dP - D) to
bf16 before dS K and dS^T Q (relative 2^-9 ~ 2e-3 per term, averaging
down over the sums), and D comes from the bf16-rounded forward output; so
the Frobenius error is about 2e-3 relative (measured 1.7e-3) and the
largest element error a few 1e-3 of the largest reference magnitude
(measured up to 3.4e-3).  Bounds: 5e-3 and 8e-3.
"""

import numpy as np
import pytest
import torch

import approximate_long_context_amd as ha
from approximate_long_context_amd.workloads import WORKLOADS, make_inputs
from oracle import HAConfig
from oracle import backward as ob
from oracle import hyperattn as oh
from oracle.gauss import projections

from _util import np32

pytestmark = pytest.mark.gpu
DEV = "cuda"

REL_F = 5e-3
REL_MAX = 8e-3


def _inputs(B, H, Hkv, n, d, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    s = d ** -0.25
    q = (torch.randn(B, H, n, d, generator=g) * s).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, n, d, generator=g) * s).to(torch.bfloat16)
    v = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16)
    do = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    return q, k, v, do


def _compare(got, ref, what):
    got = got.astype(np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    scale = float(np.max(np.abs(ref))) or 1.0
    max_err = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / (np.linalg.norm(ref) or 1.0))
    assert max_err <= REL_MAX * scale, f"{what}: max-abs {max_err:.3e} > {REL_MAX} x {scale:.3e}"
    assert rel <= REL_F, f"{what}: rel-Frobenius {rel:.3e} > {REL_F}"


CASES = [
    # B, H, Hkv, n, d, block, samples, r, seed
    (1, 2, 1, 1024, 64, 256, 128, 7, 3),      # grouped heads, 8 waves x 32 per block
    (1, 2, 2, 1000, 128, 40, 50, 6, 4),       # blocks smaller than a tile, ragged
    (2, 2, 2, 512, 64, 64, 200, 5, 5),        # many duplicate samples
    (1, 1, 1, 768, 64, 768, 30, 7, 6),        # one block = the whole segment: samples all excluded
    (1, 2, 1, 1024, 64, 128, 0, 7, 7),        # no samples
    (1, 4, 2, 2048, 128, 512, 256, 8, 8),     # d = 128, block wider than a workgroup
    (1, 2, 1, 960, 64, 96, 70, 6, 9),         # block not a multiple of the 64-row tile
    (1, 2, 1, 1000, 64, 256, 64, 7, 10),      # ragged last block (1000 = 3 x 256 + 232)
    (1, 2, 2, 1100, 128, 64, 40, 6, 11),      # ragged last block, d = 128
]


CAUSAL_CASES = [
    # B, H, Hkv, n, d, block, samples, r, min_seq_len, seed
    (1, 2, 1, 1024, 64, 64, 32, 6, 256, 21),      # two levels, 256-row leaves, grouped heads
    (1, 2, 2, 1000, 128, 25, 20, 6, 128, 22),     # 125-row leaves, blocks not a multiple of 64
    (1, 4, 2, 2048, 64, 128, 64, 7, 512, 23),     # grouped heads, leaves of two workgroups
    (1, 2, 1, 512, 64, 64, 16, 5, 512, 24),       # leaf only (no quadrant level)
    (2, 2, 2, 2048, 128, 256, 128, 7, 256, 25),   # d = 128, three levels, batch 2
    (1, 2, 1, 2048, 64, 96, 32, 6, 256, 26),      # quadrants of 1024, 512, 256 rows: ragged last blocks
]


def _run(B, H, Hkv, n, d, seed, **args):
    q, k, v, do = _inputs(B, H, Hkv, n, d, 100 + seed)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = ha.forward(qd, kd, vd, seed=seed, **args)
    dq, dk, dv = ha.backward(qd, kd, vd, out, lse, dod, seed=seed, **args)
    torch.cuda.synchronize()
    cfg = HAConfig(seed=seed, **args)
    rq, rk, rv = ob.backward(np32(q), np32(k), np32(v), np32(do), cfg)
    _compare(dq.cpu().numpy(), rq, "dq")
    _compare(dk.cpu().numpy(), rk, "dk")
    _compare(dv.cpu().numpy(), rv, "dv")


@pytest.mark.parametrize("B,H,Hkv,n,d,block,m,r,seed", CASES)
def test_backward_matches_oracle(B, H, Hkv, n, d, block, m, r, seed):
    _run(B, H, Hkv, n, d, seed, block=block, samples=m, proj_bits=r)


@pytest.mark.parametrize("B,H,Hkv,n,d,block,m,r,s,seed", CAUSAL_CASES)
def test_causal_backward_matches_oracle(B, H, Hkv, n, d, block, m, r, s, seed):
    _run(B, H, Hkv, n, d, seed, block=block, samples=m, proj_bits=r, causal=True, min_seq_len=s)


@pytest.mark.parametrize("H,Hkv,n,d,block,m,causal,s", [
    (2, 2, 1024, 64, 256, 64, False, 0),
    (8, 2, 1024, 64, 128, 512, False, 0),          # grouped heads, many duplicate draws per key
    (4, 1, 2048, 128, 96, 300, True, 256),         # causal levels, ragged blocks
    (2, 1, 1000, 64, 64, 200, True, 100),          # odd splits
])
def test_backward_deterministic(H, Hkv, n, d, block, m, causal, s):
    """dQ, dK and dV are bitwise repeatable: the sampled keys' partial rows
    are summed in a fixed order (sorted by key position and slot), one writer
    per key row; a workspace holding garbage changes nothing."""
    q, k, v, do = _inputs(1, H, Hkv, n, d, 11 + n)
    args = dict(block=block, samples=m, proj_bits=7, seed=1, causal=causal, min_seq_len=s)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = ha.forward(qd, kd, vd, **args)
    a = ha.backward(qd, kd, vd, out, lse, dod, **args)
    wsb = ha.backward_workspace_bytes(1, n, d, H, Hkv, block, m, 7, causal, s)
    ws = torch.randint(0, 255, (wsb,), dtype=torch.uint8, device=DEV)
    for _ in range(3):
        b = ha.backward(qd, kd, vd, out, lse, dod, workspace=ws, **args)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))


FP32_CASES = [
    # B, H, Hkv, n, d, block, samples, r, causal, min_seq_len, seed
    (1, 1, 1, 1024, 64, 64, 64, 7, False, 0, 31),       # the fp32 single-head workload
    (1, 4, 2, 777, 128, 96, 40, 6, False, 0, 32),       # grouped heads, ragged last block, d = 128
    (2, 2, 2, 512, 64, 64, 200, 5, False, 0, 33),       # many duplicate samples
    (1, 2, 1, 1024, 64, 64, 32, 6, True, 256, 34),      # two causal levels, grouped heads
    (1, 2, 2, 1000, 128, 64, 20, 6, True, 100, 35),     # odd splits
]


def _inputs32(B, H, Hkv, n, d, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    s = d ** -0.25
    return (torch.randn(B, H, n, d, generator=g) * s, torch.randn(B, Hkv, n, d, generator=g) * s,
            torch.randn(B, Hkv, n, d, generator=g), torch.randn(B, H, n, d, generator=g))


@pytest.mark.parametrize("B,H,Hkv,n,d,block,m,r,causal,s,seed", FP32_CASES)
def test_backward_fp32_matches_oracle(B, H, Hkv, n, d, block, m, r, causal, s, seed):
    """fp32 inputs run the fp32 kernels; against the fp64 oracle within 1e-4
    relative (Frobenius, and per element against the largest magnitude)."""
    q, k, v, do = _inputs32(B, H, Hkv, n, d, seed)
    args = dict(block=block, samples=m, proj_bits=r, causal=causal, min_seq_len=s, seed=seed)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = ha.forward(qd, kd, vd, **args)
    dq, dk, dv = ha.backward(qd, kd, vd, out, lse, dod, **args)
    dq2, dk2, dv2 = ha.backward(qd, kd, vd, out, lse, dod, **args)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)
    rq, rk, rv = ob.backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), HAConfig(**args))
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        got = got.cpu().numpy().astype(np.float64)
        scale = float(np.max(np.abs(ref))) or 1.0
        assert float(np.max(np.abs(got - ref))) <= 1e-4 * scale, what
        assert float(np.linalg.norm(got - ref) / np.linalg.norm(ref)) <= 1e-4, what


def test_backward_rect_fp32():
    q, k, v, do = _inputs32(1, 2, 1, 300, 64, 36)
    k2, v2 = _inputs32(1, 1, 1, 700, 64, 37)[1:3]
    args = dict(block=50, samples=30, proj_bits=6, seed=3)
    qd, kd, vd, dod = q.to(DEV), k2.to(DEV), v2.to(DEV), do.to(DEV)
    out, lse = ha.forward_rect(qd, kd, vd, **args)
    dq, dk, dv = ha.backward_rect(qd, kd, vd, out, lse, dod, **args)
    torch.cuda.synchronize()
    rq, rk, rv = ob.backward_rect(q.numpy(), k2.numpy(), v2.numpy(), do.numpy(), HAConfig(**args))
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        got = got.cpu().numpy().astype(np.float64)
        assert float(np.linalg.norm(got - ref) / np.linalg.norm(ref)) <= 1e-4, what


ODD_CASES = [
    # B, H, Hkv, n, d, block, samples, r, min_seq_len, seed: some span splits unevenly,
    # so quadrants are rectangular (n_q = n_k + 1) and leaves have varied lengths
    (1, 2, 1, 1000, 64, 64, 16, 5, 100, 31),      # 1000 -> 500 -> 250 -> 125 -> 62 | 63
    (1, 2, 2, 777, 128, 40, 24, 6, 150, 32),      # odd at the top, d = 128
    (1, 1, 1, 301, 64, 32, 8, 5, 64, 33),         # small ragged leaves
]


@pytest.mark.parametrize("B,H,Hkv,n,d,block,m,r,s,seed", ODD_CASES)
def test_causal_backward_odd_splits_match_oracle(B, H, Hkv, n, d, block, m, r, s, seed):
    _run(B, H, Hkv, n, d, seed, block=block, samples=m, proj_bits=r, causal=True, min_seq_len=s)


@pytest.mark.parametrize("n", [1, 3, 33])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_tiny_n(n, causal):
    """Heads of a few rows (one partial tile; causal splits down to leaves
    of one or two rows), bf16 and fp32."""
    for s in ((1, 2) if causal else (0,)):
        args = dict(block=2, samples=3, proj_bits=5, causal=causal, min_seq_len=s)
        _run(1, 2, 1, n, 64, 50 + n, **args)
        q, k, v, do = _inputs32(1, 2, 1, n, 64, 60 + n)
        qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
        out, lse = ha.forward(qd, kd, vd, seed=5, **args)
        dq, dk, dv = ha.backward(qd, kd, vd, out, lse, dod, seed=5, **args)
        torch.cuda.synchronize()
        rq, rk, rv = ob.backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), HAConfig(seed=5, **args))
        for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            got = got.cpu().numpy().astype(np.float64)
            scale = float(np.max(np.abs(ref))) or 1.0
            assert float(np.max(np.abs(got - ref))) <= 1e-4 * scale, (n, s, what)


RECT_CASES = [
    # B, H, Hkv, n_q, n_k, d, block, samples, r, seed
    (1, 2, 1, 1024, 1500, 64, 128, 64, 7, 41),     # more keys than queries, grouped heads
    (1, 2, 2, 1200, 700, 128, 64, 40, 6, 42),      # more queries than keys, d = 128
    (1, 1, 1, 777, 1000, 64, 96, 30, 5, 43),       # ragged blocks
]


@pytest.mark.parametrize("B,H,Hkv,nq,nk,d,block,m,r,seed", RECT_CASES)
def test_rect_backward_matches_oracle(B, H, Hkv, nq, nk, d, block, m, r, seed):
    g = torch.Generator(device="cpu").manual_seed(200 + seed)
    sc = d ** -0.25
    q = (torch.randn(B, H, nq, d, generator=g) * sc).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, nk, d, generator=g) * sc).to(torch.bfloat16)
    v = torch.randn(B, Hkv, nk, d, generator=g).to(torch.bfloat16)
    do = torch.randn(B, H, nq, d, generator=g).to(torch.bfloat16)
    args = dict(block=block, samples=m, proj_bits=r, seed=seed)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = ha.forward_rect(qd, kd, vd, **args)
    dq, dk, dv = ha.backward_rect(qd, kd, vd, out, lse, dod, **args)
    torch.cuda.synchronize()
    rq, rk, rv = ob.backward_rect(np32(q), np32(k), np32(v), np32(do), HAConfig(**args))
    _compare(dq.cpu().numpy(), rq, "dq")
    _compare(dk.cpu().numpy(), rk, "dk")
    _compare(dv.cpu().numpy(), rv, "dv")


@pytest.mark.slow
def test_backward_full_workload_noncausal():
    """The non-causal long131k pass (32 heads, n = 131072, d = 64, block 256,
    256 samples), the backward the benchmark times: dq, dk and dv of the
    first and last heads, every row, against the block-wise oracle (one KV
    head per query head here, so a KV head's dk, dv come from its one query
    head)."""
    w = WORKLOADS["long131k"]
    assert not w.causal and w.kv_heads == w.heads
    print("[backward long131k] generating inputs", flush=True)
    q, k, v = make_inputs(w, DEV)
    g = torch.Generator(device="cpu").manual_seed(77)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    args = w.method_args()
    out, lse = ha.forward(q, k, v, **args)
    dq, dk, dv = ha.backward(q, k, v, out, lse, do, **args)
    torch.cuda.synchronize()
    cfg = HAConfig(block=w.block, samples=w.samples, proj_bits=w.proj_bits, seed=w.seed)
    qc, kc, vc, dc = np32(q), np32(k), np32(v), np32(do)
    for h in (0, w.heads - 1):
        print(f"[backward long131k] oracle head {h}", flush=True)
        rq, rk, rv = ob.backward_head_blocks(qc, kc, vc, dc, cfg, 0, h)
        _compare(dq[0, h].cpu().numpy(), rq, f"dq head {h}")
        _compare(dk[0, h].cpu().numpy(), rk, f"dk head {h}")
        _compare(dv[0, h].cpu().numpy(), rv, f"dv head {h}")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["long131k_causal", "glm32k"])
def test_backward_full_workload_causal_dq_rows(name):
    """The causal passes the benchmark times: long131k (leaves of 4096 rows,
    five levels, d = 64) and glm32k (d = 128, 32 query heads on 2 KV heads,
    sink keys, three levels): dq of 50 rows of the first and last heads
    (leaf boundaries and both halves included) against the oracle's
    row-wise form, each row over its own leaf keys and quadrant keys, with
    D formed from the oracle's output rounded to bf16 (the backward is
    handed the forward's bf16 output; where attention sits on a few sink
    keys, dq is a small difference and the output's rounding in D shows:
    glm32k head 31 is 8.8e-3 from the fp64-output form, 4.2e-3 from this)."""
    w = WORKLOADS[name]
    assert w.causal
    print(f"[causal backward {name}] generating inputs", flush=True)
    q, k, v = make_inputs(w, DEV)
    g = torch.Generator(device="cpu").manual_seed(78)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    args = w.method_args()
    out, lse = ha.forward(q, k, v, **args)
    dq, _, _ = ha.backward(q, k, v, out, lse, do, **args)
    torch.cuda.synchronize()
    cfg = HAConfig(block=w.block, samples=w.samples, proj_bits=w.proj_bits, causal=True,
                   min_seq_len=w.min_seq_len, seed=w.seed)
    R = projections(w.seed, w.d, w.proj_bits)
    rows = np.array(sorted(set(np.random.default_rng(1).choice(w.n, 45, replace=False).tolist())
                           | {0, w.min_seq_len - 1, w.min_seq_len, w.n // 2, w.n - 1}))
    group = w.heads // w.kv_heads
    for h in (0, w.heads - 1):
        print(f"[causal backward {name}] oracle rows of head {h}", flush=True)
        qh, kh, vh = np32(q[0, h]), np32(k[0, h // group]), np32(v[0, h // group])
        ref = ob.causal_dq_rows(qh.astype(np.float64), kh.astype(np.float64), vh.astype(np.float64),
                                np32(do[0, h]).astype(np.float64), oh.ranks(qh, R), oh.ranks(kh, R), w.seed, 0, h,
                                cfg, rows, out_round=ob.round_bf16)
        _compare(dq[0, h].cpu().numpy()[rows], ref, f"dq head {h}")
