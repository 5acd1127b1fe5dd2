"""GPU parity of the whole forward (hyperattn_forward through the C ABI)
against the oracle.

Small problems are compared element by element in full; the named
full-size workloads (the sizes and launch configuration the benchmark
times) are compared on sampled rows that the oracle computes one by one,
plus bit-exact ranks and permutations over every row.
"""

import numpy as np
import pytest
import torch

import approximate_long_context_amd as ha
import oracle
from approximate_long_context_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle.hyperattn import HAConfig

from _util import compare, compare_lse, np32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cfg(w):
    return HAConfig(block=w.block, samples=w.samples, proj_bits=w.proj_bits, causal=w.causal,
                    min_seq_len=w.min_seq_len, seed=w.seed)


def _run(w, flags=0, q=None, k=None, v=None):
    if q is None:
        q, k, v = make_inputs(w, "cpu")
    out, lse = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), flags=flags, **w.method_args())
    torch.cuda.synchronize()
    return q, k, v, out, lse


SMALL = [
    WORKLOADS["small"],                                                       # fp32, d=64
    Workload("nc_bf16_d64", 2, 4, 2, 2048, 64, torch.bfloat16, 256, 128, 7, False, 0, "planted", 3, 11),
    Workload("nc_bf16_d128", 1, 3, 3, 1536, 128, torch.bfloat16, 128, 100, 8, False, 0, "iid", 9, 12),
    Workload("nc_ragged", 1, 2, 1, 1000, 64, torch.bfloat16, 40, 50, 6, False, 0, "iid", 1, 13),
    Workload("nc_fp32_d128", 1, 2, 1, 640, 128, torch.float32, 64, 32, 5, False, 0, "iid", 2, 14),
    Workload("nc_r12", 1, 2, 2, 1024, 64, torch.bfloat16, 128, 64, 12, False, 0, "iid", 4, 15),
    Workload("nc_nosamples", 1, 2, 2, 1024, 64, torch.bfloat16, 128, 0, 7, False, 0, "iid", 4, 16),
    Workload("nc_oneblock", 1, 1, 1, 512, 64, torch.bfloat16, 512, 64, 7, False, 0, "iid", 4, 17),
    Workload("c_bf16_d64", 1, 4, 2, 2048, 64, torch.bfloat16, 64, 64, 7, True, 256, "sink", 5, 18),
    Workload("c_bf16_d128", 1, 2, 1, 1024, 128, torch.bfloat16, 128, 32, 7, True, 128, "iid", 6, 19),
    Workload("c_ragged", 1, 2, 2, 1200, 64, torch.bfloat16, 50, 20, 5, True, 200, "iid", 7, 20),
    Workload("c_fp32", 1, 1, 1, 512, 64, torch.float32, 32, 16, 6, True, 64, "iid", 8, 21),
    Workload("c_leafonly", 1, 2, 1, 1000, 64, torch.bfloat16, 64, 16, 7, True, 1000, "iid", 9, 22),
    Workload("c_clusters", 1, 2, 2, 2048, 128, torch.bfloat16, 128, 128, 8, True, 512, "clusters", 10, 23),
    # ragged last block: n (or a quadrant) not a multiple of the block
    Workload("nc_lastblock", 1, 2, 1, 1000, 64, torch.bfloat16, 64, 48, 7, False, 0, "iid", 11, 24),
    Workload("nc_lastblock_d128", 1, 2, 2, 1500, 128, torch.bfloat16, 256, 64, 7, False, 0, "planted", 12, 25),
    Workload("c_lastblock", 1, 2, 1, 2048, 64, torch.bfloat16, 96, 32, 6, True, 256, "iid", 13, 26),
    # odd causal splits: node-by-node recursion with rectangular quadrants
    Workload("c_odd", 1, 2, 1, 1000, 64, torch.bfloat16, 64, 32, 6, True, 100, "iid", 14, 27),
    Workload("c_odd_d128", 1, 2, 2, 777, 128, torch.bfloat16, 128, 48, 7, True, 64, "sink", 15, 28),
    # the largest sample count fp32 at d = 128 accepts (its K/V tiles leave
    # the least LDS for the sample lists); bf16 d = 64 at the global cap
    Workload("nc_fp32_d128_maxsamples", 1, 1, 1, 1024, 128, torch.float32, 64, 1952, 6, False, 0, "iid", 16, 29),
    Workload("nc_maxsamples", 1, 2, 1, 1024, 64, torch.bfloat16, 128, 4096, 6, False, 0, "iid", 17, 30),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_forward_small_matches_oracle(w):
    q, k, v, out, lse = _run(w)
    ref_o, ref_l = oracle.forward(np32(q), np32(k), np32(v), _cfg(w))
    compare(np32(out), ref_o, w.dtype, w.name)
    compare_lse(np32(lse), ref_l, w.dtype, w.name)


@pytest.mark.parametrize("flags", [ha.HA_FLAG_MATERIALIZE, ha.HA_FLAG_UNFUSED,
                                   ha.HA_FLAG_MATERIALIZE | ha.HA_FLAG_UNFUSED])
@pytest.mark.parametrize("name", ["nc_bf16_d64", "nc_ragged", "nc_lastblock"])
def test_forward_variants_match_fused(flags, name):
    w = next(x for x in SMALL if x.name == name)
    q, k, v, out0, lse0 = _run(w)
    _, _, _, out1, lse1 = _run(w, flags, q, k, v)
    compare(np32(out1), np32(out0).astype(np.float64), w.dtype, f"flags={flags}")
    compare_lse(np32(lse1), np32(lse0), w.dtype, f"flags={flags}")
    if flags == ha.HA_FLAG_MATERIALIZE:
        assert torch.equal(out0, out1)   # same kernel, same arithmetic


def test_forward_deterministic():
    w = next(x for x in SMALL if x.name == "c_bf16_d64")
    q, k, v, out0, lse0 = _run(w)
    for _ in range(2):
        _, _, _, out1, lse1 = _run(w, 0, q, k, v)
        assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_forward_empty_and_lse_optional():
    w = WORKLOADS["small"].with_(n=0)
    q = torch.zeros(1, 1, 0, 64, device=DEV)
    out, lse = ha.forward(q, q, q, **w.method_args())
    assert out.shape == (1, 1, 0, 64)
    w = SMALL[1]
    q, k, v = make_inputs(w, DEV)
    out = torch.empty_like(q)
    rc = ha.lib().hyperattn_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), ha.HA_BF16, w.batch, w.n, w.d,
                                    w.heads, w.kv_heads, w.block, w.samples, w.proj_bits, 0, 0, w.seed,
                                    out.data_ptr(), None,
                                    torch.empty(ha.workspace_bytes(w.batch, w.n, w.d, w.heads, w.kv_heads,
                                                                   w.block, w.samples, w.proj_bits),
                                                dtype=torch.uint8, device=DEV).data_ptr(),
                                    1 << 40, None)
    torch.cuda.synchronize()
    assert rc == ha.HA_OK
    out2, _ = ha.forward(q, k, v, **w.method_args())
    assert torch.equal(out, out2)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 33])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_tiny_n(n, causal):
    """Heads of a few rows: one partial tile, blocks of the whole head,
    every sample inside the row's block (non-causal), odd splits down to
    leaves of one or two rows (causal, min_seq_len 1 and 2)."""
    for s in ((1, 2) if causal else (0,)):
        w = Workload(f"tiny_{n}", 1, 2, 1, n, 64, torch.bfloat16, 2, 3, 5, causal, s, "iid", 0, 40 + n)
        q, k, v, out, lse = _run(w)
        ref_o, ref_l = oracle.forward(np32(q), np32(k), np32(v), _cfg(w))
        compare(np32(out), ref_o, w.dtype, f"{w.name} s={s}")
        compare_lse(np32(lse), ref_l, w.dtype, f"{w.name} s={s}")


# ---------------------------------------------------------------------------
# Full-size workloads: sampled rows + bit-exact ranks/permutations
# ---------------------------------------------------------------------------

FULL = ["small", "c32k", "glm32k", "long131k", "long131k_causal", "stress512k"]


def _sample_rows(n, count, seed):
    g = np.random.default_rng(seed)
    rows = set(g.choice(n, size=count, replace=False).tolist())
    rows |= {0, 1, n // 2 - 1, n // 2, n - 1}
    return np.array(sorted(rows))


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_workload_sampled_rows(name):
    w = WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    q, k, v = make_inputs(w, DEV)
    out, lse = ha.forward(q, k, v, **w.method_args())
    torch.cuda.synchronize()
    print(f"[{name}] forward done; checking ranks", flush=True)
    # ranks of every row, bit-exact (GPU hash vs the oracle's fp32 hash)
    R = ha.projections(w.seed, w.d, w.proj_bits, DEV)
    assert np.array_equal(R.cpu().numpy(), oracle.projections(w.seed, w.d, w.proj_bits))
    heads = [(0, h) for h in sorted({0, w.heads // 2, w.heads - 1})]
    G = w.heads // w.kv_heads
    for b, h in heads[:2]:
        rq = ha.hash_rows(q[b, h].contiguous(), R).cpu().numpy()
        assert np.array_equal(rq.astype(np.uint32), oracle.ranks(np32(q[b, h]), R.cpu().numpy()))
        if not w.causal:
            perm = ha.sort_ranks(ha.hash_rows(q[b, h:h + 1].contiguous(), R), w.proj_bits).cpu().numpy()[0, 0]
            assert np.array_equal(perm, oracle.sort_perm(rq))
    rows = _sample_rows(w.n, 48 if w.n > 100000 else 96, sum(map(ord, name)))
    qc, kc, vc = np32(q), np32(k), np32(v)
    ref_o = np.zeros((len(heads), len(rows), w.d))
    ref_l = np.zeros((len(heads), len(rows)))
    for i, bh in enumerate(heads):
        print(f"[{name}] oracle rows of head {bh}", flush=True)
        o1, l1 = oracle.forward_rows(qc, kc, vc, _cfg(w), heads=[bh], rows=rows)
        ref_o[i], ref_l[i] = o1[0], l1[0]
    for i, (b, h) in enumerate(heads):
        got = np32(out[b, h])[rows]
        compare(got, ref_o[i], w.dtype, f"{name} head {h}")
        compare_lse(np32(lse[b, h])[rows], ref_l[i], w.dtype, f"{name} head {h}")
    assert torch.isfinite(out.float()).all()
    del G


@pytest.mark.slow
@pytest.mark.parametrize("name,heads", [("long131k", (0, 31)), ("long131k_causal", (0, 31)), ("stress512k", (0,)),
                                        ("c32k", (0, 31)), ("glm32k", (0, 31)), ("small", (0,))])
def test_full_workload_every_row(name, heads):
    """Whole heads at the benchmark's sizes and launch configuration: every
    row of the listed heads against the oracle (out and lse)."""
    w = WORKLOADS[name]
    print(f"[{name}] inputs and forward", flush=True)
    q, k, v = make_inputs(w, DEV)
    out, lse = ha.forward(q, k, v, **w.method_args())
    torch.cuda.synchronize()
    qc, kc, vc = np32(q), np32(k), np32(v)
    for h in heads:
        print(f"[{name}] oracle, every row of head {h}", flush=True)
        ref_o, ref_l = oracle.forward_rows(qc, kc, vc, _cfg(w), heads=[(0, h)])
        compare(np32(out[0, h]), ref_o[0], w.dtype, f"{name} head {h}")
        compare_lse(np32(lse[0, h]), ref_l[0], w.dtype, f"{name} head {h}")
