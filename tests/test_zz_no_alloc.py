"""The allocation-free forward (hyperattn_forward_noalloc) against the
workspace forward (hyperattn_forward), through the C ABI: the same kernels
on the same inputs, so outputs and lse must be identical bit for bit.
Two calls in a row share the library's scratch array, the second with a
smaller input, so the second runs over what the first left there."""

import ctypes

import pytest
import torch

import approximate_long_context_amd as ha
from approximate_long_context_amd.workloads import Workload, make_inputs

DEV = "cuda:0"

# (first call, second call with a smaller input)
PAIRS = [
    (Workload("na_nc_big", 2, 8, 2, 8192, 64, torch.bfloat16, 256, 256, 7, False, 0, "planted", 0, 11),
     Workload("na_nc_small", 1, 2, 1, 1000, 64, torch.bfloat16, 96, 64, 7, False, 0, "iid", 0, 12)),
    (Workload("na_c_big", 1, 4, 2, 4096, 128, torch.bfloat16, 128, 64, 7, True, 512, "sink", 0, 13),
     Workload("na_c_small", 1, 2, 2, 777, 64, torch.bfloat16, 64, 32, 7, True, 64, "iid", 0, 14)),
    (Workload("na_f32_big", 1, 2, 1, 2048, 128, torch.float32, 128, 64, 9, True, 256, "iid", 0, 15),
     Workload("na_f32_small", 1, 1, 1, 1024, 64, torch.float32, 64, 64, 7, False, 0, "iid", 0, 16)),
]


def _run_noalloc(w, q, k, v, with_lse=True):
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device) if with_lse else None
    args = w.method_args()
    args.pop("flags", None)
    ha.forward_noalloc(q, k, v, out, lse, **args)
    return out, lse


@pytest.mark.gpu
@pytest.mark.parametrize("pair", PAIRS, ids=[p[0].name for p in PAIRS])
def test_noalloc_equals_workspace_forward(pair):
    inputs = [tuple(t.to(DEV) for t in make_inputs(w, "cpu")) for w in pair]
    print("noalloc case", [w.name for w in pair], flush=True)
    for w in pair:
        need = ha.workspace_bytes(w.batch, w.n, w.d, w.heads, w.kv_heads, w.block, w.samples, w.proj_bits,
                                  w.causal, w.min_seq_len, w.dtype)
        assert 0 < need <= ha.NOALLOC_SCRATCH_BYTES, (w.name, need)
    got = [_run_noalloc(w, *x) for w, x in zip(pair, inputs)]     # big, then small
    torch.cuda.synchronize()
    for w, (q, k, v), (out, lse) in zip(pair, inputs, got):
        ref_out, ref_lse = ha.forward(q, k, v, **w.method_args())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16 if w.dtype == torch.bfloat16 else torch.int32),
                           ref_out.view(torch.int16 if w.dtype == torch.bfloat16 else torch.int32)), w.name
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), w.name


@pytest.mark.gpu
def test_noalloc_null_lse_and_repeat():
    w = PAIRS[0][1]
    q, k, v = (t.to(DEV) for t in make_inputs(w, "cpu"))
    a, _ = _run_noalloc(w, q, k, v, with_lse=False)
    b, lse = _run_noalloc(w, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.isfinite(lse).all()


@pytest.mark.gpu
def test_noalloc_refuses_oversized_before_launch():
    # the causal n = 131072, 32-head forward needs a 1.1 GB accumulator
    need = ha.workspace_bytes(1, 131072, 64, 32, 32, 256, 256, 7, True, 4096)
    assert need > ha.NOALLOC_SCRATCH_BYTES
    dummy = ctypes.c_void_p(256)          # never dereferenced: the size check comes first
    code = ha.lib().hyperattn_forward_noalloc(dummy, dummy, dummy, ha.HA_BF16, 1, 131072, 64, 32, 32, 256, 256, 7,
                                              1, 4096, ctypes.c_uint64(0), dummy, None, None)
    assert code == ha.HA_EWORKSPACE
    assert "scratch" in ha.lib().hyperattn_last_error().decode()
