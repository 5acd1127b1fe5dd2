"""Error propagation on the GPU: HYPERATTN_FAIL_AT makes one stage's
launcher return HA_EHIP before it enqueues anything.  The call reports the
stage, outputs that no earlier stage writes keep their contents, and the
next call without the injection gives the normal result.  (Every kernel of
the earlier stages runs to completion: nothing faults or waits.)"""

import pytest
import torch

import approximate_long_context_amd as ha
from approximate_long_context_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

NC = Workload("err_nc", 1, 4, 2, 2048, 64, torch.bfloat16, 128, 64, 7, False, 0, "iid", 0, 41)
CA = Workload("err_c", 1, 2, 1, 2048, 64, torch.bfloat16, 128, 64, 7, True, 256, "iid", 0, 42)


def _sentinel_run(w, q, k, v):
    out = torch.full_like(q, 7.0)
    lse = torch.full(q.shape[:3], 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(ha.HyperAttnError) as e:
        ha.forward(q, k, v, out=out, lse=lse, **w.method_args())
    torch.cuda.synchronize()
    return e.value, out, lse


@pytest.mark.parametrize("w,stage,writes", [
    (NC, "proj", False), (NC, "hash", False), (NC, "sort", False), (NC, "samples", False), (NC, "attend", False),
    (CA, "proj", False), (CA, "hash", False), (CA, "leaf", False), (CA, "sort", True), (CA, "samples", True),
    (CA, "quadrant", True),
])
def test_injected_stage_failure(monkeypatch, w, stage, writes):
    """`writes`: an earlier stage (the causal leaves) has already written the
    rows that no recursion level touches, so only the error is checked."""
    print(f"[{w.name}] failing at {stage}", flush=True)
    q, k, v = (t.to(DEV) for t in make_inputs(w, "cpu"))
    monkeypatch.setenv("HYPERATTN_FAIL_AT", stage)
    err, out, lse = _sentinel_run(w, q, k, v)
    assert err.code == ha.HA_EHIP and f"before the {stage} launch" in str(err)
    if not writes:
        assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
    monkeypatch.delenv("HYPERATTN_FAIL_AT")
    ref, ref_lse = ha.forward(q, k, v, **w.method_args())
    again, again_lse = ha.forward(q, k, v, **w.method_args())
    torch.cuda.synchronize()
    assert torch.equal(ref, again) and torch.equal(ref_lse, again_lse)


def test_injected_backward_failure(monkeypatch):
    w = NC
    q, k, v = (t.to(DEV) for t in make_inputs(w, "cpu"))
    out, lse = ha.forward(q, k, v, **w.method_args())
    dout = torch.randn(q.shape, device=DEV).to(torch.bfloat16)
    args = w.method_args()
    args.pop("flags", None)
    for stage in ("bwd_dq", "bwd_dkv"):
        monkeypatch.setenv("HYPERATTN_FAIL_AT", stage)
        dq = torch.full(q.shape, 7.0, device=DEV)
        with pytest.raises(ha.HyperAttnError) as e:
            ha.backward(q, k, v, out, lse, dout, dq=dq, **args)
        torch.cuda.synchronize()
        assert e.value.code == ha.HA_EHIP and stage in str(e.value)
        if stage == "bwd_dq":
            assert bool((dq == 7.0).all())
    monkeypatch.delenv("HYPERATTN_FAIL_AT")
    dq1, dk1, dv1 = ha.backward(q, k, v, out, lse, dout, **args)
    torch.cuda.synchronize()
    assert torch.isfinite(dq1).all() and torch.isfinite(dk1).all()
