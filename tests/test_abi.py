"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/hyperattn.h, its host projection routine equals
the oracle bit for bit, and invalid arguments return the documented codes
before anything is enqueued (null device pointers are passed: a call that
got past validation would fail differently)."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import approximate_long_context_amd as ha
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "hyperattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hyperattn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 15
    lib = ha.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert ha.version().startswith("hyperattn")


@pytest.mark.parametrize("d,r", [(64, 7), (128, 8), (64, 16), (128, 1), (8, 3), (100, 5)])
def test_host_projections_equal_oracle(d, r):
    for seed in list(range(25)) + [2**63 + 12345, 2**64 - 1]:
        got = ha.projections_host(seed, d, r).numpy()
        assert np.array_equal(got, oracle.projections(seed, d, r)), (seed, d, r)


def _fwd(**kw):
    args = dict(q=None, k=None, v=None, dtype=ha.HA_BF16, batch=1, n=1024, d=64, heads=4, kv_heads=2,
                block=64, samples=16, proj_bits=7, causal=0, min_seq_len=0, seed=0, flags=0,
                out=None, lse=None, ws=None, wsb=1 << 30, stream=None)
    args.update(kw)
    a = args
    return ha.lib().hyperattn_forward_ex(a["q"], a["k"], a["v"], a["dtype"], a["batch"], a["n"], a["d"],
                                         a["heads"], a["kv_heads"], a["block"], a["samples"],
                                         a["proj_bits"], a["causal"], a["min_seq_len"], a["seed"],
                                         a["flags"], a["out"], a["lse"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), ha.HA_EINVAL),
    (dict(heads=3, kv_heads=2), ha.HA_EINVAL),
    (dict(kv_heads=0), ha.HA_EINVAL),
    (dict(block=0), ha.HA_EINVAL),
    (dict(samples=-1), ha.HA_EINVAL),
    (dict(proj_bits=0), ha.HA_EINVAL),
    (dict(proj_bits=17), ha.HA_EINVAL),
    (dict(n=-5), ha.HA_EINVAL),
    (dict(d=96), ha.HA_EUNSUPPORTED),
    (dict(causal=1, min_seq_len=0), ha.HA_EINVAL),
    (dict(causal=1, min_seq_len=128, flags=1), ha.HA_EUNSUPPORTED),
    (dict(flags=8), ha.HA_EINVAL),
    (dict(samples=5000), ha.HA_EUNSUPPORTED),
    (dict(), ha.HA_EINVAL),                    # null q/k/v/out
])
def test_forward_argument_errors(kw, code):
    assert _fwd(**kw) == code
    assert ha.lib().hyperattn_last_error().decode() != ""


def test_forward_workspace_error_and_empty():
    dummy = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    assert _fwd(q=dummy, k=dummy, v=dummy, out=dummy, ws=dummy, wsb=16) == ha.HA_EWORKSPACE
    assert _fwd(q=dummy, k=dummy, v=dummy, out=dummy, ws=None, wsb=0) == ha.HA_EWORKSPACE
    assert _fwd(n=0) == ha.HA_OK
    assert _fwd(batch=0) == ha.HA_OK


def test_workspace_bytes():
    nb = ha.workspace_bytes(1, 131072, 64, 32, 32, 256, 256, 7)
    cb = ha.workspace_bytes(1, 131072, 64, 32, 32, 256, 256, 7, True, 4096)
    assert nb > 32 * 131072 * 12 and cb > 32 * 131072 * 64 * 4
    assert ha.workspace_bytes(1, 1000, 64, 1, 1, 64, 4, 7, True, 100) > 0       # odd causal splits
    assert ha.workspace_bytes(1, 1000, 64, 1, 1, 64, 4, 7) > 0                  # ragged last block
    assert ha.workspace_bytes(1, 1000, 64, 1, 1, 64, 4, 7, True, 0) == 0        # min_seq_len < 1
    big = ha.workspace_bytes(1, 4096, 64, 2, 2, 64, 4, 7, flags=ha.HA_FLAG_MATERIALIZE | ha.HA_FLAG_UNFUSED)
    assert big > ha.workspace_bytes(1, 4096, 64, 2, 2, 64, 4, 7) + 3 * 2 * 4096 * 64 * 2


def test_stage_argument_errors():
    L = ha.lib()
    assert L.hyperattn_projections_host(0, 64, 0, None) == ha.HA_EINVAL
    assert L.hyperattn_hash(None, ha.HA_BF16, 10, 64, 7, None, None, None) == ha.HA_EINVAL
    assert L.hyperattn_hash(ctypes.c_void_p(256), ha.HA_BF16, 10, 96, 7, ctypes.c_void_p(256),
                            ctypes.c_void_p(256), None) == ha.HA_EUNSUPPORTED
    assert L.hyperattn_sort(None, 2, 100, 60, 50, 60, 1, 7, None, None, 0, None) == ha.HA_EINVAL
    assert L.hyperattn_sample_indices(0, 1, 1, 1, 1, 0, 4, None, None) == ha.HA_EINVAL
    assert L.hyperattn_gather(None, ha.HA_BF16, 1, 10, 64, None, 10, None, None) == ha.HA_EINVAL
    assert L.hyperattn_causal_leaves(None, None, None, ha.HA_BF16, 1, 100, 64, 1, 1, 30, None, None,
                                     None) == ha.HA_ESHAPE
    assert L.hyperattn_merge_unsort(None, None, None, None, None, 1, 10, 64, ha.HA_BF16, None, None,
                                    None) == ha.HA_EINVAL
    assert L.hyperattn_attend(None, None, None, ha.HA_BF16, 1, 64, 64, 1, 1, 64, 4, None, None, None, 4,
                              None, None, None) == ha.HA_EINVAL


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(ha, "_lib", None)
    monkeypatch.setattr(ha, "LIB_PATH", "/nonexistent/libhyperattn.so")
    with pytest.raises(RuntimeError):
        ha.lib()


def test_rownorm_workspace_holds_no_partials():
    """The row-norm variant adds per-key weights and CDF (12 bytes a key),
    a workspace lse (4 bytes a query row) and the compact drawn rows; no
    fp32 [heads][n][d] partial and no full sorted copy."""
    B, n, d, H, Hkv, b, m, r = 1, 131072, 64, 32, 32, 256, 256, 7
    plain = ha.workspace_bytes(B, n, d, H, Hkv, b, m, r)
    rn = ha.workspace_bytes(B, n, d, H, Hkv, b, m, r, flags=ha.HA_FLAG_ROWNORM)
    extra = Hkv * n * 12 + H * n * 4 + 2 * H * m * d * 2 + H * m * 4 + (1 << 20)
    assert plain < rn <= plain + extra
    assert rn < plain + H * n * d * 2          # less than one bf16 copy of the queries


def test_sample_cap_follows_lds():
    """Sample lists live in LDS beside the K/V tiles: fp32 at d = 128 takes
    at most 1952 samples, the other builds 4096; larger counts are refused
    before any pointer is touched."""
    for dt, d, cap in ((torch.float32, 128, 1952), (torch.float32, 64, 4096), (torch.bfloat16, 128, 4096),
                       (torch.bfloat16, 64, 4096)):
        assert ha.workspace_bytes(1, 4096, d, 2, 2, 64, cap, 7, dtype=dt) > 0
        assert ha.workspace_bytes(1, 4096, d, 2, 2, 64, cap + 1, 7, dtype=dt) == 0
    L = ha.lib()
    rc = L.hyperattn_forward(None, None, None, ha.HA_F32, 1, 4096, 128, 2, 2, 64, 1953, 7, 0, 0,
                             ctypes.c_uint64(0), None, None, None, 0, None)
    assert rc == ha.HA_EUNSUPPORTED and b"LDS" in L.hyperattn_last_error()


def test_causal_rownorm_workspace():
    """Causal row-norm: per-key weights and CDF, an lse per query row and
    the drawn rows of the widest level (16 pieces at n = 131072 with
    min_seq_len 4096); the other flags stay non-causal only; no samples,
    no extra buffers."""
    B, n, d, H, Hkv, b, m, r, s = 1, 131072, 64, 32, 32, 256, 256, 7, 4096
    plain = ha.workspace_bytes(B, n, d, H, Hkv, b, m, r, causal=True, min_seq_len=s)
    rn = ha.workspace_bytes(B, n, d, H, Hkv, b, m, r, causal=True, min_seq_len=s, flags=ha.HA_FLAG_ROWNORM)
    pieces = 16
    extra = Hkv * n * 4 + Hkv * n // 2 * 8 + H * n * 4 + pieces * H * m * (4 + 2 * d * 2) + (1 << 20)
    assert plain < rn <= plain + extra
    for odd_n in (131071, 1000):
        assert ha.workspace_bytes(B, odd_n, d, H, Hkv, b, m, r, causal=True, min_seq_len=100,
                                  flags=ha.HA_FLAG_ROWNORM) > 0
    assert ha.workspace_bytes(B, n, d, H, Hkv, b, 0, r, causal=True, min_seq_len=s,
                              flags=ha.HA_FLAG_ROWNORM) == ha.workspace_bytes(B, n, d, H, Hkv, b, 0, r, causal=True,
                                                                              min_seq_len=s)
    for f in (ha.HA_FLAG_MATERIALIZE, ha.HA_FLAG_UNFUSED, ha.HA_FLAG_ROWNORM | ha.HA_FLAG_UNFUSED):
        assert ha.workspace_bytes(B, n, d, H, Hkv, b, m, r, causal=True, min_seq_len=s, flags=f) == 0


def test_forward_noalloc_argument_errors():
    """Errors of the allocation-free forward come before the scratch
    array's address is looked up and before any launch."""
    L = ha.lib()
    dummy = ctypes.c_void_p(256)   # never dereferenced

    def call(q=dummy, n=131072, causal=1, dtype=ha.HA_BF16, heads=32, d=64):
        return L.hyperattn_forward_noalloc(q, dummy, dummy, dtype, 1, n, d, heads, 32 if heads == 32 else 1, 256,
                                           256, 7, causal, 4096, ctypes.c_uint64(0), dummy, None, None)
    assert call(n=0) == ha.HA_OK
    assert call(q=None) == ha.HA_EINVAL
    assert call(dtype=5) == ha.HA_EINVAL
    assert call(d=96) == ha.HA_EUNSUPPORTED
    assert call() == ha.HA_EWORKSPACE                 # 1.1 GB causal accumulator > scratch array
    assert "scratch" in L.hyperattn_last_error().decode()
    assert ha.workspace_bytes(1, 131072, 64, 32, 32, 256, 256, 7) <= ha.NOALLOC_SCRATCH_BYTES


def test_forward_debug_argument_errors():
    """A null dump or an o/lse pair with one pointer missing is refused
    before anything is enqueued; hyperattn_debug_levels counts levels."""
    L = ha.lib()
    dummy = ctypes.c_void_p(256)
    st = ha.DebugDump()

    def call(dump):
        return L.hyperattn_forward_debug(dummy, dummy, dummy, ha.HA_BF16, 1, 2048, 64, 4, 2, 96, 48, 7, 1, 256,
                                         ctypes.c_uint64(0), dummy, dummy, dummy, 1 << 30, None, dump)
    assert call(None) == ha.HA_EINVAL
    st.o_blk = 256
    assert call(ctypes.byref(st)) == ha.HA_EINVAL
    st = ha.DebugDump()
    st.lse_leaf = 256
    assert call(ctypes.byref(st)) == ha.HA_EINVAL
    st = ha.DebugDump()
    assert L.hyperattn_forward_debug(dummy, dummy, dummy, ha.HA_BF16, 1, 2048, 96, 4, 2, 96, 48, 7, 1, 256,
                                     ctypes.c_uint64(0), dummy, dummy, dummy, 1 << 30, None,
                                     ctypes.byref(st)) == ha.HA_EUNSUPPORTED
    for n, causal, s, levels in [(2048, 1, 256, 3), (1000, 1, 100, 4), (131072, 1, 4096, 5), (4096, 1, 4096, 0),
                                 (4097, 1, 4096, 1), (777, 0, 0, 1), (0, 1, 5, 0), (10, 1, 0, -1), (-1, 0, 0, -1)]:
        assert ha.debug_levels(n, causal, s) == levels, (n, causal, s)
        if causal and n > 0 and s > 0:
            assert levels == oracle.causal_levels(n, s)


@pytest.mark.parametrize("causal,n,s", [(0, 1024, 0), (1, 2048, 256), (1, 1000, 100)])
def test_injected_failure_before_first_launch(monkeypatch, causal, n, s):
    """HYPERATTN_FAIL_AT=proj stops the forward and the backward at their first
    launcher with HA_EHIP and a message naming the stage; the host planning
    before it runs in full (dummy device pointers are never dereferenced)."""
    monkeypatch.setenv("HYPERATTN_FAIL_AT", "proj")
    L = ha.lib()
    dummy = ctypes.c_void_p(256)
    rc = L.hyperattn_forward_ex(dummy, dummy, dummy, ha.HA_BF16, 1, n, 64, 4, 2, 96, 16, 7, causal, s,
                                ctypes.c_uint64(0), 0, dummy, dummy, dummy, 1 << 40, None)
    assert rc == ha.HA_EHIP
    assert "injected failure before the proj launch" in L.hyperattn_last_error().decode()
    rc = L.hyperattn_backward(dummy, dummy, dummy, dummy, dummy, dummy, ha.HA_BF16, 1, n, 64, 4, 2, 96, 16, 7,
                              causal, s, ctypes.c_uint64(0), dummy, dummy, dummy, dummy, 1 << 40, None)
    assert rc == ha.HA_EHIP
    monkeypatch.setenv("HYPERATTN_FAIL_AT", "nothing")
    assert L.hyperattn_forward_ex(None, None, None, ha.HA_BF16, 1, n, 64, 4, 2, 96, 16, 7, causal, s,
                                  ctypes.c_uint64(0), 0, None, None, None, 0, None) == ha.HA_EINVAL


def test_backward_group_sample_limit():
    """The backward sorts a KV group's sample slots in LDS: (heads / kv_heads)
    * samples above 8192 is refused before any launch."""
    L = ha.lib()
    dummy = ctypes.c_void_p(256)
    rc = L.hyperattn_backward(dummy, dummy, dummy, dummy, dummy, dummy, ha.HA_BF16, 1, 4096, 64, 32, 1, 128, 512,
                              7, 0, 0, ctypes.c_uint64(0), dummy, dummy, dummy, dummy, 1 << 40, None)
    assert rc == ha.HA_EUNSUPPORTED and "8192" in L.hyperattn_last_error().decode()
