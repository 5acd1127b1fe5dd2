"""MI355X (gfx950) HyperAttention forward and backward: Python binding of libhyperattn.so.

Argument marshalling only: every step of the method runs in the HIP
kernels behind the C ABI declared in ``include/hyperattn.h``.  PyTorch
provides device memory and the current stream.  If the library is not
built this module raises on first use; there is no fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhyperattn.so")

HA_BF16, HA_F32 = 0, 1
HA_FLAG_MATERIALIZE, HA_FLAG_UNFUSED, HA_FLAG_ROWNORM = 1, 2, 4
HA_OK, HA_EINVAL, HA_EUNSUPPORTED, HA_EWORKSPACE, HA_ESHAPE, HA_EHIP = 0, -1, -2, -3, -4, -5
KERNEL_CLASSES = ["proj", "hash", "sort", "samples", "gather", "attend", "merge", "leaf", "quadrant",
                  "bwd_dq", "bwd_dkv"]

_c_int, _c_i64, _c_u64, _c_size, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "hyperattn_last_error": (ctypes.c_char_p, []),
    "hyperattn_version": (ctypes.c_char_p, []),
    "hyperattn_workspace_bytes": (_c_size, [_c_int] * 12),
    "hyperattn_forward": (_c_int, [_vp, _vp, _vp, _c_int] + [_c_int] * 10 + [_c_u64, _vp, _vp, _vp, _c_size, _vp]),
    "hyperattn_forward_ex": (_c_int, [_vp, _vp, _vp, _c_int] + [_c_int] * 10 + [_c_u64, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "hyperattn_forward_noalloc": (_c_int, [_vp, _vp, _vp, _c_int] + [_c_int] * 10 + [_c_u64, _vp, _vp, _vp]),
    "hyperattn_debug_levels": (_c_int, [_c_int] * 3),
    "hyperattn_forward_debug": (_c_int, [_vp, _vp, _vp, _c_int] + [_c_int] * 10 + [_c_u64, _vp, _vp, _vp, _c_size, _vp, _vp]),
    "hyperattn_backward_workspace_bytes": (_c_size, [_c_int] * 11),
    "hyperattn_backward": (_c_int, [_vp] * 6 + [_c_int] * 11 + [_c_u64, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "hyperattn_backward_rect_workspace_bytes": (_c_size, [_c_int] * 10),
    "hyperattn_backward_rect": (_c_int, [_vp] * 6 + [_c_int] * 10 + [_c_u64, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "hyperattn_projections_host": (_c_int, [_c_u64, _c_int, _c_int, _vp]),
    "hyperattn_projections": (_c_int, [_c_u64, _c_int, _c_int, _vp, _vp]),
    "hyperattn_hash": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _vp]),
    "hyperattn_sort_workspace_bytes": (_c_size, [_c_i64, _c_int, _c_int, _c_int]),
    "hyperattn_sort": (_c_int, [_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "hyperattn_sample_indices": (_c_int, [_c_u64, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "hyperattn_gather": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_int, _vp, _c_int, _vp, _vp]),
    "hyperattn_attend": (_c_int, [_vp, _vp, _vp, _c_int] + [_c_int] * 7 + [_vp, _vp, _vp, _c_int, _vp, _vp, _vp]),
    "hyperattn_merge_unsort": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "hyperattn_causal_leaves": (_c_int, [_vp, _vp, _vp, _c_int] + [_c_int] * 6 + [_vp, _vp, _vp]),
    "hyperattn_row_sqnorms": (_c_int, [_vp, _c_int, _c_i64, _c_int, _vp, _vp]),
    "hyperattn_rownorm_samples_workspace_bytes": (_c_size, [_c_int] * 3),
    "hyperattn_rownorm_samples": (_c_int, [_vp, _vp] + [_c_int] * 5 + [_c_u64, _vp, _vp, _vp, _c_size, _vp]),
    "hyperattn_column_sqmass": (_c_int, [_vp, _vp, _vp] + [_c_int] * 8 + [_vp, _vp, _vp]),
    "hyperattn_residual_ratio": (_c_int, [_vp, _vp, _vp, _c_i64, _c_int, _vp, _vp]),
    "hyperattn_rect_workspace_bytes": (_c_size, [_c_int] * 10),
    "hyperattn_forward_rect": (_c_int, [_vp, _vp, _vp] + [_c_int] * 10 + [_c_u64, _vp, _vp, _vp, _c_size, _vp]),
    "hyperattn_timing_enable": (_c_int, [_c_int]),
    "hyperattn_timing_read": (_c_int, [_vp, _vp]),
}

_lib = None


class HyperAttnError(RuntimeError):
    def __init__(self, func, code, msg):
        super().__init__(f"{func} returned {code}: {msg}")
        self.code = code


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m approximate_long_context_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(name, code):
    if code != HA_OK:
        raise HyperAttnError(name, code, lib().hyperattn_last_error().decode())


def _call(name, *args):
    _check(name, getattr(lib(), name)(*args))


def _dtype_code(t):
    if t == torch.bfloat16:
        return HA_BF16
    if t == torch.float32:
        return HA_F32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def version():
    return lib().hyperattn_version().decode()


def workspace_bytes(batch, n, d, heads, kv_heads, block, samples, proj_bits, causal=False,
                    min_seq_len=0, dtype=torch.bfloat16, flags=0):
    return lib().hyperattn_workspace_bytes(batch, n, d, heads, kv_heads, block, samples, proj_bits,
                                           int(bool(causal)), min_seq_len, _dtype_code(dtype), flags)


def forward(q, k, v, *, block, samples, proj_bits, causal=False, min_seq_len=0, seed=0,
            flags=0, out=None, lse=None, workspace=None):
    """HyperAttention forward.  q [B, H, n, d], k, v [B, Hkv, n, d] (bf16 or
    fp32, contiguous, same device).  Returns (out, lse): out like q, lse
    float32 [B, H, n] (natural log of the estimated normaliser)."""
    _need(q, "q")
    dev = q.device
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, n, d] and k, v [B, Hkv, n, d]")
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != n or k.shape[3] != d:
        raise ValueError("k, v must match q in batch, length and head dim")
    dt = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    _need(out, "out", q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    wsb = lib().hyperattn_workspace_bytes(B, n, d, H, Hkv, block, samples, proj_bits,
                                          int(bool(causal)), min_seq_len, dt, flags)
    if wsb == 0 and n > 0 and B > 0 and H > 0:
        # invalid shape: let forward report the precise error
        wsb = 256
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _call("hyperattn_forward_ex", _ptr(q), _ptr(k), _ptr(v), dt, B, n, d, H, Hkv, block, samples,
          proj_bits, int(bool(causal)), min_seq_len, ctypes.c_uint64(seed), flags, _ptr(out),
          _ptr(lse), _ptr(workspace), workspace.numel(), _stream(dev))
    return out, lse


class DebugDump(ctypes.Structure):
    """ha_debug_dump: optional device pointers of hyperattn_forward_debug."""
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("perm_q", "perm_k", "idx", "o_blk", "lse_blk", "o_smp", "lse_smp", "o_leaf", "lse_leaf")]


def debug_levels(n, causal=False, min_seq_len=0):
    """Levels of sorted problems of a forward (hyperattn_debug_levels)."""
    return lib().hyperattn_debug_levels(n, int(bool(causal)), min_seq_len)


def forward_debug(q, k, v, *, block, samples, proj_bits, causal=False, min_seq_len=0, seed=0,
                  want=("perm_q", "perm_k", "idx", "blk", "smp", "leaf")):
    """hyperattn_forward_debug: the forward plus its intermediates.  Returns
    (out, lse, dump) with dump a dict of the requested buffers, shaped as
    include/hyperattn.h states (L levels, P = 2^(L-1) node slots per level):
    perm_q [L, B*H, n], perm_k [L, B*Hkv, n], idx [L, B*H, P, m] (int32,
    filled with -1 where not written), o_blk / o_smp [L, B*H, n, d] and
    lse_blk / lse_smp [L, B*H, n] (float32, NaN where not written), o_leaf
    [B*H, n, d] and lse_leaf [B*H, n] (causal)."""
    _need(q, "q")
    dev = q.device
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    L = debug_levels(n, causal, min_seq_len)
    if L < 0:
        raise ValueError("bad n or min_seq_len")
    P = 1 << max(L - 1, 0)
    BH, BK = B * H, B * Hkv
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dump, st = {}, DebugDump()
    if "perm_q" in want:
        dump["perm_q"] = torch.full((L, BH, n), -1, **i32)
    if "perm_k" in want:
        dump["perm_k"] = torch.full((L, BK, n), -1, **i32)
    if "idx" in want:
        dump["idx"] = torch.full((L, BH, P, samples), -1, **i32)
    for part in ("blk", "smp"):
        if part in want:
            dump["o_" + part] = torch.full((L, BH, n, d), float("nan"), **f32)
            dump["lse_" + part] = torch.full((L, BH, n), float("nan"), **f32)
    if "leaf" in want and causal:
        dump["o_leaf"] = torch.full((BH, n, d), float("nan"), **f32)
        dump["lse_leaf"] = torch.full((BH, n), float("nan"), **f32)
    for name, t in dump.items():
        if t.numel():
            setattr(st, name, t.data_ptr())
    dt = _dtype_code(q.dtype)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, n), **f32)
    wsb = lib().hyperattn_workspace_bytes(B, n, d, H, Hkv, block, samples, proj_bits, int(bool(causal)),
                                          min_seq_len, dt, 0)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _call("hyperattn_forward_debug", _ptr(q), _ptr(k), _ptr(v), dt, B, n, d, H, Hkv, block, samples, proj_bits,
          int(bool(causal)), min_seq_len, ctypes.c_uint64(seed), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
          _stream(dev), ctypes.byref(st))
    return out, lse, dump


NOALLOC_SCRATCH_BYTES = 64 << 20     # HA_NOALLOC_SCRATCH_BYTES


def forward_noalloc(q, k, v, out, lse, *, block, samples, proj_bits, causal=False, min_seq_len=0, seed=0):
    """hyperattn_forward_noalloc: the forward with the library's own device
    scratch array as workspace (allocates nothing).  q [B, H, n, d], k, v
    [B, Hkv, n, d]; out (like q) and lse (float32 [B, H, n] or None) are
    the caller's.  Returns (out, lse)."""
    _need(q, "q")
    dev = q.device
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    _need(out, "out", q.dtype, dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or out.shape != q.shape:
        raise ValueError("q, out must be [B, H, n, d] and k, v [B, Hkv, n, d]")
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != n or k.shape[3] != d:
        raise ValueError("k, v must match q in batch, length and head dim")
    if lse is not None and tuple(lse.shape) != (B, H, n):
        raise ValueError("lse must be [B, H, n]")
    _call("hyperattn_forward_noalloc", _ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), B, n, d, H, Hkv, block,
          samples, proj_bits, int(bool(causal)), min_seq_len, ctypes.c_uint64(seed), _ptr(out), _ptr(lse),
          _stream(dev))
    return out, lse


def forward_rect(q, k, v, *, block, samples, proj_bits, seed=0, out=None, lse=None, workspace=None):
    """Non-causal forward of a rectangular problem: q [B, H, n_q, d], k, v
    [B, Hkv, n_k, d] (bf16 or fp32).  Returns (out like q, lse [B, H, n_q])."""
    _need(q, "q")
    dev = q.device
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, H, n_q, d] and k, v [B, Hkv, n_k, d]")
    B, H, nq, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    dt = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    wsb = lib().hyperattn_rect_workspace_bytes(B, nq, nk, d, H, Hkv, block, samples, proj_bits, dt)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _call("hyperattn_forward_rect", _ptr(q), _ptr(k), _ptr(v), dt, B, nq, nk, d, H, Hkv, block, samples, proj_bits,
          ctypes.c_uint64(seed), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(dev))
    return out, lse


def backward_workspace_bytes(batch, n, d, heads, kv_heads, block, samples, proj_bits, causal=False,
                             min_seq_len=0, dtype=torch.bfloat16):
    return lib().hyperattn_backward_workspace_bytes(batch, n, d, heads, kv_heads, block, samples, proj_bits,
                                                    int(bool(causal)), min_seq_len, _dtype_code(dtype))


def backward(q, k, v, out, lse, dout, *, block, samples, proj_bits, causal=False, min_seq_len=0,
             seed=0, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of sum(dout * out) for (out, lse) = forward(q, k, v, ...)
    with the same arguments.  bf16 or fp32 inputs (all of one dtype);
    returns float32 (dq like q, dk and dv like k)."""
    _need(q, "q")
    dev = q.device
    dt = _dtype_code(q.dtype)
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, name, q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, out, dout must be [B, H, n, d] and k, v [B, Hkv, n, d]")
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if lse.shape != (B, H, n):
        raise ValueError("lse must be [B, H, n]")
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty(k.shape, dtype=torch.float32, device=dev)
    for t, name, shp in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _need(t, name, torch.float32, dev)
        if t.shape != shp:
            raise ValueError(f"{name} must have shape {tuple(shp)}")
    wsb = lib().hyperattn_backward_workspace_bytes(B, n, d, H, Hkv, block, samples, proj_bits,
                                                   int(bool(causal)), min_seq_len, dt)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _call("hyperattn_backward", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), dt,
          B, n, d, H, Hkv, block, samples, proj_bits, int(bool(causal)), min_seq_len, ctypes.c_uint64(seed),
          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(dev))
    return dq, dk, dv


def backward_rect(q, k, v, out, lse, dout, *, block, samples, proj_bits, seed=0, dq=None, dk=None, dv=None,
                  workspace=None):
    """Gradients of sum(dout * out) for (out, lse) = forward_rect(q, k, v, ...)
    with the same arguments: q, out, dout [B, H, n_q, d], k, v [B, Hkv, n_k, d]
    (bf16 or fp32, one dtype), lse [B, H, n_q]; returns float32 (dq like q,
    dk and dv like k)."""
    _need(q, "q")
    dev = q.device
    dt = _dtype_code(q.dtype)
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, name, q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    if (q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or out.shape != q.shape or dout.shape != q.shape
            or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]):
        raise ValueError("q, out, dout must be [B, H, n_q, d] and k, v [B, Hkv, n_k, d]")
    B, H, nq, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    if lse.shape != (B, H, nq):
        raise ValueError("lse must be [B, H, n_q]")
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty(k.shape, dtype=torch.float32, device=dev) if dv is None else dv
    for t, name, shp in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _need(t, name, torch.float32, dev)
        if t.shape != shp:
            raise ValueError(f"{name} must have shape {tuple(shp)}")
    wsb = lib().hyperattn_backward_rect_workspace_bytes(B, nq, nk, d, H, Hkv, block, samples, proj_bits, dt)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _call("hyperattn_backward_rect", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), dt,
          B, nq, nk, d, H, Hkv, block, samples, proj_bits, ctypes.c_uint64(seed),
          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(dev))
    return dq, dk, dv


# ---- stage entry points ------------------------------------------------------

def projections_host(seed, d, proj_bits):
    out = torch.empty((proj_bits, d), dtype=torch.float32)
    _call("hyperattn_projections_host", ctypes.c_uint64(seed), d, proj_bits, _ptr(out))
    return out


def projections(seed, d, proj_bits, device="cuda"):
    out = torch.empty((proj_bits, d), dtype=torch.float32, device=device)
    _call("hyperattn_projections", ctypes.c_uint64(seed), d, proj_bits, _ptr(out), _stream(out.device))
    return out


def hash_rows(x, R):
    """uint16 bucket ranks of the rows of x ([..., d]) under projections R ([r, d])."""
    _need(x, "x")
    _need(R, "R", torch.float32, x.device)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    rank = torch.empty(x.shape[:-1], dtype=torch.uint16, device=x.device)
    _call("hyperattn_hash", _ptr(x), _dtype_code(x.dtype), rows, d, R.shape[0], _ptr(R), _ptr(rank),
          _stream(x.device))
    return rank


def sort_ranks(rank, proj_bits, length=None, first=0, stride=None, pieces=1):
    """Stable segmented sort of rank [heads, n] (uint16); returns int32
    [heads, pieces, length] row indices."""
    _need(rank, "rank", torch.uint16)
    heads, n = rank.shape
    length = n if length is None else length
    stride = length if stride is None else stride
    perm = torch.empty((heads, pieces, length), dtype=torch.int32, device=rank.device)
    wsb = lib().hyperattn_sort_workspace_bytes(heads, length, pieces, proj_bits)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=rank.device)
    _call("hyperattn_sort", _ptr(rank), heads, n, length, first, stride, pieces, proj_bits, _ptr(perm),
          _ptr(ws), ws.numel(), _stream(rank.device))
    return perm


def sample_indices(seed, batch, heads, ns, samples, node_first=1, node_count=1, device="cuda"):
    out = torch.empty((batch, heads, node_count, samples), dtype=torch.int32, device=device)
    _call("hyperattn_sample_indices", ctypes.c_uint64(seed), batch, heads, node_first, node_count, ns,
          samples, _ptr(out), _stream(out.device))
    return out


def row_sqnorms(x):
    """fp32 squared norms of the rows of x ([..., d]) in the row-norm
    variant's fixed order."""
    _need(x, "x")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    w = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _call("hyperattn_row_sqnorms", _ptr(x), _dtype_code(x.dtype), rows, d, _ptr(w), _stream(x.device))
    return w


def rownorm_samples(w, perm_k, heads, samples, seed):
    """Draws of the row-norm variant: w fp32 [B, Hkv, n] squared value-row
    norms, perm_k int32 [B, Hkv, n] the keys' sort permutation.  Returns
    (cum int64 [B, Hkv, n], sidx int32 [B, heads, samples])."""
    _need(w, "w", torch.float32)
    _need(perm_k, "perm_k", torch.int32, w.device)
    B, Hkv, n = w.shape
    cum = torch.empty((B, Hkv, n), dtype=torch.int64, device=w.device)
    sidx = torch.empty((B, heads, samples), dtype=torch.int32, device=w.device)
    wsb = lib().hyperattn_rownorm_samples_workspace_bytes(B, Hkv, n)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=w.device)
    _call("hyperattn_rownorm_samples", _ptr(w), _ptr(perm_k), B, heads, Hkv, n, samples, ctypes.c_uint64(seed),
          _ptr(cum), _ptr(sidx), _ptr(ws), wsb, _stream(w.device))
    return cum, sidx


def column_sqmass(q, k, lse, *, causal=False, skip=0):
    """(colmass [B, H, n], alpha [B, H]) of the exact softmax matrix given
    its exact lse (natural log, [B, H, n]); bf16 q [B, H, n, d], k
    [B, Hkv, n, d]."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    _need(lse, "lse", torch.float32, q.device)
    B, H, n, d = q.shape
    colmass = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    alpha = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _call("hyperattn_column_sqmass", _ptr(q), _ptr(k), _ptr(lse), HA_BF16, B, n, d, H, k.shape[1],
          int(bool(causal)), skip, _ptr(colmass), _ptr(alpha), _stream(q.device))
    return colmass, alpha


def residual_ratio(lse_exact, lse_block, perm_q):
    """kappa per problem from the exact lse (row order), the block part's
    lse (sorted positions) and the queries' permutation, all [..., n]."""
    _need(lse_exact, "lse_exact", torch.float32)
    _need(lse_block, "lse_block", torch.float32, lse_exact.device)
    _need(perm_q, "perm_q", torch.int32, lse_exact.device)
    n = lse_exact.shape[-1]
    problems = lse_exact.numel() // n if n else 0
    kappa = torch.empty(lse_exact.shape[:-1], dtype=torch.float32, device=lse_exact.device)
    _call("hyperattn_residual_ratio", _ptr(lse_exact), _ptr(lse_block), _ptr(perm_q), problems, n, _ptr(kappa),
          _stream(lse_exact.device))
    return kappa


def gather_rows(src, perm):
    """dst[h, j] = src[h, perm[h, j]] for src [heads, n, d], perm int32 [heads, rows]."""
    _need(src, "src")
    _need(perm, "perm", torch.int32, src.device)
    heads, n, d = src.shape
    rows = perm.shape[-1]
    dst = torch.empty((heads, rows, d), dtype=src.dtype, device=src.device)
    _call("hyperattn_gather", _ptr(src), _dtype_code(src.dtype), heads, n, d, _ptr(perm), rows,
          _ptr(dst), _stream(src.device))
    return dst


def attend(q, k, v, perm_q, perm_k, idx, *, block, samples, parts):
    """Block (parts=1), sampled (2) or fused (3) part of a non-causal problem,
    fp32 (o, lse) at sorted positions."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    o = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    _call("hyperattn_attend", _ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), B, n, d, H, Hkv, block,
          samples, _ptr(perm_q), _ptr(perm_k), _ptr(idx), parts, _ptr(o), _ptr(lse), _stream(q.device))
    return o, lse


def merge_unsort(o1, lse1, o2, lse2, perm_q, dtype=torch.bfloat16):
    heads, n, d = o1.shape[-3], o1.shape[-2], o1.shape[-1]
    lead = o1.shape[:-2]
    heads = int(o1.numel() // (n * d)) if n * d else 0
    out = torch.empty(o1.shape, dtype=dtype, device=o1.device)
    lse = torch.empty(lead + (n,), dtype=torch.float32, device=o1.device)
    _call("hyperattn_merge_unsort", _ptr(o1), _ptr(lse1), _ptr(o2), _ptr(lse2), _ptr(perm_q), heads, n, d,
          _dtype_code(dtype), _ptr(out), _ptr(lse), _stream(o1.device))
    return out, lse


def causal_leaves(q, k, v, leaf_len):
    B, H, n, d = q.shape
    o = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    _call("hyperattn_causal_leaves", _ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), B, n, d, H,
          k.shape[1], leaf_len, _ptr(o), _ptr(lse), _stream(q.device))
    return o, lse


def timing_enable(on=True):
    _call("hyperattn_timing_enable", int(bool(on)))


def timing_read():
    """{kernel class: (total ms, launches)} since the last timing_enable."""
    ms = (ctypes.c_double * len(KERNEL_CLASSES))()
    cnt = (ctypes.c_int64 * len(KERNEL_CLASSES))()
    _call("hyperattn_timing_read", ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(cnt, ctypes.c_void_p))
    return {name: (ms[i], cnt[i]) for i, name in enumerate(KERNEL_CLASSES)}
