"""Memory-efficient exact attention on AMD MI355X (gfx950).

Thin ctypes binding over ``libmea.so`` (C ABI in ``include/mea.h``). The
functions here only marshal arguments: they check tensor placement and
layout, allocate outputs with torch when the caller does not pass them, and
call the C entry points of the same names on the current torch stream. All
arithmetic runs in the library's HIP kernels; there is no fallback path, and
every function raises if the library has not been built.
"""

import contextlib
import ctypes
import os

__all__ = [
    "MeaError", "DTYPE_F32", "DTYPE_BF16", "lib", "library_path",
    "attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_status_str", "mea_version",
    "attn_fwd_ex", "attn_bwd_ex", "attn_bwd_ex_workspace_bytes",
    "attn_fwd_splitkv", "attn_fwd_splitkv_num_splits", "attn_fwd_splitkv_workspace_bytes",
    "attn_bwd_noalloc", "NOALLOC_SCRATCH_BYTES", "load", "using", "timing_library_path",
]

DTYPE_F32 = 0
DTYPE_BF16 = 1
# size of the scratch array attn_bwd_noalloc runs in (MEA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

_STATUS = ["MEA_OK", "MEA_ERR_NULL", "MEA_ERR_SHAPE", "MEA_ERR_UNSUPPORTED",
           "MEA_ERR_ALIGN", "MEA_ERR_WORKSPACE", "MEA_ERR_LAUNCH", "MEA_ERR_ALIAS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path():
    return os.path.join(_HERE, "libmea.so")


def timing_library_path():
    """The timing build (same kernels, plus end-of-tile cycle counters)."""
    return os.path.join(_HERE, "libmea_synctimers.so")


class MeaError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, fn, status):
        self.status = int(status)
        super().__init__(f"{fn} failed: {attn_status_str(self.status)} ({self.status})")


def lib():
    """The loaded ``libmea.so`` (ctypes.CDLL), with argument types declared."""
    global _LIB
    if _LIB is None:
        _LIB = load(library_path())
    return _LIB


@contextlib.contextmanager
def using(handle):
    """Route the wrappers below through another build of the library (a handle
    from ``load``, e.g. the timing library) inside the ``with`` block."""
    global _LIB
    saved = lib()
    _LIB = handle
    try:
        yield handle
    finally:
        _LIB = saved


def load(path):
    """A ctypes handle on a build of the library at ``path``, with the C ABI's
    argument types declared."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m memory_efficient_exact_amd.build` "
            "(or __graft_entry__.build()). There is no fallback implementation.")
    L = ctypes.CDLL(path)
    i64, vp, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.attn_fwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    L.attn_fwd.restype = i32
    L.attn_bwd_workspace_bytes.argtypes = [i32, i64, i64, i64, i64]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_bwd.restype = i32
    L.attn_bwd_noalloc.argtypes = [i32, i64, i64, i64, i64] + [vp] * 11
    L.attn_bwd_noalloc.restype = i32
    L.attn_fwd_ex.argtypes = [i32, i64, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    L.attn_fwd_ex.restype = i32
    L.attn_bwd_ex_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, i64]
    L.attn_bwd_ex_workspace_bytes.restype = sz
    L.attn_bwd_ex.argtypes = [i32, i64, i64, i64, i64, i64, i64] + [vp] * 11 + [sz, vp]
    L.attn_bwd_ex.restype = i32
    L.attn_fwd_splitkv.argtypes = [i32, i64, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, i64,
                                   vp, sz, vp]
    L.attn_fwd_splitkv.restype = i32
    L.attn_fwd_splitkv_num_splits.argtypes = [i32, i64, i64, i64, i64, i64, i64, i64]
    L.attn_fwd_splitkv_num_splits.restype = i64
    L.attn_fwd_splitkv_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, i64, i64]
    L.attn_fwd_splitkv_workspace_bytes.restype = sz
    L.attn_status_str.argtypes = [i32]
    L.attn_status_str.restype = ctypes.c_char_p
    L.mea_version.argtypes = []
    L.mea_version.restype = i32
    return L


def attn_status_str(status):
    """Name of a status code, from the library (falls back to the table if unbuilt)."""
    try:
        return lib().attn_status_str(int(status)).decode()
    except RuntimeError:
        s = int(status)
        return _STATUS[s] if 0 <= s < len(_STATUS) else "MEA_UNKNOWN_STATUS"


def mea_version():
    return lib().mea_version()


def attn_bwd_workspace_bytes(dt, B, H, n, d):
    return lib().attn_bwd_workspace_bytes(int(dt), int(B), int(H), int(n), int(d))


def attn_bwd_ex_workspace_bytes(dt, B, H, H_kv, n_q, n_k, d):
    return lib().attn_bwd_ex_workspace_bytes(*(int(x) for x in (dt, B, H, H_kv, n_q, n_k, d)))


def attn_fwd_splitkv_num_splits(dt, B, H, H_kv, n_q, n_k, d, num_splits=0):
    return lib().attn_fwd_splitkv_num_splits(
        *(int(x) for x in (dt, B, H, H_kv, n_q, n_k, d, num_splits)))


def attn_fwd_splitkv_workspace_bytes(dt, B, H, H_kv, n_q, n_k, d, num_splits=0):
    return lib().attn_fwd_splitkv_workspace_bytes(
        *(int(x) for x in (dt, B, H, H_kv, n_q, n_k, d, num_splits)))


# ------------------------------------------------------------ torch marshalling

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}; expected torch.bfloat16 or torch.float32")


# The checks below run on every call, so each takes one combined test on the
# common path and builds its message only when the test fails.

def _check_as(name, t, shape, like, dev=None):
    """t must be a contiguous GPU tensor of `shape` with like's dtype and device
    (`dev`: like's device index, when the caller has it already)."""
    if dev is None:
        dev = like.get_device()
    if dev >= 0 and t.get_device() == dev and t.shape == shape and t.dtype == like.dtype \
            and t.is_contiguous():
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != like.dtype:
        raise ValueError(f"{name} must have shape {tuple(shape)} dtype {like.dtype}, "
                         f"got {tuple(t.shape)} {t.dtype}")
    raise ValueError(f"{name} must be contiguous")


def _check(name, t, like, dev=None):
    _check_as(name, t, like.shape, like, dev)


def _check_stat(name, t, q, dev=None, rows=None):
    """t must be a contiguous float32 GPU tensor of shape q.shape[:3] on q's device."""
    import torch
    if dev is None:
        dev = q.get_device()
    if rows is None:
        rows = q.shape[:3]
    if dev >= 0 and t.get_device() == dev and t.shape == rows and t.dtype == torch.float32 \
            and t.is_contiguous():
        return
    if not t.is_cuda or t.device != q.device:
        raise ValueError(f"{name} must be on {q.device}")
    if tuple(t.shape) != tuple(q.shape[:3]):
        raise ValueError(f"{name} must have shape {tuple(q.shape[:3])}, got {tuple(t.shape)}")
    raise ValueError(f"{name} must be contiguous float32")


def _gqa_shapes(q, k, v):
    """(B, H, H_kv, n_q, n_k, d) of q [B,H,n_q,d] and k, v [B,H_kv,n_k,d]."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, n_q, d] and k, v [B, H_kv, n_k, d]")
    B, H, n_q, d = q.shape
    H_kv, n_k = k.shape[1], k.shape[2]
    di = q.get_device()
    _check_as("q", q, q.shape, q, di)
    kv = (B, H_kv, n_k, d)
    _check_as("k", k, kv, q, di)
    _check_as("v", v, kv, q, di)
    return B, H, H_kv, n_q, n_k, d


def _fwd_outputs(q, out, row_max, row_sum, stats):
    import torch
    if out is None:
        out = torch.empty_like(q)
    _check_as("out", out, q.shape, q)
    if (row_max is None) != (row_sum is None):
        raise ValueError("pass both row_max and row_sum, or neither")
    if row_max is None and stats:
        row_max = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        row_sum = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if row_max is not None:
        di, rows = q.get_device(), q.shape[:3]
        _check_stat("row_max", row_max, q, di, rows)
        _check_stat("row_sum", row_sum, q, di, rows)
    return out, row_max, row_sum


def _workspace(workspace, need, device):
    """(workspace, its size in bytes): a contiguous tensor on `device`,
    allocated with `need` bytes (at least 16) when the caller passes none."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if workspace.device != device:
        raise ValueError(f"workspace is on {workspace.device}, expected {device}")
    return workspace, workspace.numel() * workspace.element_size()


def _stream(stream, device):
    """Raw hipStream_t of `stream`, or of torch's current stream on `device`."""
    if stream is not None:
        return stream.cuda_stream
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _call(device, fn, *args):
    """Call a library entry point with `device` current (the kernels launch on
    the current HIP device); the device switch is skipped when it already is."""
    import torch
    if torch.cuda.current_device() == device.index:
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


def attn_fwd(q, k, v, out=None, row_max=None, row_sum=None, stats=True, stream=None):
    """O = softmax(q k^T / sqrt(d)) v for contiguous [B, H, n, d] GPU tensors.

    Returns (o, row_max, row_sum); the statistics are None when ``stats`` is
    False and none are passed. Outputs not passed are allocated with torch.
    Enqueued on ``stream`` (default: torch's current stream); not synchronised.
    """
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, n, d]")
    dt = _dtype_code(q)
    di = q.get_device()
    _check("q", q, q, di)
    _check("k", k, q, di)
    _check("v", v, q, di)
    if out is None:
        out = torch.empty_like(q)
    _check("out", out, q, di)
    if (row_max is None) != (row_sum is None):
        raise ValueError("pass both row_max and row_sum, or neither")
    if row_max is None and stats:
        row_max = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        row_sum = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if row_max is not None:
        rows = q.shape[:3]
        _check_stat("row_max", row_max, q, di, rows)
        _check_stat("row_sum", row_sum, q, di, rows)
    B, H, n, d = q.shape
    dev = q.device
    st = _call(dev, lib().attn_fwd, dt, B, H, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
               _ptr(row_max), _ptr(row_sum), _stream(stream, dev))
    if st != 0:
        raise MeaError("attn_fwd", st)
    return out, row_max, row_sum


def attn_bwd(q, k, v, o, do, row_max, row_sum, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """Gradients (dq, dk, dv) of sum(o * do), recomputing P from the saved
    row statistics. Same tensor conventions as ``attn_fwd``; ``workspace`` is
    a GPU tensor of at least ``attn_bwd_workspace_bytes`` bytes (allocated if
    not passed)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, n, d]")
    dt = _dtype_code(q)
    di = q.get_device()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, q, di)
    rows = q.shape[:3]
    _check_stat("row_max", row_max, q, di, rows)
    _check_stat("row_sum", row_sum, q, di, rows)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, q, di)
    B, H, n, d = q.shape
    workspace, wbytes = _workspace(workspace, attn_bwd_workspace_bytes(dt, B, H, n, d), q.device)
    dev = q.device
    st = _call(dev, lib().attn_bwd, dt, B, H, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
               _ptr(row_max), _ptr(row_sum), _ptr(dq), _ptr(dk), _ptr(dv),
               _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise MeaError("attn_bwd", st)
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, row_max, row_sum, dq, dk, dv, stream=None):
    """``attn_bwd`` for callers that cannot allocate: no workspace argument (the
    library runs in its own per-GPU scratch array of NOALLOC_SCRATCH_BYTES), and
    the outputs dq, dk, dv must be passed, so the call allocates nothing.
    Calls that may overlap on one GPU race on the scratch array."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, n, d]")
    dt = _dtype_code(q)
    di = q.get_device()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check(name, t, q, di)
    rows = q.shape[:3]
    _check_stat("row_max", row_max, q, di, rows)
    _check_stat("row_sum", row_sum, q, di, rows)
    B, H, n, d = q.shape
    dev = q.device
    st = _call(dev, lib().attn_bwd_noalloc, dt, B, H, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
               _ptr(do), _ptr(row_max), _ptr(row_sum), _ptr(dq), _ptr(dk), _ptr(dv),
               _stream(stream, dev))
    if st != 0:
        raise MeaError("attn_bwd_noalloc", st)
    return dq, dk, dv


def attn_fwd_ex(q, k, v, out=None, row_max=None, row_sum=None, stats=True, stream=None):
    """Forward with separate lengths and shared key/value heads: q [B, H, n_q, d],
    k and v [B, H_kv, n_k, d] with H a multiple of H_kv; query head h reads
    key/value head h // (H // H_kv). Returns (o, row_max, row_sum) as ``attn_fwd``."""
    dt = _dtype_code(q)
    B, H, H_kv, n_q, n_k, d = _gqa_shapes(q, k, v)
    out, row_max, row_sum = _fwd_outputs(q, out, row_max, row_sum, stats)
    dev = q.device
    st = _call(dev, lib().attn_fwd_ex, dt, B, H, H_kv, n_q, n_k, d, _ptr(q), _ptr(k), _ptr(v),
               _ptr(out), _ptr(row_max), _ptr(row_sum), _stream(stream, dev))
    if st != 0:
        raise MeaError("attn_fwd_ex", st)
    return out, row_max, row_sum


def attn_bwd_ex(q, k, v, o, do, row_max, row_sum, dq=None, dk=None, dv=None, workspace=None,
                stream=None):
    """Backward of ``attn_fwd_ex``: (dq [B, H, n_q, d], dk and dv [B, H_kv, n_k, d]);
    dk and dv sum over the query heads that share each key/value head."""
    import torch
    dt = _dtype_code(q)
    B, H, H_kv, n_q, n_k, d = _gqa_shapes(q, k, v)
    _check_as("o", o, q.shape, q)
    _check_as("do", do, q.shape, q)
    _check_stat("row_max", row_max, q)
    _check_stat("row_sum", row_sum, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_as("dq", dq, q.shape, q)
    _check_as("dk", dk, k.shape, q)
    _check_as("dv", dv, v.shape, q)
    workspace, wbytes = _workspace(workspace, attn_bwd_ex_workspace_bytes(dt, B, H, H_kv, n_q, n_k, d),
                                   q.device)
    dev = q.device
    st = _call(dev, lib().attn_bwd_ex, dt, B, H, H_kv, n_q, n_k, d, _ptr(q), _ptr(k), _ptr(v),
               _ptr(o), _ptr(do), _ptr(row_max), _ptr(row_sum), _ptr(dq), _ptr(dk), _ptr(dv),
               _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise MeaError("attn_bwd_ex", st)
    return dq, dk, dv


def attn_fwd_splitkv(q, k, v, num_splits=0, out=None, row_max=None, row_sum=None, stats=True,
                     workspace=None, stream=None):
    """``attn_fwd_ex`` with every head's keys cut into ranges reduced by separate
    workgroups and merged afterwards (for small grids and decoding).
    ``num_splits`` 0 lets the library choose. ``workspace`` (a GPU tensor of at
    least ``attn_fwd_splitkv_workspace_bytes`` bytes) is allocated if not passed."""
    dt = _dtype_code(q)
    B, H, H_kv, n_q, n_k, d = _gqa_shapes(q, k, v)
    out, row_max, row_sum = _fwd_outputs(q, out, row_max, row_sum, stats)
    need = attn_fwd_splitkv_workspace_bytes(dt, B, H, H_kv, n_q, n_k, d, num_splits)
    workspace, wbytes = _workspace(workspace, need, q.device)
    dev = q.device
    st = _call(dev, lib().attn_fwd_splitkv, dt, B, H, H_kv, n_q, n_k, d, _ptr(q), _ptr(k),
               _ptr(v), _ptr(out), _ptr(row_max), _ptr(row_sum), int(num_splits),
               _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise MeaError("attn_fwd_splitkv", st)
    return out, row_max, row_sum
