"""Thin ctypes binding of liblla (argument marshalling only).

Every step of the forward runs in the library's HIP kernels; this module checks tensor
shapes, dtypes and devices, allocates the output when asked, and passes raw device
pointers and the current HIP stream to the C entry points of the same names.  There is
no CPU fallback: if ``liblla.so`` is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["lla_forward", "lla_forward_ex", "lla_forward_ws", "lla_workspace_size",
           "lla_forward_workspace_bytes", "lla_pool_trim", "lla_forward_noalloc",
           "lla_forward_fallback_rows",
           "lla_path_available", "lla_parallax_forward", "lla_parallax_forward_ex",
           "lla_parallax_forward_ws", "lla_parallax_workspace_size", "lla_parallax_path_available",
           "lla_parallax_decode", "lla_parallax_decode_ws", "lla_parallax_decode_workspace_size",
           "lla_decode", "lla_decode_ws", "lla_decode_workspace_size",
           "lla_profile_enable", "lla_profile_collect",
           "lla_status_string", "lla_version", "LLAError",
           "library_path", "load_library", "STATUS", "PATHS", "DTYPES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS = {0: "LLA_OK", 1: "LLA_ERR_NULL", 2: "LLA_ERR_SHAPE", 3: "LLA_ERR_PARAM",
          4: "LLA_ERR_UNSUPPORTED", 5: "LLA_ERR_WORKSPACE", 6: "LLA_ERR_HIP", 7: "LLA_ERR_ALIAS",
          8: "LLA_ERR_SCRATCH_LIMIT"}
PATHS = {"auto": 0, "exact": 1, "fast": 2, "cg": 3}
DTYPES = {"f32": 0, "bf16": 1}


class LLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name} ({lla_status_string(status)})")


def library_path() -> str:
    return os.path.join(_HERE, "liblla.so")


def load_library():
    """Load liblla.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    i64, f64, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.lla_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f64, f64, ctypes.c_int, vp]
    lib.lla_forward.restype = ctypes.c_int
    lib.lla_forward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f64, f64, ctypes.c_int,
                                   vp, ctypes.c_int]
    lib.lla_forward_ex.restype = ctypes.c_int
    lib.lla_status_string.argtypes = [ctypes.c_int]
    lib.lla_status_string.restype = ctypes.c_char_p
    lib.lla_path_available.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64]
    lib.lla_path_available.restype = ctypes.c_int
    lib.lla_version.argtypes = []
    lib.lla_version.restype = ctypes.c_int
    lib.lla_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.lla_workspace_size.restype = ctypes.c_size_t
    lib.lla_forward_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.lla_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.lla_forward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f64, f64, ctypes.c_int, vp,
                                        ctypes.c_int]
    lib.lla_forward_noalloc.restype = ctypes.c_int
    lib.lla_pool_trim.argtypes = []
    lib.lla_pool_trim.restype = ctypes.c_int
    lib.lla_forward_fallback_rows.argtypes = [vp, ctypes.c_size_t, i64, i64, i64, i64, ctypes.c_int,
                                              ctypes.c_int, ctypes.POINTER(i64), vp]
    lib.lla_forward_fallback_rows.restype = ctypes.c_int
    lib.lla_forward_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f64, f64, ctypes.c_int,
                                   vp, ctypes.c_int, vp, ctypes.c_size_t]
    lib.lla_forward_ws.restype = ctypes.c_int
    lib.lla_parallax_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f64, ctypes.c_int, vp]
    lib.lla_parallax_forward.restype = ctypes.c_int
    lib.lla_parallax_forward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f64, ctypes.c_int, vp,
                                            ctypes.c_int]
    lib.lla_parallax_forward_ex.restype = ctypes.c_int
    lib.lla_parallax_forward_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f64, ctypes.c_int, vp,
                                            ctypes.c_int, vp, ctypes.c_size_t]
    lib.lla_parallax_forward_ws.restype = ctypes.c_int
    lib.lla_parallax_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.lla_parallax_workspace_size.restype = ctypes.c_size_t
    lib.lla_parallax_forward_stats.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f64, ctypes.c_int, vp,
                                               ctypes.c_int, vp, ctypes.c_size_t]
    lib.lla_parallax_forward_stats.restype = ctypes.c_int
    lib.lla_parallax_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f64,
                                          ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_size_t]
    lib.lla_parallax_backward.restype = ctypes.c_int
    lib.lla_parallax_backward_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.lla_parallax_backward_workspace_size.restype = ctypes.c_size_t
    lib.lla_parallax_path_available.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64]
    lib.lla_parallax_path_available.restype = ctypes.c_int
    lib.lla_parallax_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f64, ctypes.c_int, vp]
    lib.lla_parallax_decode.restype = ctypes.c_int
    lib.lla_parallax_decode_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f64, ctypes.c_int, vp, vp,
                                           ctypes.c_size_t]
    lib.lla_parallax_decode_ws.restype = ctypes.c_int
    lib.lla_parallax_decode_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.lla_parallax_decode_workspace_size.restype = ctypes.c_size_t
    lib.lla_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f64, f64, ctypes.c_int, vp]
    lib.lla_decode.restype = ctypes.c_int
    lib.lla_decode_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f64, f64, ctypes.c_int, vp, vp, ctypes.c_size_t]
    lib.lla_decode_ws.restype = ctypes.c_int
    lib.lla_decode_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.lla_decode_workspace_size.restype = ctypes.c_size_t
    lib.lla_profile_enable.argtypes = [ctypes.c_int]
    lib.lla_profile_enable.restype = ctypes.c_int
    lib.lla_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_float), ctypes.c_int]
    lib.lla_profile_collect.restype = ctypes.c_int
    _LIB = lib
    return lib


def lla_status_string(status: int) -> str:
    return load_library().lla_status_string(int(status)).decode()


def lla_path_available(path: str, dtype: str, d: int) -> bool:
    """Whether kernel path "auto" / "exact" / "fast" covers (dtype "f32"/"bf16", d)."""
    return bool(load_library().lla_path_available(PATHS[path], DTYPES[dtype], int(d)))


def lla_version() -> int:
    return int(load_library().lla_version())


def _marshal(q, k, v, out):
    import torch
    dtype = _marshal_inputs(q, k, v)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    elif out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous float32 tensor of q's shape on q's device")
    return dtype, out


def _marshal_inputs(q, k, v):
    import torch
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError(f"q, k, v must share one [B, H, n, d] shape; got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if q.dtype == torch.float32:
        dtype = DTYPES["f32"]
    elif q.dtype == torch.bfloat16:
        dtype = DTYPES["bf16"]
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    return dtype


def lla_forward_ex(q, k, v, h: float, lam: float, path: str = "auto", out=None, stream=None):
    """LLA forward of device tensors q, k, v [B, H, n, d] (fp32 or bf16) -> fp32 out.

    ``path`` is "auto", "exact" or "fast"; ``stream`` a torch stream (default: current)."""
    import torch
    dtype, out = _marshal(q, k, v, out)
    B, H, n, d = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().lla_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       B, H, n, d, float(h), float(lam), dtype,
                                       ctypes.c_void_p(stream.cuda_stream), PATHS[path])
    if st != 0:
        raise LLAError(st, "lla_forward_ex")
    return out


def lla_forward(q, k, v, h: float, lam: float, out=None, stream=None):
    """LLA forward through the library's default path selection."""
    import torch
    dtype, out = _marshal(q, k, v, out)
    B, H, n, d = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().lla_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    B, H, n, d, float(h), float(lam), dtype,
                                    ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise LLAError(st, "lla_forward")
    return out


def lla_workspace_size(B: int, H: int, n: int, d: int, dtype: str, path: str = "auto") -> int:
    """Bytes of device scratch the chosen path needs (0 if none)."""
    return int(load_library().lla_workspace_size(B, H, n, d, DTYPES[dtype], PATHS[path]))


def lla_forward_workspace_bytes(B: int, H: int, n: int, d: int, dtype: str) -> int:
    """Bytes of device scratch lla_forward_ws needs on the default (auto) path (0 if none)."""
    return int(load_library().lla_forward_workspace_bytes(B, H, n, d, DTYPES[dtype]))


def lla_forward_noalloc(q, k, v, h: float, lam: float, path: str = "auto", out=None, stream=None):
    """LLA forward whose scratch is the library's static device buffer (no allocation by the
    library; `out` is allocated here unless given)."""
    import torch
    dtype, out = _marshal(q, k, v, out)
    B, H, n, d = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().lla_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            B, H, n, d, float(h), float(lam), dtype,
                                            ctypes.c_void_p(stream.cuda_stream), PATHS[path])
    if st != 0:
        raise LLAError(st, "lla_forward_noalloc")
    return out


def lla_pool_trim() -> None:
    """Return the library pool's cached blocks (from pool-backed calls) to the system."""
    st = load_library().lla_pool_trim()
    if st != 0:
        raise LLAError(st, "lla_pool_trim")


def lla_forward_ws(q, k, v, h: float, lam: float, workspace, path: str = "auto", out=None,
                   stream=None):
    """LLA forward with caller-provided scratch (a device tensor of at least
    lla_workspace_size bytes, or None when none is needed); allocates nothing but `out`."""
    import torch
    dtype, out = _marshal(q, k, v, out)
    B, H, n, d = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = load_library().lla_forward_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       B, H, n, d, float(h), float(lam), dtype,
                                       ctypes.c_void_p(stream.cuda_stream), PATHS[path],
                                       ctypes.c_void_p(ws_ptr) if ws_ptr else None, ws_bytes)
    if st != 0:
        raise LLAError(st, "lla_forward_ws")
    return out


def lla_forward_fallback_rows(workspace, shape, dtype: str, path: str = "auto", stream=None) -> int:
    """Rows that the matrix-core path of the last lla_forward_ws call on `workspace` (a device
    tensor; problem `shape` = (B, H, n, d), input dtype "bf16" or "f32") recomputed on the
    fp64 kernel.  Waits for `stream` (default: the current stream)."""
    import torch
    B, H, n, d = (int(x) for x in shape)
    if stream is None:
        stream = torch.cuda.current_stream()
    if workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rows = ctypes.c_int64(0)
    st = load_library().lla_forward_fallback_rows(ctypes.c_void_p(ws_ptr) if ws_ptr else None, ws_bytes,
                                                  B, H, n, d, DTYPES[dtype], PATHS[path], ctypes.byref(rows),
                                                  ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise LLAError(st, "lla_forward_fallback_rows")
    return rows.value


def _marshal_probe(q, rho):
    if rho.shape != q.shape or rho.dtype != q.dtype:
        raise ValueError(f"rho must have q's shape and dtype; got {tuple(rho.shape)}, {rho.dtype}")
    if not rho.is_cuda or not rho.is_contiguous() or rho.device != q.device:
        raise ValueError("rho must be a contiguous device tensor on q's device")


def lla_parallax_forward(q, k, v, rho, h: float, path: str = "auto", out=None, stream=None):
    """Parallax forward of device tensors q, k, v, rho [B, H, n, d] (fp32 or bf16) -> fp32
    out: o_i = softmax attention - Sigma_KV rho_i.  ``path`` is "auto", "exact" or "fast"."""
    import torch
    dtype, out = _marshal(q, k, v, out)
    _marshal_probe(q, rho)
    B, H, n, d = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load_library()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), rho.data_ptr(), out.data_ptr(), B, H, n, d, float(h),
            dtype, ctypes.c_void_p(stream.cuda_stream))
    if path == "auto":
        st = lib.lla_parallax_forward(*args)
    else:
        st = lib.lla_parallax_forward_ex(*args, PATHS[path])
    if st != 0:
        raise LLAError(st, "lla_parallax_forward")
    return out


def lla_parallax_forward_ex(q, k, v, rho, h: float, path: str = "auto", out=None, stream=None):
    """lla_parallax_forward with an explicit kernel path."""
    return lla_parallax_forward(q, k, v, rho, h, path=path, out=out, stream=stream)


def lla_parallax_workspace_size(B: int, H: int, n: int, d: int, dtype: str, path: str = "auto") -> int:
    """Bytes of device scratch the chosen Parallax path needs (0 if none)."""
    return int(load_library().lla_parallax_workspace_size(B, H, n, d, DTYPES[dtype], PATHS[path]))


def lla_parallax_path_available(path: str, dtype: str, d: int) -> bool:
    """Whether Parallax kernel path "auto" / "exact" / "fast" covers (dtype, d)."""
    return bool(load_library().lla_parallax_path_available(PATHS[path], DTYPES[dtype], int(d)))


def _device_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t.data_ptr()


def lla_parallax_forward_stats(q, k, v, rho, h: float, path: str = "auto", out=None, lse=None, stream=None,
                               workspace=None):
    """Parallax forward that also writes the per-row base-2 log-sum-exp of the scores the
    backward reads: returns (out [B, H, n, d] fp32, lse [B, H, n] fp32).  ``workspace``:
    None (library pool) or a device tensor of at least lla_parallax_workspace_size bytes."""
    import torch
    dtype, out = _marshal(q, k, v, out)
    _marshal_probe(q, rho)
    B, H, n, d = q.shape
    if lse is None:
        lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    elif tuple(lse.shape) != (B, H, n) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, n]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    wp = _device_ptr(workspace, "workspace")
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().lla_parallax_forward_stats(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), rho.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, n, d,
        float(h), dtype, ctypes.c_void_p(stream.cuda_stream), PATHS[path], wp, wb)
    if st != 0:
        raise LLAError(st, "lla_parallax_forward_stats")
    return out, lse


def lla_parallax_backward(q, k, v, rho, dout, lse, h: float, path: str = "auto", grads=None, stream=None,
                          workspace=None):
    """Gradients (dq, dk, dv, drho), fp32 [B, H, n, d], of sum(o * dout) for the Parallax
    forward of q, k, v, rho whose log-sum-exp lla_parallax_forward_stats wrote; dout in the
    inputs' dtype.  ``grads``: optional four preallocated fp32 tensors.  ``workspace``: None
    (library pool) or a device tensor of at least lla_parallax_backward_workspace_size bytes."""
    import torch
    dtype = _marshal_inputs(q, k, v)
    _marshal_probe(q, rho)
    _marshal_probe(q, dout)
    B, H, n, d = q.shape
    if tuple(lse.shape) != (B, H, n) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, n]")
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(4))
    for gname, gt in zip(("dq", "dk", "dv", "drho"), grads):
        if gt.shape != q.shape or gt.dtype != torch.float32:
            raise ValueError(f"{gname} must be float32 of q's shape")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    wp = _device_ptr(workspace, "workspace")
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptrs = [_device_ptr(t, nm) for t, nm in ((lse, "lse"),) + tuple(zip(grads, ("dq", "dk", "dv", "drho")))]
    st = load_library().lla_parallax_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), rho.data_ptr(), dout.data_ptr(), *ptrs, B, H, n, d, float(h),
        dtype, ctypes.c_void_p(stream.cuda_stream), PATHS[path], wp, wb)
    if st != 0:
        raise LLAError(st, "lla_parallax_backward")
    return grads


def lla_parallax_backward_workspace_size(B: int, H: int, n: int, d: int, dtype: str, path: str = "auto") -> int:
    """Bytes of device scratch lla_parallax_backward needs on ``path``."""
    return int(load_library().lla_parallax_backward_workspace_size(B, H, n, d, DTYPES[dtype], PATHS[path]))


def lla_parallax_forward_ws(q, k, v, rho, h: float, workspace, path: str = "auto", out=None, stream=None):
    """Parallax forward with caller-provided scratch (a device tensor of at least
    lla_parallax_workspace_size bytes, or None when none is needed)."""
    import torch
    dtype, out = _marshal(q, k, v, out)
    _marshal_probe(q, rho)
    B, H, n, d = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = load_library().lla_parallax_forward_ws(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), rho.data_ptr(), out.data_ptr(), B, H, n, d, float(h), dtype,
        ctypes.c_void_p(stream.cuda_stream), PATHS[path], ctypes.c_void_p(ws_ptr) if ws_ptr else None, ws_bytes)
    if st != 0:
        raise LLAError(st, "lla_parallax_forward_ws")
    return out


def _marshal_decode(q, k, v, rho, out):
    import torch
    if q.dim() != 3 or k.dim() != 4 or k.shape != v.shape or q.shape != rho.shape \
            or tuple(q.shape) != (k.shape[0], k.shape[1], k.shape[3]):
        raise ValueError(f"decode takes q, rho [B, H, d] and k, v [B, H, L, d]; got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}, {tuple(rho.shape)}")
    if not (q.dtype == k.dtype == v.dtype == rho.dtype):
        raise ValueError("q, k, v, rho must share one dtype")
    if q.dtype == torch.float32:
        dtype = DTYPES["f32"]
    elif q.dtype == torch.bfloat16:
        dtype = DTYPES["bf16"]
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("rho", rho)):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous device tensor on q's device")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    elif out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous float32 tensor of q's shape on q's device")
    return dtype, out


def lla_parallax_decode(q, k, v, rho, h: float, out=None, stream=None):
    """Parallax decode step: q, rho [B, H, d] against the cache k, v [B, H, L, d] (fp32 or
    bf16) -> fp32 out [B, H, d]."""
    import torch
    dtype, out = _marshal_decode(q, k, v, rho, out)
    B, H, L, d = k.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().lla_parallax_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), rho.data_ptr(),
                                            out.data_ptr(), B, H, L, d, float(h), dtype,
                                            ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise LLAError(st, "lla_parallax_decode")
    return out


def lla_parallax_decode_workspace_size(B: int, H: int, L: int, d: int, dtype: str) -> int:
    """Bytes of device scratch a decode step needs (0 if none)."""
    return int(load_library().lla_parallax_decode_workspace_size(B, H, L, d, DTYPES[dtype]))


def lla_parallax_decode_ws(q, k, v, rho, h: float, workspace, out=None, stream=None):
    """Parallax decode step with caller-provided scratch (a device tensor of at least
    lla_parallax_decode_workspace_size bytes, or None when none is needed)."""
    import torch
    dtype, out = _marshal_decode(q, k, v, rho, out)
    B, H, L, d = k.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = load_library().lla_parallax_decode_ws(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), rho.data_ptr(), out.data_ptr(), B, H, L, d, float(h), dtype,
        ctypes.c_void_p(stream.cuda_stream), ctypes.c_void_p(ws_ptr) if ws_ptr else None, ws_bytes)
    if st != 0:
        raise LLAError(st, "lla_parallax_decode_ws")
    return out


def lla_decode(q, k, v, h: float, lam: float, out=None, stream=None, workspace=None, use_ws=False):
    """LLA decode step: q [B, H, d] against the cache k, v [B, H, L, d] (fp32 or bf16) -> fp32
    out [B, H, d].  With ``use_ws`` the caller's ``workspace`` tensor (or None when none is
    needed) is passed to lla_decode_ws instead of the library pool."""
    import torch
    dtype, out = _marshal_decode(q, k, v, q, out)
    B, H, L, d = k.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load_library()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, d, float(h), float(lam), dtype,
            ctypes.c_void_p(stream.cuda_stream))
    if use_ws:
        if workspace is None:
            ws_ptr, ws_bytes = None, 0
        else:
            if not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous device tensor")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = lib.lla_decode_ws(*args, ctypes.c_void_p(ws_ptr) if ws_ptr else None, ws_bytes)
    else:
        st = lib.lla_decode(*args)
    if st != 0:
        raise LLAError(st, "lla_decode_ws" if use_ws else "lla_decode")
    return out


def lla_decode_ws(q, k, v, h: float, lam: float, workspace, out=None, stream=None):
    """lla_decode with caller-provided scratch (allocates nothing but `out`)."""
    return lla_decode(q, k, v, h, lam, out=out, stream=stream, workspace=workspace, use_ws=True)


def lla_decode_workspace_size(B: int, H: int, L: int, d: int, dtype: str) -> int:
    """Bytes of device scratch an LLA decode step needs."""
    return int(load_library().lla_decode_workspace_size(B, H, L, d, DTYPES[dtype]))


def lla_profile_enable(enable: bool = True) -> bool:
    """Bracket every library kernel launch with HIP events; returns the previous setting."""
    return bool(load_library().lla_profile_enable(1 if enable else 0))


def lla_profile_collect(max_entries: int = 4096):
    """[(kernel name, milliseconds), ...] of the launches recorded since the last collect."""
    names = (ctypes.c_char_p * max_entries)()
    ms = (ctypes.c_float * max_entries)()
    cnt = load_library().lla_profile_collect(names, ms, max_entries)
    return [(names[i].decode(), float(ms[i])) for i in range(cnt)]
