"""Python binding of libgt_attn.so — biased full-graph attention on gfx950.

Argument marshalling only: every step runs in the library's HIP kernels (or, for
``spd_build``, its native host code). PyTorch provides device memory and the
current stream. There is no fallback: if the library is not built, every call
raises.

    out, lse = fwd(q, k, v, spd, table)
    dq, dk, dv, dtable = bwd(q, k, v, spd, table, out, lse, dout)
    spd = spd_build(indptr, indices, N, C)          # host numpy, uint8 [N, N]
    spd = spd_build_device(indptr, indices, N, C)   # the same codes built on the GPU
    q, k, v = qkv_fwd(x, w)                         # one layer's projections
    dx, dw = qkv_bwd(x, w, dq, dk, dv)
    x_last, dx0, dw, dtable = stack_fwd_bwd(x0, w, tables, spd, dout, H)
    out_b, lse_b = fwd_block(q_rows, k_blk, v_blk, spd[rows, cols], table)   # one key block
    merge(out, lse, out_b, lse_b, out, lse)                                  # running merge
    bwd_block(q_rows, k_blk, v_blk, spd[rows, cols], spd_t[cols, rows], table, out, lse,
              dout_rows, dq, dk, dv, dtable, accumulate=True)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# GT_ATTN_LIBRARY selects another build of the same library (the host-sanitizer build).
LIB_PATH = os.environ.get("GT_ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libgt_attn.so")
GT_F32, GT_BF16 = 0, 1
GT_OK, GT_EINVAL, GT_EUNSUPPORTED, GT_EHIP = 0, -1, -2, -3
ACC_DQ, ACC_DKV, ACC_DTABLE, ACC_ALL = 1, 2, 4, 7   # gt_attn_bwd_block accumulate bits

_lib = None


class GtError(RuntimeError):
    def __init__(self, name: str, code: int, msg: str):
        super().__init__(f"{name} failed with status {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m graph_transformer_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.gt_attn_fwd.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, I32, I32, P]
        L.gt_attn_fwd_ws.argtypes = [P, P, P, P, P, P, P, P, SZ, I64, I32, I32, I32, I32, P]
        L.gt_attn_fwd_ws.restype = ctypes.c_int
        L.gt_attn_fwd_workspace_bytes.argtypes = [I64, I32, I32, I32, I32]
        L.gt_attn_fwd_workspace_bytes.restype = SZ
        L.gt_attn_fwd_block_workspace_bytes.argtypes = [I64, I64, I32, I32, I32, I32]
        L.gt_attn_fwd_block_workspace_bytes.restype = SZ
        L.gt_attn_fwd.restype = ctypes.c_int
        L.gt_attn_bwd_workspace_bytes.argtypes = [I64, I32, I32, I32, I32]
        L.gt_attn_bwd_workspace_bytes.restype = SZ
        L.gt_attn_bwd.argtypes = [P] * 14 + [SZ, I64, I32, I32, I32, I32, P]
        L.gt_attn_bwd.restype = ctypes.c_int
        L.gt_attn_bwd_static.argtypes = [P] * 13 + [I64, I32, I32, I32, I32, P]
        L.gt_attn_bwd_static.restype = ctypes.c_int
        L.gt_spd_build.argtypes = [P, P, I64, I32, P, I32]
        L.gt_spd_build_device_workspace_bytes.argtypes = [I64, I64, I32]
        L.gt_spd_build_device_workspace_bytes.restype = SZ
        L.gt_spd_build_device.argtypes = [P, P, I64, I32, P, P, SZ, P]
        L.gt_spd_build_device.restype = ctypes.c_int
        L.gt_spd_build.restype = ctypes.c_int
        L.gt_last_error.argtypes = []
        L.gt_last_error.restype = ctypes.c_char_p
        L.gt_version.argtypes = []
        L.gt_version.restype = ctypes.c_char_p
        L.gt_trace_enable.argtypes = [I32]
        L.gt_trace_enable.restype = ctypes.c_int
        L.gt_trace_collect.argtypes = [P, P, I32]
        L.gt_trace_collect.restype = ctypes.c_int
        L.gt_probe_peak.argtypes = [I32, I32, I32, P, P]
        L.gt_probe_peak.restype = ctypes.c_int
        L.gt_kernel_name.argtypes = [I32]
        L.gt_kernel_name.restype = ctypes.c_char_p
        L.gt_qkv_fwd.argtypes = [P, P, P, P, P, I64, I32, I32, P]
        L.gt_qkv_fwd.restype = ctypes.c_int
        L.gt_qkv_bwd_workspace_bytes.argtypes = [I64, I32]
        L.gt_qkv_bwd_workspace_bytes.restype = SZ
        L.gt_qkv_bwd.argtypes = [P] * 8 + [SZ, I64, I32, I32, P]
        L.gt_qkv_bwd.restype = ctypes.c_int
        L.gt_store.argtypes = [P, P, I64, I32, P]
        L.gt_store.restype = ctypes.c_int
        L.gt_stack_workspace_bytes.argtypes = [I64, I32, I32, I32, I32, I32]
        L.gt_stack_workspace_bytes.restype = SZ
        L.gt_stack_fwd_bwd.argtypes = [P] * 11 + [SZ, I64, I32, I32, I32, I32, I32, P]
        L.gt_model_param_count.argtypes = [I32, I32]
        L.gt_model_param_count.restype = I32
        L.gt_model_workspace_bytes.argtypes = [I64, I32, I32, I32, I32, I32]
        L.gt_model_workspace_bytes.restype = SZ
        L.gt_model_fwd_bwd.argtypes = [P] * 11 + [SZ, I64, I32, I32, I32, I32, I32, P]
        L.gt_model_fwd_bwd.restype = ctypes.c_int
        L.gt_attn_fwd_block.argtypes = [P, P, P, P, I64, P, P, P, P, SZ, I64, I64, I32, I32, I32, I32, I32, P]
        L.gt_attn_fwd_block.restype = ctypes.c_int
        L.gt_attn_merge.argtypes = [P] * 6 + [I64, I32, I32, P]
        L.gt_attn_merge.restype = ctypes.c_int
        L.gt_attn_bwd_block_workspace_bytes.argtypes = [I64, I64, I32, I32, I32, I32]
        L.gt_attn_bwd_block_workspace_bytes.restype = SZ
        L.gt_attn_bwd_block.argtypes = [P, P, P, P, I64, P, I64] + [P] * 9 + [SZ, I64, I64, I32, I32, I32, I32,
                                                                               I32, P]
        L.gt_attn_bwd_block.restype = ctypes.c_int
        L.gt_stack_fwd_bwd.restype = ctypes.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().gt_last_error().decode()


def _check(name: str, rc: int):
    if rc != GT_OK:
        raise GtError(name, rc, last_error())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GT_F32
    if t.dtype == torch.bfloat16:
        return GT_BF16
    raise TypeError(f"q/k/v/dout must be float32 or bfloat16, got {t.dtype}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a binding call with `stream` (when given) as torch's current stream, so that the
    outputs and temporary workspaces it allocates belong to the stream its kernels run on:
    the caching allocator then hands a dropped temporary to later work on that stream only,
    which the stream orders after the kernels that used it."""
    import functools
    import inspect
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = kwargs.get("stream", args[pos] if len(args) > pos else None)
        if stream is None:
            return fn(*args, **kwargs)
        import torch
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrapper


def _dev(t, name, dtype=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _workspace(nbytes, workspace, device, name="workspace"):
    """(pointer, size) of a caller's workspace, or of a new one; none when nbytes is 0."""
    import torch
    if nbytes == 0 and workspace is None:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return _dev(workspace, name), _nbytes(workspace)


def fwd_workspace_bytes(N: int, H: int, D: int, NB: int, dtype: int) -> int:
    return int(lib().gt_attn_fwd_workspace_bytes(N, H, D, NB, dtype))


@_on_stream
def fwd(q, k, v, spd, table, out=None, lse=None, workspace=None, stream=None):
    """Forward: q, k, v [N,H,D] (float32 or bfloat16), spd [N,N] uint8, table [H,NB] float32.
    Returns (out [N,H,D] float32, lse [N,H] float32)."""
    import torch
    N, H, D = q.shape
    NB = table.shape[1]
    dt = _dtype_code(q)
    need = fwd_workspace_bytes(N, H, D, NB, dt)
    if out is None:
        out = torch.empty((N, H, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((N, H), dtype=torch.float32, device=q.device)
    args = [_dev(q, "q", q.dtype, (N, H, D)), _dev(k, "k", q.dtype, (N, H, D)),
            _dev(v, "v", q.dtype, (N, H, D)), _dev(spd, "spd", torch.uint8, (N, N)),
            _dev(table, "table", torch.float32, (H, NB)), _dev(out, "out", torch.float32, (N, H, D)),
            _dev(lse, "lse", torch.float32, (N, H))]
    if need == 0:
        _check("gt_attn_fwd", lib().gt_attn_fwd(*args, N, H, D, NB, dt, _stream(stream)))
    else:  # a graph small enough that the key loop is split
        wp, wn = _workspace(need, workspace, q.device)
        _check("gt_attn_fwd_ws", lib().gt_attn_fwd_ws(*args, wp, wn, N, H, D, NB, dt, _stream(stream)))
    return out, lse


def bwd_workspace_bytes(N: int, H: int, D: int, NB: int, dtype: int) -> int:
    return int(lib().gt_attn_bwd_workspace_bytes(N, H, D, NB, dtype))


@_on_stream
def bwd(q, k, v, spd, table, out, lse, dout, dq=None, dk=None, dv=None, dtable=None,
        workspace=None, stream=None, spd_t=None):
    """Backward of fwd for loss sum(dout*out). Returns (dq, dk, dv [N,H,D] float32, dtable [H,NB]).

    spd_t is the transpose of spd; None means spd is symmetric (undirected graph)."""
    import torch
    N, H, D = q.shape
    NB = table.shape[1]
    dt = _dtype_code(q)
    f32 = torch.float32
    dq = torch.empty((N, H, D), dtype=f32, device=q.device) if dq is None else dq
    dk = torch.empty((N, H, D), dtype=f32, device=q.device) if dk is None else dk
    dv = torch.empty((N, H, D), dtype=f32, device=q.device) if dv is None else dv
    dtable = torch.empty((H, NB), dtype=f32, device=q.device) if dtable is None else dtable
    wsb = bwd_workspace_bytes(N, H, D, NB, dt)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=q.device)
    args = [_dev(q, "q", q.dtype, (N, H, D)), _dev(k, "k", q.dtype, (N, H, D)),
            _dev(v, "v", q.dtype, (N, H, D)), _dev(spd, "spd", torch.uint8, (N, N)),
            _dev(spd if spd_t is None else spd_t, "spd_t", torch.uint8, (N, N)),
            _dev(table, "table", f32, (H, NB)), _dev(out, "out", f32, (N, H, D)),
            _dev(lse, "lse", f32, (N, H)), _dev(dout, "dout", q.dtype, (N, H, D)),
            _dev(dq, "dq", f32, (N, H, D)), _dev(dk, "dk", f32, (N, H, D)),
            _dev(dv, "dv", f32, (N, H, D)), _dev(dtable, "dtable", f32, (H, NB)),
            _dev(workspace, "workspace")]
    _check("gt_attn_bwd", lib().gt_attn_bwd(*args, workspace.numel() * workspace.element_size(),
                                            N, H, D, NB, dt, _stream(stream)))
    return dq, dk, dv, dtable


BWD_STATIC_SCRATCH_BYTES = 128 << 20   # GT_BWD_STATIC_SCRATCH_BYTES


@_on_stream
def bwd_static(q, k, v, spd, table, out, lse, dout, dq, dk, dv, dtable, stream=None, spd_t=None):
    """bwd through gt_attn_bwd_static: the library's fixed per-GPU scratch array instead of a
    workspace. The caller passes every output (nothing is allocated here or in the call)."""
    import torch
    N, H, D = q.shape
    NB = table.shape[1]
    dt = _dtype_code(q)
    f32 = torch.float32
    args = [_dev(q, "q", q.dtype, (N, H, D)), _dev(k, "k", q.dtype, (N, H, D)),
            _dev(v, "v", q.dtype, (N, H, D)), _dev(spd, "spd", torch.uint8, (N, N)),
            _dev(spd if spd_t is None else spd_t, "spd_t", torch.uint8, (N, N)),
            _dev(table, "table", f32, (H, NB)), _dev(out, "out", f32, (N, H, D)),
            _dev(lse, "lse", f32, (N, H)), _dev(dout, "dout", q.dtype, (N, H, D)),
            _dev(dq, "dq", f32, (N, H, D)), _dev(dk, "dk", f32, (N, H, D)),
            _dev(dv, "dv", f32, (N, H, D)), _dev(dtable, "dtable", f32, (H, NB))]
    _check("gt_attn_bwd_static", lib().gt_attn_bwd_static(*args, N, H, D, NB, dt, _stream(stream)))
    return dq, dk, dv, dtable


def _codes(t, name, rows, cols):
    """A 2-D uint8 GPU view [rows, cols] whose elements are contiguous along a row; its
    rows may lie further apart (a column slice of a larger code matrix). Returns the
    pointer and the row stride in elements."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.uint8:
        raise TypeError(f"{name} must be a uint8 GPU tensor")
    if tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(rows, cols)}")
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be contiguous along its rows")
    ld = t.stride(0) if rows > 1 else cols
    if ld < cols:
        raise ValueError(f"{name}: row stride {ld} < {cols}")
    return ctypes.c_void_p(t.data_ptr()), ld


def fwd_block_workspace_bytes(Nq: int, Nk: int, H: int, D: int, NB: int, dtype: int) -> int:
    return int(lib().gt_attn_fwd_block_workspace_bytes(Nq, Nk, H, D, NB, dtype))


@_on_stream
def fwd_block(q, k, v, spd, table, out=None, lse=None, workspace=None, accumulate=False, stream=None):
    """Attention of Nq query rows restricted to one block of Nk keys.

    q [Nq,H,D], k, v [Nk,H,D] (float32 or bfloat16); spd [Nq,Nk] uint8, usually a
    slice spd_all[r0:r1, c0:c1] (rows may be strided); table [H,NB] float32.
    Returns the block's (out [Nq,H,D], lse [Nq,H]) float32. With accumulate=True, out
    and lse hold a result over other keys on entry and the block is merged into them."""
    import torch
    Nq, H, D = q.shape
    Nk = k.shape[0]
    NB = table.shape[1]
    dt = _dtype_code(q)
    f32 = torch.float32
    if accumulate and (out is None or lse is None):
        raise ValueError("accumulate=True needs the running out and lse")
    out = torch.empty((Nq, H, D), dtype=f32, device=q.device) if out is None else out
    lse = torch.empty((Nq, H), dtype=f32, device=q.device) if lse is None else lse
    sp, ld = _codes(spd, "spd", Nq, Nk)
    wp, wn = _workspace(fwd_block_workspace_bytes(Nq, Nk, H, D, NB, dt), workspace, q.device)
    args = [_dev(q, "q", q.dtype, (Nq, H, D)), _dev(k, "k", q.dtype, (Nk, H, D)),
            _dev(v, "v", q.dtype, (Nk, H, D)), sp, ld, _dev(table, "table", f32, (H, NB)),
            _dev(out, "out", f32, (Nq, H, D)), _dev(lse, "lse", f32, (Nq, H)), wp, wn]
    _check("gt_attn_fwd_block", lib().gt_attn_fwd_block(*args, Nq, Nk, H, D, NB, dt, int(bool(accumulate)),
                                                        _stream(stream)))
    return out, lse


@_on_stream
def merge(out_a, lse_a, out_b, lse_b, out=None, lse=None, stream=None):
    """Merge two partial results over disjoint key sets by their lse. out/lse may be
    out_a/lse_a (running merge). Returns (out, lse)."""
    import torch
    Nq, H, D = out_a.shape
    f32 = torch.float32
    out = torch.empty_like(out_a) if out is None else out
    lse = torch.empty_like(lse_a) if lse is None else lse
    args = [_dev(out_a, "out_a", f32, (Nq, H, D)), _dev(lse_a, "lse_a", f32, (Nq, H)),
            _dev(out_b, "out_b", f32, (Nq, H, D)), _dev(lse_b, "lse_b", f32, (Nq, H)),
            _dev(out, "out", f32, (Nq, H, D)), _dev(lse, "lse", f32, (Nq, H))]
    _check("gt_attn_merge", lib().gt_attn_merge(*args, Nq, H, D, _stream(stream)))
    return out, lse


def bwd_block_workspace_bytes(Nq: int, Nk: int, H: int, D: int, NB: int, dtype: int) -> int:
    return int(lib().gt_attn_bwd_block_workspace_bytes(Nq, Nk, H, D, NB, dtype))


@_on_stream
def bwd_block(q, k, v, spd, spd_t, table, out, lse, dout, dq=None, dk=None, dv=None, dtable=None,
              accumulate=False, workspace=None, stream=None):
    """Backward of one key block given the MERGED out/lse over all keys.

    spd [Nq,Nk] and spd_t [Nk,Nq] are the block's code slices (spd_t rows = keys).
    Returns dq [Nq,H,D] (this block's share), dk, dv [Nk,H,D], dtable [H,NB].
    accumulate: True adds all four into the given tensors, False overwrites them, or
    an int of ACC_DQ | ACC_DKV | ACC_DTABLE bits picks per output."""
    import torch
    Nq, H, D = q.shape
    Nk = k.shape[0]
    NB = table.shape[1]
    dt = _dtype_code(q)
    f32 = torch.float32
    acc = ACC_ALL if accumulate is True else (0 if accumulate is False else int(accumulate))
    need = ((ACC_DQ, dq, "dq"), (ACC_DKV, dk, "dk"), (ACC_DKV, dv, "dv"), (ACC_DTABLE, dtable, "dtable"))
    for bit, t, name in need:
        if acc & bit and t is None:
            raise ValueError(f"accumulating into {name} needs {name} to be given")
    dq = torch.empty((Nq, H, D), dtype=f32, device=q.device) if dq is None else dq
    dk = torch.empty((Nk, H, D), dtype=f32, device=q.device) if dk is None else dk
    dv = torch.empty((Nk, H, D), dtype=f32, device=q.device) if dv is None else dv
    dtable = torch.empty((H, NB), dtype=f32, device=q.device) if dtable is None else dtable
    wsb = bwd_block_workspace_bytes(Nq, Nk, H, D, NB, dt)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=q.device)
    sp, ld = _codes(spd, "spd", Nq, Nk)
    spt, ldt = _codes(spd_t, "spd_t", Nk, Nq)
    args = [_dev(q, "q", q.dtype, (Nq, H, D)), _dev(k, "k", q.dtype, (Nk, H, D)),
            _dev(v, "v", q.dtype, (Nk, H, D)), sp, ld, spt, ldt,
            _dev(table, "table", f32, (H, NB)), _dev(out, "out", f32, (Nq, H, D)),
            _dev(lse, "lse", f32, (Nq, H)), _dev(dout, "dout", q.dtype, (Nq, H, D)),
            _dev(dq, "dq", f32, (Nq, H, D)), _dev(dk, "dk", f32, (Nk, H, D)),
            _dev(dv, "dv", f32, (Nk, H, D)), _dev(dtable, "dtable", f32, (H, NB)),
            _dev(workspace, "workspace")]
    _check("gt_attn_bwd_block", lib().gt_attn_bwd_block(*args, _nbytes(workspace), Nq, Nk, H, D, NB, dt,
                                                        acc, _stream(stream)))
    return dq, dk, dv, dtable


def spd_build(indptr, indices, N: int, C: int, nthreads: int = 0, out=None) -> np.ndarray:
    """Clipped hop-distance codes uint8 [N, N] of an undirected CSR graph (host, native)."""
    indptr = np.ascontiguousarray(indptr, dtype=np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    if indptr.shape != (N + 1,):
        raise ValueError("indptr must have N+1 entries")
    if out is None:
        out = np.empty((N, N), dtype=np.uint8)
    if out.dtype != np.uint8 or out.shape != (N, N) or not out.flags.c_contiguous:
        raise ValueError("out must be a C-contiguous uint8 [N, N] array")
    ip = indices.ctypes.data if indices.size else None
    _check("gt_spd_build", lib().gt_spd_build(indptr.ctypes.data, ip, N, C, out.ctypes.data, nthreads))
    return out


@_on_stream
def spd_build_device(indptr, indices, N: int, C: int, out=None, workspace=None, stream=None):
    """The codes of spd_build computed on the GPU: uint8 [N, N] on the current device."""
    import torch
    indptr = np.ascontiguousarray(indptr, dtype=np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    if indptr.shape != (N + 1,):
        raise ValueError("indptr must have N+1 entries")
    if out is None:
        out = torch.empty((N, N), dtype=torch.uint8, device="cuda")
    nbytes = int(lib().gt_spd_build_device_workspace_bytes(N, int(indptr[-1]), C))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=out.device)
    ip = indices.ctypes.data if indices.size else None
    _check("gt_spd_build_device", lib().gt_spd_build_device(
        indptr.ctypes.data, ip, N, C, _dev(out, "spd", torch.uint8, (N, N)), _dev(workspace, "workspace"),
        _nbytes(workspace), _stream(stream)))
    return out


# One layer's parameter vector of the full model, in order (hid = ffn = 64).
MODEL_PARAM_ORDER = (("g1", 1), ("b1", 1), ("wq", 2), ("wk", 2), ("wv", 2), ("wo", 2), ("g2", 1), ("b2", 1),
                     ("w1", 2), ("c1", 1), ("w2", 2), ("c2", 1))


def model_pack(named, hid: int = 64):
    """float32 [L, P] parameter vectors from named per-layer arrays ([L, hid] or
    [L, hid, hid], names as in MODEL_PARAM_ORDER)."""
    parts = []
    for name, rank in MODEL_PARAM_ORDER:
        a = np.asarray(named[name], dtype=np.float32)
        L = a.shape[0]
        parts.append(a.reshape(L, hid ** rank))
    out = np.ascontiguousarray(np.concatenate(parts, axis=1))
    assert out.shape[1] == int(lib().gt_model_param_count(hid, hid))
    return out


@_on_stream
def model_fwd_bwd(x0, params, tables, spd, dout, H: int, dtype=None, spd_t=None, workspace=None, stream=None):
    """The full-layer model: x0, dout [N, 64] float32; params [L, P] float32 (model_pack);
    tables [L, H, NB] float32; spd [N, N] uint8. dtype: storage type of Q/K/V and the
    attention's output gradient (torch.bfloat16 or torch.float32).
    Returns (x_last [N,64], dx0 [N,64], dparams [L,P], dtables [L,H,NB])."""
    import torch
    N, hid = x0.shape
    L, P = params.shape
    NB = tables.shape[2]
    D = hid // H
    dt = GT_BF16 if dtype in (None, torch.bfloat16) else GT_F32
    f32 = torch.float32
    x_last = torch.empty((N, hid), dtype=f32, device=x0.device)
    dx0 = torch.empty((N, hid), dtype=f32, device=x0.device)
    dparams = torch.empty((L, P), dtype=f32, device=x0.device)
    dtables = torch.empty((L, H, NB), dtype=f32, device=x0.device)
    nbytes = int(lib().gt_model_workspace_bytes(N, L, H, D, NB, dt))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x0.device)
    args = [_dev(x0, "x0", f32, (N, hid)), _dev(params, "params", f32, (L, P)),
            _dev(tables, "tables", f32, (L, H, NB)), _dev(spd, "spd", torch.uint8, (N, N)),
            _dev(spd if spd_t is None else spd_t, "spd_t", torch.uint8, (N, N)), _dev(dout, "dout", f32, (N, hid)),
            _dev(x_last, "x_last"), _dev(dx0, "dx0"), _dev(dparams, "dparams"), _dev(dtables, "dtables"),
            _dev(workspace, "workspace")]
    _check("gt_model_fwd_bwd", lib().gt_model_fwd_bwd(*args, _nbytes(workspace), N, L, H, D, NB, dt, _stream(stream)))
    return x_last, dx0, dparams, dtables


def version() -> str:
    return lib().gt_version().decode()


def _empty_like_shape(shape, dtype, device):
    import torch
    return torch.empty(shape, dtype=dtype, device=device)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


@_on_stream
def qkv_fwd(x, w, q=None, k=None, v=None, stream=None):
    """One layer's projections: x [N, hid], w [3, hid, hid] (float32 or bfloat16).
    Returns q, k, v [N, hid] in x's dtype (float32 accumulation, then rounded)."""
    N, hid = x.shape
    dt = _dtype_code(x)
    q, k, v = (_empty_like_shape((N, hid), x.dtype, x.device) if t is None else t for t in (q, k, v))
    args = [_dev(x, "x", x.dtype, (N, hid)), _dev(w, "w", x.dtype, (3, hid, hid)),
            _dev(q, "q", x.dtype, (N, hid)), _dev(k, "k", x.dtype, (N, hid)), _dev(v, "v", x.dtype, (N, hid))]
    _check("gt_qkv_fwd", lib().gt_qkv_fwd(*args, N, hid, dt, _stream(stream)))
    return q, k, v


@_on_stream
def qkv_bwd(x, w, dq, dk, dv, dx=None, dw=None, workspace=None, stream=None):
    """Backward of qkv_fwd for float32 dq, dk, dv [N, hid]: returns dx [N, hid], dw [3, hid, hid]."""
    import torch
    N, hid = x.shape
    dt = _dtype_code(x)
    f32 = torch.float32
    dx = _empty_like_shape((N, hid), f32, x.device) if dx is None else dx
    dw = _empty_like_shape((3, hid, hid), f32, x.device) if dw is None else dw
    if workspace is None:
        workspace = torch.empty(max(int(lib().gt_qkv_bwd_workspace_bytes(N, hid)), 256), dtype=torch.uint8,
                                device=x.device)
    args = [_dev(x, "x", x.dtype, (N, hid)), _dev(w, "w", x.dtype, (3, hid, hid)),
            _dev(dq, "dq", f32, (N, hid)), _dev(dk, "dk", f32, (N, hid)), _dev(dv, "dv", f32, (N, hid)),
            _dev(dx, "dx", f32, (N, hid)), _dev(dw, "dw", f32, (3, hid, hid)), _dev(workspace, "workspace")]
    _check("gt_qkv_bwd", lib().gt_qkv_bwd(*args, _nbytes(workspace), N, hid, dt, _stream(stream)))
    return dx, dw


@_on_stream
def store(src, dtype, dst=None, stream=None):
    """float32 tensor -> dtype (torch.bfloat16: round to nearest even; torch.float32: copy)."""
    import torch
    dt = GT_BF16 if dtype == torch.bfloat16 else GT_F32
    dst = _empty_like_shape(tuple(src.shape), dtype, src.device) if dst is None else dst
    args = [_dev(src, "src", torch.float32), _dev(dst, "dst", dtype, tuple(src.shape))]
    _check("gt_store", lib().gt_store(*args, src.numel(), dt, _stream(stream)))
    return dst


def stack_workspace_bytes(N: int, L: int, H: int, D: int, NB: int, dtype: int) -> int:
    return int(lib().gt_stack_workspace_bytes(N, L, H, D, NB, dtype))


@_on_stream
def stack_fwd_bwd(x0, w, tables, spd, dout, H: int, spd_t=None, workspace=None, stream=None):
    """Forward and backward of L stacked layers (see gt_stack_fwd_bwd) for loss sum(dout * X_L).
    x0, dout [N, hid]; w [L, 3, hid, hid]; tables [L, H, NB] float32; spd [N, N] uint8.
    Returns (x_last [N, hid] in x0's dtype, dx0 [N, hid], dw [L, 3, hid, hid], dtable [L, H, NB])."""
    import torch
    N, hid = x0.shape
    L, _, NB = tables.shape
    D = hid // H
    dt = _dtype_code(x0)
    f32 = torch.float32
    x_last = _empty_like_shape((N, hid), x0.dtype, x0.device)
    dx0 = _empty_like_shape((N, hid), f32, x0.device)
    dw = _empty_like_shape((L, 3, hid, hid), f32, x0.device)
    dtable = _empty_like_shape((L, H, NB), f32, x0.device)
    wsb = stack_workspace_bytes(N, L, H, D, NB, dt)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x0.device)
    args = [_dev(x0, "x0", x0.dtype, (N, hid)), _dev(w, "w", x0.dtype, (L, 3, hid, hid)),
            _dev(tables, "tables", f32, (L, H, NB)), _dev(spd, "spd", torch.uint8, (N, N)),
            _dev(spd if spd_t is None else spd_t, "spd_t", torch.uint8, (N, N)),
            _dev(dout, "dout", x0.dtype, (N, hid)), _dev(x_last, "x_last"), _dev(dx0, "dx0"), _dev(dw, "dw"),
            _dev(dtable, "dtable"), _dev(workspace, "workspace")]
    _check("gt_stack_fwd_bwd", lib().gt_stack_fwd_bwd(*args, _nbytes(workspace), N, L, H, D, NB, dt,
                                                      _stream(stream)))
    return x_last, dx0, dw, dtable


KERNEL_COUNT = 17


def kernel_names():
    return [lib().gt_kernel_name(i).decode() for i in range(KERNEL_COUNT)]


def trace(on: bool):
    """Bracket every kernel the library enqueues from this thread with HIP events."""
    _check("gt_trace_enable", lib().gt_trace_enable(1 if on else 0))


def trace_collect() -> dict:
    """Wait for traced kernels; {kernel name: (launches, total ms)} since the last collect."""
    counts = (ctypes.c_int32 * KERNEL_COUNT)()
    ms = (ctypes.c_double * KERNEL_COUNT)()
    _check("gt_trace_collect", lib().gt_trace_collect(counts, ms, KERNEL_COUNT))
    return {n: (int(counts[i]), float(ms[i])) for i, n in enumerate(kernel_names()) if counts[i]}


PROBES = {0: ("exp2", "Gop/s"), 1: ("fma", "Gop/s"), 2: ("exp2 with 4 fma", "Gexp/s"),
          3: ("mfma 32x32x8 bf16", "TFLOP/s"), 4: ("mfma 32x32x16 bf16", "TFLOP/s")}


def probe_peak(kind: int, blocks: int = 4096, iters: int = 2048, repeats: int = 3) -> float:
    """Measured rate of one unit (see gt_probe_peak); best of `repeats` timed launches."""
    import torch
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    best = None
    for _ in range(repeats + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        _check("gt_probe_peak", lib().gt_probe_peak(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                                    ctypes.c_void_p(s.cuda_stream)))
        b.record()
        b.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    if kind in (0, 1, 2):
        return blocks * 256 * iters * 8 / (best * 1e-3) / 1e9
    flops = 16384 if kind == 3 else 32768
    return blocks * 4 * iters * 4 * flops / (best * 1e-3) / 1e12
