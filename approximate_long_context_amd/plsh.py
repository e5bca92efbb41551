"""ctypes binding of libplsh (include/plsh.h): argument marshalling only.

Every step of the estimator runs inside the library; torch supplies device
memory and the current HIP stream.  Loading fails loudly when the library has
not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libplsh.so")

PLSH_OK, PLSH_ERR_ARG, PLSH_ERR_TABLE, PLSH_ERR_UNSUPPORTED, PLSH_ERR_CAPACITY, PLSH_ERR_HIP = range(6)
PLSH_BF16, PLSH_F32 = 0, 1
STATUS_NAMES = {0: "PLSH_OK", 1: "PLSH_ERR_ARG", 2: "PLSH_ERR_TABLE", 3: "PLSH_ERR_UNSUPPORTED",
                4: "PLSH_ERR_CAPACITY", 5: "PLSH_ERR_HIP"}

EXPORTED = ["plsh_sample_tables", "plsh_build_tables", "plsh_validate_tables", "plsh_count_work",
            "plsh_alibi_attention", "plsh_alibi_attention_ws", "plsh_attention_workspace_size",
            "plsh_alibi_attention_noalloc", "plsh_alibi_records", "plsh_alibi_attention_from_records",
            "plsh_debug_block_intervals",
            "plsh_debug_attention_reference", "plsh_alibi_attention_unfused", "plsh_alibi_attention_walk",
            "plsh_alibi_attention_backward", "plsh_alibi_attention_backward_saved",
            "plsh_alibi_attention_lse", "plsh_exact_alibi_attention",
            "plsh_sample_params_device", "plsh_kernel_timer", "plsh_kernel_timer_read", "plsh_last_error"]


class PlshError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _Tables(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("heads", ctypes.c_int32), ("s", ctypes.c_int32),
                ("params", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("starts", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libplsh.so (built by approximate_long_context_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m approximate_long_context_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
        TP = ctypes.POINTER(_Tables)
        L.plsh_sample_tables.argtypes = [u64, i32, i32, vp, i32, vp, vp, vp, i64, ctypes.POINTER(i64)]
        L.plsh_build_tables.argtypes = [i32, i32, i32, vp, vp, vp, i64, ctypes.POINTER(i64)]
        L.plsh_validate_tables.argtypes = [TP]
        L.plsh_count_work.argtypes = [TP, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        attn = [vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp, i32, TP, i32, vp]
        L.plsh_alibi_attention.argtypes = attn
        L.plsh_debug_attention_reference.argtypes = attn
        L.plsh_alibi_attention_unfused.argtypes = attn
        L.plsh_alibi_attention_walk.argtypes = attn
        L.plsh_alibi_attention_noalloc.argtypes = attn
        L.plsh_alibi_attention_ws.argtypes = attn[:-1] + [vp, i64, vp]
        L.plsh_alibi_attention_from_records.argtypes = attn[:-1] + [vp, i64, vp]
        L.plsh_alibi_records.argtypes = [TP, i32, vp, i64, vp]
        L.plsh_attention_workspace_size.argtypes = [i32, i32, i32, ctypes.c_int, ctypes.POINTER(i64)]
        L.plsh_alibi_attention_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                    ctypes.c_int, vp, i32, TP, i32, vp]
        L.plsh_alibi_attention_backward_saved.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                          i32, i32, ctypes.c_int, vp, i32, TP, i32, vp]
        L.plsh_alibi_attention_lse.argtypes = attn[:-1] + [vp, vp, i64, vp]
        L.plsh_debug_block_intervals.argtypes = [TP, vp, vp]
        L.plsh_exact_alibi_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                                 vp, i32, vp]
        L.plsh_sample_params_device.argtypes = [u64, i32, vp, i32, vp, vp]
        L.plsh_kernel_timer.argtypes = [i32]
        L.plsh_kernel_timer_read.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]
        for f in EXPORTED[:-1]:
            getattr(L, f).restype = ctypes.c_int
        L.plsh_last_error.restype = ctypes.c_char_p
        L.plsh_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != PLSH_OK:
        raise PlshError(status, lib().plsh_last_error().decode())


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


@dataclass
class Tables:
    """Boundary table of s hashes per head (host arrays; see include/plsh.h)."""
    n: int
    heads: int
    s: int
    params: np.ndarray   # float64 [heads*s, 2]
    offsets: np.ndarray  # int32 [heads*s + 1]
    starts: np.ndarray   # int32 [offsets[-1]]

    def c_struct(self) -> _Tables:
        return _Tables(self.n, self.heads, self.s, _ptr(self.params), _ptr(self.offsets),
                       _ptr(self.starts))

    def to(self, device) -> "DeviceTables":
        return DeviceTables(self.n, self.heads, self.s,
                            torch.from_numpy(self.params).to(device),
                            torch.from_numpy(self.offsets).to(device),
                            torch.from_numpy(self.starts).to(device))

    def starts_of(self, h: int, k: int) -> np.ndarray:
        r = h * self.s + k
        return self.starts[self.offsets[r]:self.offsets[r + 1]]


@dataclass
class DeviceTables:
    """The same table resident on the GPU (torch tensors own the memory)."""
    n: int
    heads: int
    s: int
    params: torch.Tensor
    offsets: torch.Tensor
    starts: torch.Tensor

    def c_struct(self) -> _Tables:
        return _Tables(self.n, self.heads, self.s, self.params.data_ptr(), self.offsets.data_ptr(),
                       self.starts.data_ptr())


def sample_tables(seed: int, n: int, sigma: Sequence[float], s: int) -> Tables:
    """plsh_sample_tables.  The starts buffer is first sized from the
    expected table size (a pitch drawn from Gamma(2, sigma) has E[1/delta] =
    1/sigma, so a hash has about n/sigma + 2 entries, at most n + 1), with
    room to spare, so that one call usually fills it; only a table larger
    than that takes the protocol's second call."""
    L = lib()
    sig = np.ascontiguousarray(sigma, dtype=np.float64)
    heads = len(sig)
    params = np.empty((heads * s, 2), dtype=np.float64)
    offsets = np.empty(heads * s + 1, dtype=np.int32)
    need = ctypes.c_int64(0)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        per_row = np.minimum(float(max(n, 0) + 1), 2.0 * n / sig + 3.0)
    per_row = np.where(np.isfinite(per_row) & (per_row > 0), per_row, float(max(n, 0) + 1))
    guess = int(min(float(heads) * s * (max(n, 0) + 1), s * float(per_row.sum()) + 2.0 * (max(n, 0) + 1)))
    starts = np.empty(max(guess, 1), dtype=np.int32)
    st = L.plsh_sample_tables(seed, n, heads, _ptr(sig), s, _ptr(params), _ptr(offsets),
                              _ptr(starts), starts.size, ctypes.byref(need))
    if st == PLSH_ERR_CAPACITY and need.value > starts.size:
        starts = np.empty(max(need.value, 1), dtype=np.int32)
        st = L.plsh_sample_tables(seed, n, heads, _ptr(sig), s, _ptr(params), _ptr(offsets),
                                  _ptr(starts), starts.size, ctypes.byref(need))
    _check(st)
    return Tables(n, heads, s, params, offsets, starts[:need.value].copy())


def sample_params_device(seed: int, sigma: Sequence[float], s: int, device,
                         stream: Optional[int] = None) -> torch.Tensor:
    """plsh_sample_params_device: float64 [heads * s, 2] (delta, u) drawn on
    the GPU, bit for bit those of sample_tables(seed, ...)."""
    if torch.device(device).type != "cuda":
        raise PlshError(PLSH_ERR_ARG, f"device must be a CUDA device, not {device}")
    sig = np.ascontiguousarray(sigma, dtype=np.float64)
    params = torch.empty((sig.size * s, 2), dtype=torch.float64, device=device)
    if stream is None:
        stream = torch.cuda.current_stream(params.device).cuda_stream
    _check(lib().plsh_sample_params_device(seed, sig.size, _ptr(sig), s, params.data_ptr(), stream))
    return params


def device_sampled_tables(seed: int, n: int, sigma: Sequence[float], s: int, device,
                          stream: Optional[int] = None) -> "DeviceTables":
    """Tables for the attention entry points with parameters drawn on the GPU
    (per-step resampling without a host round trip).  The attention kernels
    read only params; offsets and starts stay empty."""
    params = sample_params_device(seed, sigma, s, device, stream)
    empty = torch.empty(0, dtype=torch.int32, device=params.device)
    return DeviceTables(n, len(sigma), s, params, empty, empty)


def build_tables(n: int, heads: int, s: int, params) -> Tables:
    """plsh_build_tables: the table of caller-given (delta, u) rows,
    [heads*s, 2] float64 (two-call protocol)."""
    L = lib()
    prm = np.ascontiguousarray(params, dtype=np.float64).reshape(heads * s, 2)
    offsets = np.empty(heads * s + 1, dtype=np.int32)
    need = ctypes.c_int64(0)
    _check(L.plsh_build_tables(n, heads, s, _ptr(prm), _ptr(offsets), None, 0, ctypes.byref(need)))
    starts = np.empty(max(need.value, 1), dtype=np.int32)
    _check(L.plsh_build_tables(n, heads, s, _ptr(prm), _ptr(offsets), _ptr(starts), starts.size,
                               ctypes.byref(need)))
    return Tables(n, heads, s, prm.copy(), offsets, starts[:need.value])


def fixed_block_tables(n: int, width: Sequence[float], s: int = 1) -> Tables:
    """The "fixed blocks" baseline: per head one deterministic hash of pitch
    width[h] and offset 0 (blocks [0, w), [w, 2w), ... for integer w),
    repeated for the s samples."""
    w = np.asarray(width, dtype=np.float64)
    params = np.zeros((len(w) * s, 2), dtype=np.float64)
    params[:, 0] = np.repeat(w, s)
    return build_tables(n, len(w), s, params)


def validate_tables(t: Tables) -> None:
    st = t.c_struct()
    _check(lib().plsh_validate_tables(ctypes.byref(st)))


def count_work(t: Tables, causal: bool):
    """(pairs_alg, pairs_distinct) per batch element."""
    st = t.c_struct()
    a, d = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().plsh_count_work(ctypes.byref(st), int(bool(causal)), ctypes.byref(a), ctypes.byref(d)))
    return a.value, d.value


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PLSH_BF16
    if t.dtype == torch.float32:
        return PLSH_F32
    raise PlshError(PLSH_ERR_UNSUPPORTED, f"dtype {t.dtype} not supported")


def _require_device_tables(tables, device: torch.device) -> None:
    """The kernels dereference params on the device: only a DeviceTables whose
    params is a contiguous float64 [heads*s, 2] tensor on `device` may reach
    the library (a host Tables would hand it host addresses)."""
    if not isinstance(tables, DeviceTables):
        raise PlshError(PLSH_ERR_ARG, "tables must be a DeviceTables (Tables.to(device)), "
                                      f"not {type(tables).__name__}")
    p = tables.params
    if not isinstance(p, torch.Tensor) or p.device != device or p.dtype != torch.float64 or \
            not p.is_contiguous() or tuple(p.shape) != (tables.heads * tables.s, 2):
        raise PlshError(PLSH_ERR_ARG, "tables.params must be a contiguous float64 "
                                      f"[heads*s, 2] tensor on {device}")


def _require_cuda(device: Optional[torch.device] = None, **tensors) -> torch.device:
    """Every tensor is a contiguous CUDA tensor on one device (the first's,
    or `device`); returns that device."""
    for name, x in tensors.items():
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            raise PlshError(PLSH_ERR_ARG, f"{name} must be a CUDA tensor")
        if device is None:
            device = x.device
        elif x.device != device:
            raise PlshError(PLSH_ERR_ARG, f"{name} is on {x.device}, expected {device}")
        if not x.is_contiguous():
            raise PlshError(PLSH_ERR_ARG, f"{name} must be contiguous")
    return device


def _require_like(name: str, x: torch.Tensor, ref: torch.Tensor) -> None:
    if tuple(x.shape) != tuple(ref.shape) or x.dtype != ref.dtype:
        raise PlshError(PLSH_ERR_ARG, f"{name} must have shape {tuple(ref.shape)} and dtype {ref.dtype}")


def _attention(fn, q, k, v, sigma, s, tables: DeviceTables, causal, out, stream, ws=None):
    dev = _require_cuda(q=q, k=k, v=v)
    _require_device_tables(tables, dev)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise PlshError(PLSH_ERR_ARG, "q [B,H,n,d], k/v [B,Hkv,n,d] with one dtype expected")
    B, H, n, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    _require_cuda(dev, out=out)
    _require_like("out", out, q)
    sig = np.ascontiguousarray(sigma, dtype=np.float64)
    if sig.size != H:
        raise PlshError(PLSH_ERR_ARG, "sigma must have one entry per query head")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = tables.c_struct()
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, n, H, k.shape[1], d,
            _dtype_code(q), _ptr(sig), s, ctypes.byref(st), int(bool(causal))]
    if ws is not None:
        args += list(ws)
    _check(fn(*args, stream))
    return out


def workspace_size(n: int, heads: int, s: int, dtype: torch.dtype) -> int:
    """plsh_attention_workspace_size: bytes of workspace attention() takes."""
    nb = ctypes.c_int64(0)
    code = PLSH_BF16 if dtype == torch.bfloat16 else PLSH_F32 if dtype == torch.float32 else -1
    _check(lib().plsh_attention_workspace_size(n, heads, s, code, ctypes.byref(nb)))
    return nb.value


def attention(q, k, v, sigma, s, tables: DeviceTables, causal: bool = False,
              out: Optional[torch.Tensor] = None, stream: Optional[int] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The estimator, q [B,H,n,d], k/v [B,Hkv,n,d]: plsh_alibi_attention_ws
    with `workspace` (a device uint8 tensor of at least workspace_size()
    bytes) or, on torch's current stream, one from torch's caching
    allocator.  The call runs on `stream` if given (with no workspace it is
    then plsh_alibi_attention, with the library's stream-ordered workspace),
    else on torch's current stream."""
    if stream is not None and workspace is None:
        return _attention(lib().plsh_alibi_attention, q, k, v, sigma, s, tables, causal, out, stream)
    need = workspace_size(q.shape[2], q.shape[1], s, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise PlshError(PLSH_ERR_ARG, "workspace must be a contiguous uint8 tensor on q's device")
    ws = (workspace.data_ptr(), workspace.numel())
    return _attention(lib().plsh_alibi_attention_ws, q, k, v, sigma, s, tables, causal, out, stream, ws)


def _require_workspace(workspace, device: torch.device) -> None:
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or \
            not workspace.is_contiguous() or workspace.device != device:
        raise PlshError(PLSH_ERR_ARG, f"workspace must be a contiguous uint8 tensor on {device}")


def build_records(tables: DeviceTables, causal: bool, workspace: torch.Tensor,
                  stream: Optional[int] = None) -> torch.Tensor:
    """plsh_alibi_records: the block-edge records of `tables` (the pre-pass
    alone) into `workspace` (a device uint8 tensor of at least
    workspace_size(n, heads, s, torch.bfloat16) bytes), for
    attention_from_records with the same tables and causal flag."""
    if not isinstance(tables, DeviceTables):
        raise PlshError(PLSH_ERR_ARG, "tables must be a DeviceTables (Tables.to(device))")
    dev = tables.params.device
    _require_device_tables(tables, dev)
    _require_workspace(workspace, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = tables.c_struct()
    _check(lib().plsh_alibi_records(ctypes.byref(st), int(bool(causal)), workspace.data_ptr(),
                                    workspace.numel(), stream))
    return workspace


def attention_from_records(q, k, v, sigma, s, tables: DeviceTables, workspace: torch.Tensor,
                           causal: bool = False, out: Optional[torch.Tensor] = None,
                           stream: Optional[int] = None) -> torch.Tensor:
    """plsh_alibi_attention_from_records: the attention kernel alone, over
    the records build_records wrote to `workspace` for the same tables and
    causal flag (bitwise the output of attention())."""
    _require_workspace(workspace, q.device)
    ws = (workspace.data_ptr(), workspace.numel())
    return _attention(lib().plsh_alibi_attention_from_records, q, k, v, sigma, s, tables, causal, out, stream, ws)


def attention_noalloc(q, k, v, sigma, s, tables: DeviceTables, causal: bool = False,
                      out: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
    """plsh_alibi_attention_noalloc: the records in the library's static
    scratch (the call allocates no device memory; pass `out` to allocate
    nothing here either).  Calls that overlap on one device race."""
    return _attention(lib().plsh_alibi_attention_noalloc, q, k, v, sigma, s, tables, causal, out, stream)


def attention_library_workspace(q, k, v, sigma, s, tables: DeviceTables, causal: bool = False,
                                out: Optional[torch.Tensor] = None,
                                stream: Optional[int] = None) -> torch.Tensor:
    """plsh_alibi_attention: the workspace from the library's stream-ordered
    allocator, taken and released on the stream inside the call."""
    return _attention(lib().plsh_alibi_attention, q, k, v, sigma, s, tables, causal, out, stream)


def attention_unfused(q, k, v, sigma, s, tables: DeviceTables, causal: bool = False,
                      out: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
    """plsh_alibi_attention_unfused: s single-sample passes plus a
    log-sum-exp combine (ablation of the sample fusion)."""
    return _attention(lib().plsh_alibi_attention_unfused, q, k, v, sigma, s, tables, causal, out, stream)


def attention_walk(q, k, v, sigma, s, tables: DeviceTables, causal: bool = False,
                   out: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
    """plsh_alibi_attention_walk: the samples walked one by one with 0/1
    masks inside one kernel (ablation of the sample fusion)."""
    return _attention(lib().plsh_alibi_attention_walk, q, k, v, sigma, s, tables, causal, out, stream)


def attention_with_lse(q, k, v, sigma, s, tables: DeviceTables, causal: bool = False,
                       out: Optional[torch.Tensor] = None, stream: Optional[int] = None,
                       lse2: Optional[torch.Tensor] = None):
    """plsh_alibi_attention_lse: (out, lse2), lse2 float32 [B, H, ceil32(n)]
    = log2 of each row's normaliser (rows past n hold 0), for
    attention_backward(..., out=out, lse2=lse2)."""
    B, H, n, d = q.shape
    shape = (B, H, (n + 31) // 32 * 32)
    if lse2 is None:
        lse2 = torch.empty(shape, dtype=torch.float32, device=q.device)
    elif lse2.dtype != torch.float32 or tuple(lse2.shape) != shape or not lse2.is_contiguous() or \
            lse2.device != q.device:
        raise PlshError(PLSH_ERR_ARG, "lse2 must be a contiguous float32 [B, H, ceil32(n)] tensor on q's device")
    if stream is None:
        need = workspace_size(n, H, s, q.dtype)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        ws_args = (ws.data_ptr(), ws.numel())
    else:   # an explicit stream: the library's stream-ordered workspace
        ws_args = (None, 0)

    def fn(*args):
        return lib().plsh_alibi_attention_lse(*args[:-1], lse2.data_ptr(), *ws_args, args[-1])
    out = _attention(fn, q, k, v, sigma, s, tables, causal, out, stream)
    return out, lse2


def attention_backward(q, k, v, dout, sigma, s, tables: DeviceTables, causal: bool = False,
                       stream: Optional[int] = None, out: Optional[torch.Tensor] = None,
                       lse2: Optional[torch.Tensor] = None):
    """(dq, dk, dv) for the upstream gradient dout of the estimate (fixed
    tables): plsh_alibi_attention_backward, or, given the forward's out and
    lse2 (attention_with_lse), plsh_alibi_attention_backward_saved."""
    if (out is None) != (lse2 is None):
        raise PlshError(PLSH_ERR_ARG, "out and lse2 go together")
    dev = _require_cuda(q=q, k=k, v=v, dout=dout)
    if out is not None:
        _require_cuda(dev, out=out, lse2=lse2)
    _require_device_tables(tables, dev)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or dout.shape != q.shape or \
            len({q.dtype, k.dtype, v.dtype, dout.dtype}) != 1:
        raise PlshError(PLSH_ERR_ARG, "q/dout [B,H,n,d], k/v [B,Hkv,n,d] with one dtype expected")
    B, H, n, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    sig = np.ascontiguousarray(sigma, dtype=np.float64)
    if sig.size != H:
        raise PlshError(PLSH_ERR_ARG, "sigma must have one entry per query head")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = tables.c_struct()
    if out is None:
        _check(lib().plsh_alibi_attention_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, n, H,
                                                   k.shape[1], d, _dtype_code(q), _ptr(sig), s,
                                                   ctypes.byref(st), int(bool(causal)), stream))
        return dq, dk, dv
    if out.shape != q.shape or out.dtype != q.dtype or lse2.dtype != torch.float32 or \
            tuple(lse2.shape) != (B, H, (n + 31) // 32 * 32):
        raise PlshError(PLSH_ERR_ARG, "out [B,H,n,d] of q's dtype and lse2 float32 [B,H,ceil32(n)] expected")
    _check(lib().plsh_alibi_attention_backward_saved(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                     lse2.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                                     dk.data_ptr(), dv.data_ptr(), B, n, H, k.shape[1], d,
                                                     _dtype_code(q), _ptr(sig), s, ctypes.byref(st),
                                                     int(bool(causal)), stream))
    return dq, dk, dv


def exact_alibi_attention(q, k, v, sigma, causal: bool = False, out: Optional[torch.Tensor] = None,
                          stream: Optional[int] = None) -> torch.Tensor:
    """plsh_exact_alibi_attention (dense exact ALiBi, bf16) on the current
    stream: q [B,H,n,d], k/v [B,Hkv,n,d]."""
    dev = _require_cuda(q=q, k=k, v=v)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise PlshError(PLSH_ERR_ARG, "q [B,H,n,d], k/v [B,Hkv,n,d] with one dtype expected")
    B, H, n, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    _require_cuda(dev, out=out)
    _require_like("out", out, q)
    sig = np.ascontiguousarray(sigma, dtype=np.float64)
    if sig.size != H:
        raise PlshError(PLSH_ERR_ARG, "sigma must have one entry per query head")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().plsh_exact_alibi_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, n,
                                            H, k.shape[1], d, _dtype_code(q), _ptr(sig), int(bool(causal)),
                                            stream))
    return out


def attention_reference(q, k, v, sigma, s, tables: DeviceTables, causal: bool = False,
                        out: Optional[torch.Tensor] = None, stream: Optional[int] = None):
    """plsh_debug_attention_reference: the one-row-per-wave VALU formulation."""
    return _attention(lib().plsh_debug_attention_reference, q, k, v, sigma, s, tables, causal, out,
                      stream)


def debug_block_intervals(tables: DeviceTables, stream: Optional[int] = None) -> torch.Tensor:
    """int32 [heads*s, n, 2] (lo, hi) recomputed on the GPU."""
    if not isinstance(tables, DeviceTables) or tables.params.device.type != "cuda":
        raise PlshError(PLSH_ERR_ARG, "tables must be a DeviceTables with params on the GPU")
    _require_device_tables(tables, tables.params.device)
    lohi = torch.empty((tables.heads * tables.s, tables.n, 2), dtype=torch.int32,
                       device=tables.params.device)
    if stream is None:
        stream = torch.cuda.current_stream(lohi.device).cuda_stream
    st = tables.c_struct()
    _check(lib().plsh_debug_block_intervals(ctypes.byref(st), lohi.data_ptr(), stream))
    return lohi


def kernel_timer(enable: bool) -> None:
    """plsh_kernel_timer: time the attention kernel of this thread's calls."""
    _check(lib().plsh_kernel_timer(int(bool(enable))))


def kernel_timer_read():
    """plsh_kernel_timer_read -> (launches, total_ms) since the last read."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    _check(lib().plsh_kernel_timer_read(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value
