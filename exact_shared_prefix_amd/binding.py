"""Thin ctypes binding over libdualkv.so (include/dualkv.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or cannot be loaded, every
call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdualkv.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
EXPORTS = ("dualkv_fwd_workspace_bytes", "dualkv_bwd_workspace_bytes", "dualkv_fwd",
           "dualkv_bwd", "dualkv_bwd_phases", "dualkv_status_string",
           "dualkv_fwd_workspace_bytes_groups", "dualkv_bwd_workspace_bytes_groups",
           "dualkv_fwd_groups", "dualkv_bwd_groups",
           "dualkv_fwd_workspace_bytes_tree", "dualkv_bwd_workspace_bytes_tree",
           "dualkv_fwd_tree", "dualkv_bwd_tree", "dualkv_fwd_noalloc")
NOALLOC_SCRATCH_BYTES = 128 << 20   # DUALKV_NOALLOC_SCRATCH_BYTES
PHASE_PRE, PHASE_MAIN, PHASE_FINISH, PHASE_DQ, PHASE_ALL = 1, 2, 4, 8, 15

_lib = None


class DualKVError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (build it first if it was never built here)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    c_int, c_size, c_float, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.dualkv_fwd_workspace_bytes.restype = c_size
    lib.dualkv_fwd_workspace_bytes.argtypes = [c_int, c_int, c_int, i32p, c_int, c_int, c_int]
    lib.dualkv_bwd_workspace_bytes.restype = c_size
    lib.dualkv_bwd_workspace_bytes.argtypes = [c_int, c_int, c_int, i32p, c_int, c_int, c_int, c_int]
    lib.dualkv_fwd.restype = c_int
    lib.dualkv_fwd.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, i32p, c_int, c_int, c_int,
                               c_float, vp, c_size, vp]
    lib.dualkv_bwd.restype = c_int
    lib.dualkv_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, i32p,
                               c_int, c_int, c_int, c_float, c_int, vp, c_size, vp]
    lib.dualkv_bwd_phases.restype = c_int
    lib.dualkv_bwd_phases.argtypes = lib.dualkv_bwd.argtypes + [c_int]
    gargs = [c_int, i32p, i32p, i32p, c_int, c_int, c_int]
    lib.dualkv_fwd_workspace_bytes_groups.restype = c_size
    lib.dualkv_fwd_workspace_bytes_groups.argtypes = gargs
    lib.dualkv_bwd_workspace_bytes_groups.restype = c_size
    lib.dualkv_bwd_workspace_bytes_groups.argtypes = gargs + [c_int]
    lib.dualkv_fwd_groups.restype = c_int
    lib.dualkv_fwd_groups.argtypes = [vp, vp, vp, vp, vp] + gargs + [c_float, vp, c_size, vp]
    lib.dualkv_bwd_groups.restype = c_int
    lib.dualkv_bwd_groups.argtypes = [vp] * 9 + gargs + [c_float, c_int, vp, c_size, vp]
    targs = [c_int, i32p, i32p, c_int, c_int, c_int]
    lib.dualkv_fwd_workspace_bytes_tree.restype = c_size
    lib.dualkv_fwd_workspace_bytes_tree.argtypes = targs
    lib.dualkv_bwd_workspace_bytes_tree.restype = c_size
    lib.dualkv_bwd_workspace_bytes_tree.argtypes = targs + [c_int]
    lib.dualkv_fwd_tree.restype = c_int
    lib.dualkv_fwd_tree.argtypes = [vp, vp, vp, vp, vp] + targs + [c_float, vp, c_size, vp]
    lib.dualkv_bwd_tree.restype = c_int
    lib.dualkv_bwd_tree.argtypes = [vp] * 9 + targs + [c_float, c_int, vp, c_size, vp]
    lib.dualkv_fwd_noalloc.restype = c_int
    lib.dualkv_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, i32p, c_int, c_int,
                                       c_int, c_float, vp]
    lib.dualkv_status_string.restype = ctypes.c_char_p
    lib.dualkv_status_string.argtypes = [c_int]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dualkv_status_string(status).decode()


def _check(status: int) -> None:
    if status != OK:
        raise DualKVError(status, status_string(status))


class Packing:
    """P and the response lengths, as the ABI wants them (R or offsets)."""

    def __init__(self, P: int, lengths: Optional[Sequence[int]] = None, R: Optional[int] = None,
                 N: Optional[int] = None):
        self.P = int(P)
        if lengths is None:
            if R is None or N is None:
                raise ValueError("give lengths, or both R and N")
            lengths = [int(R)] * int(N)
        self.lengths = [int(x) for x in lengths]
        self.N = len(self.lengths)
        self.uniform = self.N > 0 and all(x == self.lengths[0] for x in self.lengths)
        self.R = self.lengths[0] if self.uniform else 0
        offs = [self.P]
        for x in self.lengths:
            offs.append(offs[-1] + x)
        self.T = offs[-1]
        self._offsets = (ctypes.c_int32 * (self.N + 1))(*offs)
        self._ws = {}  # workspace sizes already asked of the library

    def offsets_ptr(self):
        if self.uniform:
            return None
        return ctypes.cast(self._offsets, ctypes.POINTER(ctypes.c_int32))


class GroupPacking:
    """Several shared-prompt groups packed back to back: groups is a sequence
    of (P_b, response lengths of group b)."""

    def __init__(self, groups: Sequence):
        self.groups = [(int(P), [int(x) for x in L]) for P, L in groups]
        self.B = len(self.groups)
        self.T = sum(P + sum(L) for P, L in self.groups)
        n_resp = sum(len(L) for _, L in self.groups)
        self._P = (ctypes.c_int32 * max(1, self.B))(*[P for P, _ in self.groups])
        self._N = (ctypes.c_int32 * max(1, self.B))(*[len(L) for _, L in self.groups])
        self._R = (ctypes.c_int32 * max(1, n_resp))(*[x for _, L in self.groups for x in L])
        self._ws = {}

    def args(self):
        i32p = ctypes.POINTER(ctypes.c_int32)
        return (self.B, ctypes.cast(self._P, i32p), ctypes.cast(self._N, i32p),
                ctypes.cast(self._R, i32p))


class TreePacking:
    """Segments of a prefix forest in depth-first order: node_len[i] rows each,
    node_parent[i] = parent segment (-1 for a root)."""

    def __init__(self, node_len: Sequence[int], node_parent: Sequence[int]):
        self.node_len = [int(x) for x in node_len]
        self.node_parent = [int(x) for x in node_parent]
        self.n = len(self.node_len)
        self.T = sum(self.node_len)
        self._len = (ctypes.c_int32 * max(1, self.n))(*self.node_len)
        self._par = (ctypes.c_int32 * max(1, self.n))(*self.node_parent)
        self._ws = {}

    def args(self):
        i32p = ctypes.POINTER(ctypes.c_int32)
        return (self.n, ctypes.cast(self._len, i32p), ctypes.cast(self._par, i32p))


def _stream_ptr(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _alloc_on(stream):
    """Context for the tensors a call allocates (outputs, workspace): they come
    from the launch stream's pool, so the caching allocator cannot hand their
    memory to other work before the kernels enqueued on that stream ran."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _workspace(ws, nbytes: int, device):
    """The caller's workspace if it is a contiguous uint8 tensor of at least
    nbytes on `device`, else a fresh one (allocated under _alloc_on)."""
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"workspace: expected a contiguous uint8 tensor on {device}, got "
                         f"{ws.dtype} on {ws.device}" + ("" if ws.is_contiguous() else " (strided)"))
    if ws.numel() < nbytes:
        raise ValueError(f"workspace: {ws.numel()} bytes, the call needs {nbytes}")
    return ws


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, shape, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")


def fwd_workspace_bytes(pk: Packing, Hq: int, Hkv: int, d: int) -> int:
    key = ("fwd", Hq, Hkv, d)
    if key in pk._ws:
        return pk._ws[key]
    n = load().dualkv_fwd_workspace_bytes(pk.P, pk.R, pk.N, pk.offsets_ptr(), Hq, Hkv, d)
    pk._ws[key] = n
    if n == 0:
        raise DualKVError(ERR_INVALID_ARG, "invalid problem shape")
    return n


def bwd_workspace_bytes(pk: Packing, Hq: int, Hkv: int, d: int, deterministic: bool = False) -> int:
    key = ("bwd", Hq, Hkv, d, bool(deterministic))
    if key in pk._ws:
        return pk._ws[key]
    n = load().dualkv_bwd_workspace_bytes(pk.P, pk.R, pk.N, pk.offsets_ptr(), Hq, Hkv, d,
                                          int(deterministic))
    pk._ws[key] = n
    if n == 0:
        raise DualKVError(ERR_INVALID_ARG, "invalid problem shape")
    return n


def _fwd_common(q, k, v, T: int, scale, out, lse, workspace, stream, nws_fn):
    """Checks and allocations shared by the forward wrappers; returns
    (Hq, Hkv, d, scale, out, lse, workspace)."""
    _, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _check_tensor("q", q, (T, Hq, d), torch.bfloat16, dev)
    _check_tensor("k", k, (T, Hkv, d), torch.bfloat16, dev)
    _check_tensor("v", v, (T, Hkv, d), torch.bfloat16, dev)
    scale = d ** -0.5 if scale is None else scale
    nws = nws_fn(Hq, Hkv, d)
    with _alloc_on(stream):
        out = torch.empty_like(q) if out is None else out
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev) if lse is None else lse
        workspace = _workspace(workspace, nws, dev)
    _check_tensor("o", out, (T, Hq, d), torch.bfloat16, dev)
    _check_tensor("lse", lse, (Hq, T), torch.float32, dev)
    return Hq, Hkv, d, scale, out, lse, workspace


def _bwd_common(q, k, v, o, lse, do, T: int, scale, dq, dk, dv, workspace, stream, nws_fn):
    """Checks and allocations shared by the backward wrappers; returns
    (Hq, Hkv, d, scale, dq, dk, dv, workspace)."""
    _, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t, hh in (("q", q, Hq), ("o", o, Hq), ("do", do, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        _check_tensor(name, t, (T, hh, d), torch.bfloat16, dev)
    _check_tensor("lse", lse, (Hq, T), torch.float32, dev)
    scale = d ** -0.5 if scale is None else scale
    nws = nws_fn(Hq, Hkv, d)
    with _alloc_on(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        workspace = _workspace(workspace, nws, dev)
    for name, t, hh in (("dq", dq, Hq), ("dk", dk, Hkv), ("dv", dv, Hkv)):
        _check_tensor(name, t, (T, hh, d), torch.bfloat16, dev)
    return Hq, Hkv, d, scale, dq, dk, dv, workspace


def _cached_ws(cache: dict, key, query) -> int:
    if key not in cache:
        cache[key] = query()
    n = cache[key]
    if n == 0:
        raise DualKVError(ERR_INVALID_ARG, "invalid problem shape")
    return n


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pk: Packing,
        scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
        stream=None):
    """dualkv_fwd. q [T,Hq,d], k/v [T,Hkv,d] bf16 on the GPU -> (o, lse)."""
    Hq, Hkv, d, scale, out, lse, workspace = _fwd_common(
        q, k, v, pk.T, scale, out, lse, workspace, stream,
        lambda Hq, Hkv, d: fwd_workspace_bytes(pk, Hq, Hkv, d))
    _check(load().dualkv_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), pk.P, pk.R, pk.N,
                             pk.offsets_ptr(), Hq, Hkv, d, float(scale), _ptr(workspace),
                             workspace.numel(), _stream_ptr(stream)))
    return out, lse


def bwd(q, k, v, o, lse, do, pk: Packing, scale: Optional[float] = None,
        dq=None, dk=None, dv=None, workspace=None, deterministic: bool = False, stream=None,
        phases: int = PHASE_ALL):
    """dualkv_bwd -> (dq, dk, dv), bf16, same layouts as q, k, v.

    phases selects a subset of the backward's stream-ordered phases
    (dualkv_bwd_phases: PHASE_PRE, PHASE_MAIN (dK, dV), PHASE_DQ, PHASE_FINISH);
    the outputs are complete only once all of them ran on the same workspace,
    PHASE_PRE first and PHASE_MAIN before PHASE_FINISH."""
    Hq, Hkv, d, scale, dq, dk, dv, workspace = _bwd_common(
        q, k, v, o, lse, do, pk.T, scale, dq, dk, dv, workspace, stream,
        lambda Hq, Hkv, d: bwd_workspace_bytes(pk, Hq, Hkv, d, deterministic))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            pk.P, pk.R, pk.N, pk.offsets_ptr(), Hq, Hkv, d, float(scale), int(deterministic),
            _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    if phases == PHASE_ALL:
        _check(load().dualkv_bwd(*args))
    else:
        _check(load().dualkv_bwd_phases(*args, int(phases)))
    return dq, dk, dv


def fwd_groups(q, k, v, gp: GroupPacking, scale: Optional[float] = None, out=None, lse=None,
               workspace=None, stream=None):
    """dualkv_fwd_groups -> (o, lse); layouts as fwd()."""
    Hq, Hkv, d, scale, out, lse, workspace = _fwd_common(
        q, k, v, gp.T, scale, out, lse, workspace, stream,
        lambda Hq, Hkv, d: _cached_ws(gp._ws, ("fwd", Hq, Hkv, d),
                                      lambda: load().dualkv_fwd_workspace_bytes_groups(*gp.args(), Hq, Hkv, d)))
    _check(load().dualkv_fwd_groups(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *gp.args(),
                                    Hq, Hkv, d, float(scale), _ptr(workspace), workspace.numel(),
                                    _stream_ptr(stream)))
    return out, lse


def bwd_groups(q, k, v, o, lse, do, gp: GroupPacking, scale: Optional[float] = None,
               dq=None, dk=None, dv=None, workspace=None, deterministic: bool = False,
               stream=None):
    """dualkv_bwd_groups -> (dq, dk, dv); layouts as bwd()."""
    Hq, Hkv, d, scale, dq, dk, dv, workspace = _bwd_common(
        q, k, v, o, lse, do, gp.T, scale, dq, dk, dv, workspace, stream,
        lambda Hq, Hkv, d: _cached_ws(gp._ws, ("bwd", Hq, Hkv, d, bool(deterministic)),
                                      lambda: load().dualkv_bwd_workspace_bytes_groups(
                                          *gp.args(), Hq, Hkv, d, int(deterministic))))
    _check(load().dualkv_bwd_groups(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                    _ptr(dq), _ptr(dk), _ptr(dv), *gp.args(), Hq, Hkv, d,
                                    float(scale), int(deterministic), _ptr(workspace),
                                    workspace.numel(), _stream_ptr(stream)))
    return dq, dk, dv


def fwd_tree(q, k, v, tp: TreePacking, scale: Optional[float] = None, out=None, lse=None,
             workspace=None, stream=None):
    """dualkv_fwd_tree -> (o, lse); layouts as fwd()."""
    Hq, Hkv, d, scale, out, lse, workspace = _fwd_common(
        q, k, v, tp.T, scale, out, lse, workspace, stream,
        lambda Hq, Hkv, d: _cached_ws(tp._ws, ("fwd", Hq, Hkv, d),
                                      lambda: load().dualkv_fwd_workspace_bytes_tree(*tp.args(), Hq, Hkv, d)))
    _check(load().dualkv_fwd_tree(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *tp.args(),
                                  Hq, Hkv, d, float(scale), _ptr(workspace), workspace.numel(),
                                  _stream_ptr(stream)))
    return out, lse


def bwd_tree(q, k, v, o, lse, do, tp: TreePacking, scale: Optional[float] = None,
             dq=None, dk=None, dv=None, workspace=None, deterministic: bool = False, stream=None):
    """dualkv_bwd_tree -> (dq, dk, dv); layouts as bwd()."""
    Hq, Hkv, d, scale, dq, dk, dv, workspace = _bwd_common(
        q, k, v, o, lse, do, tp.T, scale, dq, dk, dv, workspace, stream,
        lambda Hq, Hkv, d: _cached_ws(tp._ws, ("bwd", Hq, Hkv, d, bool(deterministic)),
                                      lambda: load().dualkv_bwd_workspace_bytes_tree(
                                          *tp.args(), Hq, Hkv, d, int(deterministic))))
    _check(load().dualkv_bwd_tree(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                  _ptr(dq), _ptr(dk), _ptr(dv), *tp.args(), Hq, Hkv, d,
                                  float(scale), int(deterministic), _ptr(workspace),
                                  workspace.numel(), _stream_ptr(stream)))
    return dq, dk, dv


def fwd_noalloc(q, k, v, pk: Packing, scale: Optional[float] = None, out=None, lse=None, stream=None):
    """dualkv_fwd_noalloc -> (o, lse): the forward with the library's fixed
    device scratch instead of a workspace (the library call allocates nothing;
    o and lse are allocated here only if not given)."""
    _, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t, hh in (("q", q, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        _check_tensor(name, t, (pk.T, hh, d), torch.bfloat16, dev)
    scale = d ** -0.5 if scale is None else scale
    with _alloc_on(stream):
        out = torch.empty_like(q) if out is None else out
        lse = torch.empty((Hq, pk.T), dtype=torch.float32, device=dev) if lse is None else lse
    _check_tensor("o", out, (pk.T, Hq, d), torch.bfloat16, dev)
    _check_tensor("lse", lse, (Hq, pk.T), torch.float32, dev)
    _check(load().dualkv_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), pk.P, pk.R,
                                     pk.N, pk.offsets_ptr(), Hq, Hkv, d, float(scale),
                                     _stream_ptr(stream)))
    return out, lse


class DualKVAttention(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in libdualkv."""

    @staticmethod
    def forward(ctx, q, k, v, pk: Packing, scale=None):
        o, lse = fwd(q, k, v, pk, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.pk, ctx.scale = pk, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), ctx.pk, ctx.scale)
        return dq, dk, dv, None, None
