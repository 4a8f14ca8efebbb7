"""Python binding of libssmscan.so (the MI355X selective-scan library).

The functions named like the C ABI (``ssm_scan_create``,
``ssm_selective_scan_fwd``, ``ssd_chunk_scan_workspace_size``,
``ssd_chunk_scan_fwd``, ...) only marshal arguments: tensors become device
pointers, sizes come from tensor shapes, and the stream is PyTorch's current
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind.  If the library has not been built, every
call raises.

``selective_scan_fwd`` and ``ssd_chunk_scan`` are conveniences that also
allocate the outputs (and the SSD workspace) with PyTorch.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssmscan.so")

SSM_OK, SSM_ERR_INVALID_ARG, SSM_ERR_UNSUPPORTED, SSM_ERR_HIP = 0, 1, 2, 3
SSM_F32, SSM_BF16 = 0, 1

# Every symbol declared in include/ssm_scan.h.
EXPORTS = ("ssm_status_string", "ssm_last_error_message", "ssm_scan_create",
           "ssm_scan_destroy", "ssm_selective_scan_fwd", "ssm_selective_scan_fwd_with_state",
           "ssm_selective_scan_fwd_grouped", "ssm_selective_scan_fwd_workspace_size",
           "ssm_selective_scan_fwd_ws", "ssm_selective_scan_fwd_noalloc",
           "ssm_selective_state_update", "ssm_selective_state_update_grouped",
           "ssm_selective_scan_bwd_workspace_size",
           "ssm_selective_scan_bwd", "ssm_selective_scan_bwd_grouped_workspace_size",
           "ssm_selective_scan_bwd_grouped",
           "ssd_chunk_scan_workspace_size", "ssd_chunk_scan_fwd",
           "ssd_chunk_scan_fwd_with_state", "ssd_state_update")

_lib = None
_lib_lock = threading.Lock()
_handles: Dict[int, ctypes.c_void_p] = {}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class SsmScanError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} -- {message}")


def load_library() -> ctypes.CDLL:
    """Load libssmscan.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mamba_selective_scan_ssm_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.ssm_status_string.restype = ctypes.c_char_p
        lib.ssm_status_string.argtypes = [ctypes.c_int]
        lib.ssm_last_error_message.restype = ctypes.c_char_p
        lib.ssm_last_error_message.argtypes = []
        lib.ssm_scan_create.restype = ctypes.c_int
        lib.ssm_scan_create.argtypes = [ctypes.POINTER(_vp), ctypes.c_int]
        lib.ssm_scan_destroy.restype = ctypes.c_int
        lib.ssm_scan_destroy.argtypes = [_vp]
        lib.ssm_selective_scan_fwd.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp,
            _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssm_selective_scan_fwd_with_state.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_with_state.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
            _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssm_selective_scan_fwd_grouped.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_grouped.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
            _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssm_selective_scan_fwd_workspace_size.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_workspace_size.argtypes = [
            _vp, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssm_selective_scan_fwd_ws.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_ws.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
            _i64, _i64, _i64, _i64, _i64, _vp, ctypes.c_size_t, ctypes.c_int, _vp]
        lib.ssm_selective_scan_fwd_noalloc.restype = ctypes.c_int
        lib.ssm_selective_scan_fwd_noalloc.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
            _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssd_state_update.restype = ctypes.c_int
        lib.ssd_state_update.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
            _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssm_selective_state_update.restype = ctypes.c_int
        lib.ssm_selective_state_update.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
            _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssm_selective_state_update_grouped.restype = ctypes.c_int
        lib.ssm_selective_state_update_grouped.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
            _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssm_selective_scan_bwd_workspace_size.restype = ctypes.c_int
        lib.ssm_selective_scan_bwd_workspace_size.argtypes = [
            _vp, _i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssm_selective_scan_bwd.restype = ctypes.c_int
        lib.ssm_selective_scan_bwd.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
            _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssm_selective_scan_bwd_grouped_workspace_size.restype = ctypes.c_int
        lib.ssm_selective_scan_bwd_grouped_workspace_size.argtypes = [
            _vp, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssm_selective_scan_bwd_grouped.restype = ctypes.c_int
        lib.ssm_selective_scan_bwd_grouped.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
            _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssd_chunk_scan_workspace_size.restype = ctypes.c_int
        lib.ssd_chunk_scan_workspace_size.argtypes = [
            _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssd_chunk_scan_fwd.restype = ctypes.c_int
        lib.ssd_chunk_scan_fwd.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
            ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        lib.ssd_chunk_scan_fwd_with_state.restype = ctypes.c_int
        lib.ssd_chunk_scan_fwd_with_state.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
            ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().ssm_status_string(int(status)).decode()


ssm_status_string = status_string


def ssm_last_error_message() -> str:
    return load_library().ssm_last_error_message().decode()


def _check(fn: str, status: int) -> None:
    if status != SSM_OK:
        raise SsmScanError(fn, status, ssm_last_error_message())


# ---------------------------------------------------------------------------
# Raw C-ABI mirrors (pointers and sizes)
# ---------------------------------------------------------------------------

def ssm_scan_create(device: int) -> ctypes.c_void_p:
    h = _vp()
    _check("ssm_scan_create", load_library().ssm_scan_create(ctypes.byref(h), int(device)))
    return h


def ssm_scan_destroy(handle) -> None:
    _check("ssm_scan_destroy", load_library().ssm_scan_destroy(handle))


def get_handle(device: int) -> ctypes.c_void_p:
    """Process-wide handle for a device (created on first use)."""
    with _lib_lock:
        h = _handles.get(device)
    if h is None:
        h = ssm_scan_create(device)
        with _lib_lock:
            _handles.setdefault(device, h)
            h = _handles[device]
    return h


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need_cuda_contig(name, t, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class _Spec:
    """Expected dtype and shape of the tensors of one call, checked before
    anything reaches the library (the C ABI sees only pointers and sizes, so
    a tensor smaller than its sizes say would be read past its end)."""

    def __init__(self, fn: str):
        self.fn = fn
        self.device = None

    def _fail(self, msg):
        raise ValueError(f"{self.fn}: {msg}")

    def tensor(self, name, t, dtype=None, shape=None, optional=False):
        import torch
        if t is None:
            if optional:
                return
            self._fail(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            self._fail(f"{name} must be a torch.Tensor")
        if dtype is not None and t.dtype != dtype:
            self._fail(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
            self._fail(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if self.device is None:
            self.device = t.device
        elif t.device != self.device:
            self._fail(f"{name} is on {t.device}, other tensors on {self.device}")

    def in_dtype(self, name, t):
        """The input dtype of the call (float32 or bfloat16), from `t`."""
        import torch
        self.tensor(name, t)
        if t.dtype not in (torch.float32, torch.bfloat16):
            self._fail(f"{name} must be float32 or bfloat16, got {t.dtype}")
        return t.dtype

    def ndim(self, name, t, n):
        self.tensor(name, t)
        if t.dim() != n:
            self._fail(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _mamba1_spec(fn, u, delta, A, B, C, D, z, delta_bias, y, last_state, initial_state=None,
                 grouped=None):
    """Checks the Mamba-1 forward tensors; returns (batch, dim, dstate,
    seqlen, ngroups).  grouped: True = B, C must be [batch, ngroups, dstate,
    seqlen]; False = [batch, dstate, seqlen]; None = either."""
    import torch
    sp = _Spec(fn)
    dt = sp.in_dtype("u", u)
    sp.ndim("u", u, 3)
    batch, dim, seqlen = (int(v) for v in u.shape)
    sp.ndim("A", A, 2)
    dstate = int(A.shape[1])
    f32 = torch.float32
    sp.tensor("A", A, f32, (dim, dstate))
    sp.tensor("delta", delta, dt, u.shape)
    four = B is not None and B.dim() == 4
    if grouped is True and not four:
        sp._fail(f"B must be [batch, ngroups, dstate, seqlen], got {tuple(B.shape)}")
    if grouped is False and four:
        sp._fail(f"B must be [batch, dstate, seqlen], got {tuple(B.shape)}")
    if four:
        ngroups = int(B.shape[1])
        if ngroups < 1 or dim % ngroups:
            sp._fail(f"ngroups {ngroups} must divide dim {dim}")
        bshape = (batch, ngroups, dstate, seqlen)
    else:
        ngroups = 1
        bshape = (batch, dstate, seqlen)
    sp.tensor("B", B, dt, bshape)
    sp.tensor("C", C, dt, bshape)
    sp.tensor("D", D, f32, (dim,), optional=True)
    sp.tensor("z", z, dt, u.shape, optional=True)
    sp.tensor("delta_bias", delta_bias, f32, (dim,), optional=True)
    sp.tensor("initial_state", initial_state, f32, (batch, dim, dstate), optional=True)
    sp.tensor("y", y, dt, u.shape)
    sp.tensor("last_state", last_state, f32, (batch, dim, dstate), optional=True)
    return batch, dim, dstate, seqlen, ngroups


def _ssd_spec(fn, x, dt, A, B, C, D, dt_bias, y, final_state, initial_state=None,
              workspace=None):
    """Checks the SSD chunked-scan tensors; returns (batch, seqlen, nheads,
    headdim, dstate, ngroups)."""
    import torch
    sp = _Spec(fn)
    ty = sp.in_dtype("x", x)
    sp.ndim("x", x, 4)
    batch, seqlen, nheads, headdim = (int(v) for v in x.shape)
    sp.ndim("B", B, 4)
    ngroups, dstate = int(B.shape[2]), int(B.shape[3])
    f32 = torch.float32
    sp.tensor("dt", dt, ty, (batch, seqlen, nheads))
    sp.tensor("A", A, f32, (nheads,))
    sp.tensor("B", B, ty, (batch, seqlen, ngroups, dstate))
    sp.tensor("C", C, ty, (batch, seqlen, ngroups, dstate))
    sp.tensor("D", D, f32, (nheads,), optional=True)
    sp.tensor("dt_bias", dt_bias, f32, (nheads,), optional=True)
    sp.tensor("initial_state", initial_state, f32, (batch, nheads, headdim, dstate),
              optional=True)
    sp.tensor("y", y, ty, x.shape)
    sp.tensor("final_state", final_state, f32, (batch, nheads, headdim, dstate), optional=True)
    if workspace is not None:
        sp.tensor("workspace", workspace, torch.uint8)
    return batch, seqlen, nheads, headdim, dstate, ngroups


def _stream_ptr(device) -> int:
    import torch
    return int(torch.cuda.current_stream(device).cuda_stream)


def ssm_selective_scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, y,
                           last_state, handle=None) -> None:
    """Enqueue the Mamba-1 scan on the current stream (tensor form of the C
    entry point of the same name; y and last_state are caller-allocated)."""
    _mamba1_spec("ssm_selective_scan_fwd", u, delta, A, B, C, D, z, delta_bias, y, last_state,
                 grouped=False)
    for name, t, opt in (("u", u, False), ("delta", delta, False), ("A", A, False),
                         ("B", B, False), ("C", C, False), ("D", D, True), ("z", z, True),
                         ("delta_bias", delta_bias, True), ("y", y, False),
                         ("last_state", last_state, True)):
        _need_cuda_contig(name, t, opt)
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    dev = u.device.index if u.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    st = load_library().ssm_selective_scan_fwd(
        handle, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), _ptr(last_state),
        batch, dim, dstate, seqlen, _dtype_code(u), _stream_ptr(u.device))
    _check("ssm_selective_scan_fwd", st)


def ssm_selective_scan_fwd_with_state(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                      initial_state, y, last_state, handle=None) -> None:
    """ssm_selective_scan_fwd with an initial state [batch, dim, dstate]
    float32 (None = zero; may be last_state itself for an in-place update)."""
    _mamba1_spec("ssm_selective_scan_fwd_with_state", u, delta, A, B, C, D, z, delta_bias, y,
                 last_state, initial_state, grouped=False)
    for name, t, opt in (("u", u, False), ("delta", delta, False), ("A", A, False),
                         ("B", B, False), ("C", C, False), ("D", D, True), ("z", z, True),
                         ("delta_bias", delta_bias, True), ("initial_state", initial_state, True),
                         ("y", y, False), ("last_state", last_state, True)):
        _need_cuda_contig(name, t, opt)
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    dev = u.device.index if u.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    st = load_library().ssm_selective_scan_fwd_with_state(
        handle, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state), _ptr(y),
        _ptr(last_state), batch, dim, dstate, seqlen, _dtype_code(u), _stream_ptr(u.device))
    _check("ssm_selective_scan_fwd_with_state", st)


def ssm_selective_scan_fwd_grouped(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                   initial_state, y, last_state, handle=None) -> None:
    """ssm_selective_scan_fwd_with_state with B, C [batch, ngroups, dstate,
    seqlen]: channel d reads group d // (dim // ngroups)."""
    _mamba1_spec("ssm_selective_scan_fwd_grouped", u, delta, A, B, C, D, z, delta_bias, y,
                 last_state, initial_state, grouped=True)
    for name, t, opt in (("u", u, False), ("delta", delta, False), ("A", A, False),
                         ("B", B, False), ("C", C, False), ("D", D, True), ("z", z, True),
                         ("delta_bias", delta_bias, True), ("initial_state", initial_state, True),
                         ("y", y, False), ("last_state", last_state, True)):
        _need_cuda_contig(name, t, opt)
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    if B.dim() != 4 or C.shape != B.shape or tuple(B.shape) != (batch, B.shape[1], dstate, seqlen):
        raise ValueError("B and C must be [batch, ngroups, dstate, seqlen], got "
                         f"{tuple(B.shape)} and {tuple(C.shape)}")
    dev = u.device.index if u.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    st = load_library().ssm_selective_scan_fwd_grouped(
        handle, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state), _ptr(y),
        _ptr(last_state), batch, dim, dstate, seqlen, B.shape[1], _dtype_code(u),
        _stream_ptr(u.device))
    _check("ssm_selective_scan_fwd_grouped", st)


def ssm_selective_scan_fwd_workspace_size(batch, dim, dstate, seqlen, ngroups=1, device=0,
                                          handle=None) -> int:
    """Workspace bytes ssm_selective_scan_fwd_ws can use (0: none needed)."""
    if handle is None:
        handle = get_handle(device)
    out = ctypes.c_size_t(0)
    st = load_library().ssm_selective_scan_fwd_workspace_size(
        handle, batch, dim, dstate, seqlen, ngroups, ctypes.byref(out))
    _check("ssm_selective_scan_fwd_workspace_size", st)
    return int(out.value)


def ssm_selective_scan_fwd_ws(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                              initial_state, y, last_state, workspace, handle=None) -> None:
    """ssm_selective_scan_fwd_grouped with a device workspace (uint8 tensor or
    None).  B, C: [batch, dstate, seqlen] or [batch, ngroups, dstate, seqlen]."""
    _mamba1_spec("ssm_selective_scan_fwd_ws", u, delta, A, B, C, D, z, delta_bias, y, last_state,
                 initial_state)
    if workspace is not None:
        import torch
        if workspace.dtype != torch.uint8:
            raise ValueError("ssm_selective_scan_fwd_ws: workspace must be a uint8 tensor")
    for name, t, opt in (("u", u, False), ("delta", delta, False), ("A", A, False),
                         ("B", B, False), ("C", C, False), ("D", D, True), ("z", z, True),
                         ("delta_bias", delta_bias, True), ("initial_state", initial_state, True),
                         ("y", y, False), ("last_state", last_state, True),
                         ("workspace", workspace, True)):
        _need_cuda_contig(name, t, opt)
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    ngroups = B.shape[1] if B.dim() == 4 else 1
    dev = u.device.index if u.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().ssm_selective_scan_fwd_ws(
        handle, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state), _ptr(y),
        _ptr(last_state), batch, dim, dstate, seqlen, ngroups, _ptr(workspace), nbytes,
        _dtype_code(u), _stream_ptr(u.device))
    _check("ssm_selective_scan_fwd_ws", st)


def ssm_selective_scan_fwd_noalloc(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                   initial_state, y, last_state, handle=None) -> None:
    """ssm_selective_scan_fwd_ws without a workspace argument: the time split
    uses the library's per-GPU scratch array, so the call allocates nothing
    (calls on one GPU that overlap in time race on that scratch).  B, C:
    [batch, dstate, seqlen] or [batch, ngroups, dstate, seqlen]."""
    _, _, _, _, ngroups = _mamba1_spec("ssm_selective_scan_fwd_noalloc", u, delta, A, B, C, D,
                                       z, delta_bias, y, last_state, initial_state)
    for name, t, opt in (("u", u, False), ("delta", delta, False), ("A", A, False),
                         ("B", B, False), ("C", C, False), ("D", D, True), ("z", z, True),
                         ("delta_bias", delta_bias, True), ("initial_state", initial_state, True),
                         ("y", y, False), ("last_state", last_state, True)):
        _need_cuda_contig(name, t, opt)
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    dev = u.device.index if u.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    st = load_library().ssm_selective_scan_fwd_noalloc(
        handle, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state), _ptr(y),
        _ptr(last_state), batch, dim, dstate, seqlen, ngroups, _dtype_code(u),
        _stream_ptr(u.device))
    _check("ssm_selective_scan_fwd_noalloc", st)


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=True, return_last_state=True, initial_state=None,
                       time_split=True):
    """Allocating form: returns (y, last_state or None).  B and C are
    [batch, dstate, seqlen], or [batch, ngroups, dstate, seqlen] (grouped).
    With time_split, a workspace is allocated when the rows alone would
    leave the device idle (ssm_selective_scan_fwd_ws)."""
    import torch
    y = torch.empty_like(u)
    ls = (torch.empty((u.shape[0], u.shape[1], A.shape[1]), dtype=torch.float32,
                      device=u.device) if return_last_state else None)
    if time_split:
        ngroups = B.shape[1] if B.dim() == 4 else 1
        dev = u.device.index if u.device.index is not None else 0
        nbytes = ssm_selective_scan_fwd_workspace_size(u.shape[0], u.shape[1], A.shape[1],
                                                       u.shape[2], ngroups, device=dev)
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=u.device)
            ssm_selective_scan_fwd_ws(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                      initial_state, y, ls, ws)
            return y, ls
    if B.dim() == 4:
        ssm_selective_scan_fwd_grouped(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                       initial_state, y, ls)
    elif initial_state is None:
        ssm_selective_scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, y, ls)
    else:
        ssm_selective_scan_fwd_with_state(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                          initial_state, y, ls)
    return y, ls


def ssm_selective_state_update(state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, y,
                               handle=None) -> None:
    """One decode step, state [batch, dim, dstate] float32 updated in place;
    u, delta, z, y: [batch, dim]; B, C: [batch, dstate], or [batch, ngroups,
    dstate] (ssm_selective_state_update_grouped: channel d reads group
    d // (dim // ngroups))."""
    import torch
    fn = ("ssm_selective_state_update_grouped" if getattr(B, "dim", lambda: 0)() == 3
          else "ssm_selective_state_update")
    sp = _Spec(fn)
    ty = sp.in_dtype("u", u)
    sp.ndim("u", u, 2)
    sp.ndim("A", A, 2)
    batch, dim = (int(v) for v in u.shape)
    dstate = int(A.shape[1])
    grouped = fn.endswith("_grouped")
    ngroups = int(B.shape[1]) if grouped else 1
    if ngroups < 1 or dim % ngroups:
        raise ValueError(f"{fn}: B has {ngroups} groups, which must divide dim {dim}")
    bc = (batch, ngroups, dstate) if grouped else (batch, dstate)
    f32 = torch.float32
    sp.tensor("A", A, f32, (dim, dstate))
    sp.tensor("state", state, f32, (batch, dim, dstate))
    sp.tensor("delta", delta, ty, (batch, dim))
    sp.tensor("B", B, ty, bc)
    sp.tensor("C", C, ty, bc)
    sp.tensor("D", D, f32, (dim,), optional=True)
    sp.tensor("z", z, ty, (batch, dim), optional=True)
    sp.tensor("delta_bias", delta_bias, f32, (dim,), optional=True)
    sp.tensor("y", y, ty, (batch, dim))
    for name, t, opt in (("state", state, False), ("u", u, False), ("delta", delta, False),
                         ("A", A, False), ("B", B, False), ("C", C, False), ("D", D, True),
                         ("z", z, True), ("delta_bias", delta_bias, True), ("y", y, False)):
        _need_cuda_contig(name, t, opt)
    batch, dim = u.shape
    dstate = A.shape[1]
    dev = u.device.index if u.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    args = [handle, _ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), batch, dim, dstate]
    if grouped:
        args.append(ngroups)
    st = getattr(load_library(), fn)(*args, _dtype_code(u), _stream_ptr(u.device))
    _check(fn, st)


def ssm_selective_scan_bwd_workspace_size(batch, dim, dstate, seqlen, handle=None,
                                          device: int = 0) -> int:
    if handle is None:
        handle = get_handle(device)
    n = ctypes.c_size_t()
    st = load_library().ssm_selective_scan_bwd_workspace_size(handle, batch, dim, dstate, seqlen,
                                                              ctypes.byref(n))
    _check("ssm_selective_scan_bwd_workspace_size", st)
    return int(n.value)


def ssm_selective_scan_bwd_grouped_workspace_size(batch, dim, dstate, seqlen, ngroups,
                                                  handle=None, device: int = 0) -> int:
    if handle is None:
        handle = get_handle(device)
    n = ctypes.c_size_t()
    st = load_library().ssm_selective_scan_bwd_grouped_workspace_size(
        handle, batch, dim, dstate, seqlen, ngroups, ctypes.byref(n))
    _check("ssm_selective_scan_bwd_grouped_workspace_size", st)
    return int(n.value)


def ssm_selective_scan_bwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, initial_state,
                           dy, dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                           dinitial_state, workspace, handle=None) -> None:
    """Enqueue the Mamba-1 backward pass (tensor form of the C entry point;
    every gradient and the workspace are caller-allocated)."""
    _bwd_call("ssm_selective_scan_bwd", False, u, delta, A, B, C, D, z, delta_bias,
              delta_softplus, initial_state, dy, dlast_state, du, ddelta, dA, dB, dC, dD, dz,
              ddelta_bias, dinitial_state, workspace, handle)


def ssm_selective_scan_bwd_grouped(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                   initial_state, dy, dlast_state, du, ddelta, dA, dB, dC, dD,
                                   dz, ddelta_bias, dinitial_state, workspace,
                                   handle=None) -> None:
    """The backward pass with B, C (and dB, dC) [batch, ngroups, dstate,
    seqlen]."""
    _bwd_call("ssm_selective_scan_bwd_grouped", True, u, delta, A, B, C, D, z, delta_bias,
              delta_softplus, initial_state, dy, dlast_state, du, ddelta, dA, dB, dC, dD, dz,
              ddelta_bias, dinitial_state, workspace, handle)


def _bwd_call(fn, grouped, u, delta, A, B, C, D, z, delta_bias, delta_softplus, initial_state,
              dy, dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state,
              workspace, handle):
    import torch
    batch, dim, dstate, seqlen, ngroups = _mamba1_spec(
        fn, u, delta, A, B, C, D, z, delta_bias, du, None, initial_state, grouped=grouped)
    bc_shape = (batch, ngroups, dstate, seqlen) if grouped else (batch, dstate, seqlen)
    sp = _Spec(fn)
    f32 = torch.float32
    sp.tensor("dy", dy, u.dtype, u.shape)
    sp.tensor("dlast_state", dlast_state, f32, (batch, dim, dstate), optional=True)
    sp.tensor("ddelta", ddelta, u.dtype, u.shape)
    sp.tensor("dz", dz, u.dtype, u.shape, optional=z is None)
    sp.tensor("dA", dA, f32, (dim, dstate))
    sp.tensor("dB", dB, f32, bc_shape)
    sp.tensor("dC", dC, f32, bc_shape)
    sp.tensor("dD", dD, f32, (dim,), optional=True)
    sp.tensor("ddelta_bias", ddelta_bias, f32, (dim,), optional=True)
    sp.tensor("dinitial_state", dinitial_state, f32, (batch, dim, dstate), optional=True)
    sp.tensor("workspace", workspace, torch.uint8)
    for name, t, opt in (("u", u, False), ("delta", delta, False), ("A", A, False),
                         ("B", B, False), ("C", C, False), ("D", D, True), ("z", z, True),
                         ("delta_bias", delta_bias, True), ("initial_state", initial_state, True),
                         ("dy", dy, False), ("dlast_state", dlast_state, True),
                         ("du", du, False), ("ddelta", ddelta, False), ("dA", dA, False),
                         ("dB", dB, False), ("dC", dC, False), ("dD", dD, True), ("dz", dz, True),
                         ("ddelta_bias", ddelta_bias, True),
                         ("dinitial_state", dinitial_state, True),
                         ("workspace", workspace, False)):
        _need_cuda_contig(name, t, opt)
    dev = u.device.index if u.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    args = [handle, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state), _ptr(dy),
            _ptr(dlast_state), _ptr(du), _ptr(ddelta), _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD),
            _ptr(dz), _ptr(ddelta_bias), _ptr(dinitial_state), _ptr(workspace),
            workspace.numel() * workspace.element_size(), batch, dim, dstate, seqlen]
    if grouped:
        args.append(ngroups)
    st = getattr(load_library(), fn)(*args, _dtype_code(u), _stream_ptr(u.device))
    _check(fn, st)


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                       delta_softplus=True, initial_state=None, dlast_state=None):
    """Allocating form: returns a dict of gradients (du, ddelta, dz in the
    input dtype; dA, dB, dC, dD, ddelta_bias, dinitial_state float32; the
    optional ones are None when their input is None).  B, C may be
    [batch, ngroups, dstate, seqlen] (the grouped entry point; dB, dC then
    have that shape)."""
    import torch
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    dev = u.device
    grouped = B.dim() == 4
    ngroups = int(B.shape[1]) if grouped else 1
    bc_shape = (batch, ngroups, dstate, seqlen) if grouped else (batch, dstate, seqlen)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u),
         "dA": torch.empty((dim, dstate), **f32), "dB": torch.empty(bc_shape, **f32),
         "dC": torch.empty(bc_shape, **f32),
         "dD": torch.empty((dim,), **f32) if D is not None else None,
         "dz": torch.empty_like(u) if z is not None else None,
         "ddelta_bias": torch.empty((dim,), **f32) if delta_bias is not None else None,
         "dinitial_state": (torch.empty((batch, dim, dstate), **f32)
                            if initial_state is not None else None)}
    nbytes = ssm_selective_scan_bwd_grouped_workspace_size(
        batch, dim, dstate, seqlen, ngroups, device=dev.index if dev.index is not None else 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    call = ssm_selective_scan_bwd_grouped if grouped else ssm_selective_scan_bwd
    call(u, delta, A, B, C, D, z, delta_bias, delta_softplus, initial_state, dy, dlast_state,
         g["du"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"], g["ddelta_bias"],
         g["dinitial_state"], ws)
    return g


_SCAN_FN = None


def _scan_function():
    """torch.autograd.Function over the forward and backward entry points
    (built on first use so that importing this module needs no torch)."""
    global _SCAN_FN
    if _SCAN_FN is not None:
        return _SCAN_FN
    import torch

    class SelectiveScanFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, u, delta, A, B, C, D, z, delta_bias, initial_state, delta_softplus):
            ins = [None if t is None else t.contiguous()
                   for t in (u, delta, A, B, C, D, z, delta_bias, initial_state)]
            y, ls = selective_scan_fwd(*ins[:5], D=ins[5], z=ins[6], delta_bias=ins[7],
                                       delta_softplus=delta_softplus, initial_state=ins[8])
            ctx.save_for_backward(*[t if t is not None else torch.empty(0) for t in ins])
            ctx.present = [t is not None for t in ins]
            ctx.delta_softplus = delta_softplus
            return y, ls

        @staticmethod
        def backward(ctx, dy, dls):
            ins = [t if p else None for t, p in zip(ctx.saved_tensors, ctx.present)]
            u, delta, A, B, C, D, z, delta_bias, h0 = ins
            dy = torch.zeros_like(u) if dy is None else dy.to(u.dtype).contiguous()
            dls = None if dls is None else dls.float().contiguous()
            g = selective_scan_bwd(u, delta, A, B, C, dy, D=D, z=z, delta_bias=delta_bias,
                                   delta_softplus=ctx.delta_softplus, initial_state=h0,
                                   dlast_state=dls)
            cast = lambda t, like: None if t is None else t.to(like.dtype)
            return (g["du"], g["ddelta"], cast(g["dA"], A), cast(g["dB"], B), cast(g["dC"], C),
                    cast(g["dD"], D) if D is not None else None,
                    g["dz"] if z is not None else None,
                    cast(g["ddelta_bias"], delta_bias) if delta_bias is not None else None,
                    cast(g["dinitial_state"], h0) if h0 is not None else None, None)

    _SCAN_FN = SelectiveScanFn
    return _SCAN_FN


def selective_scan_fn(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                      initial_state=None, return_last_state=False):
    """Differentiable Mamba-1 selective scan: the forward and backward HIP
    kernels behind torch.autograd (B, C [batch, dstate, seqlen] or grouped
    [batch, ngroups, dstate, seqlen]; the backward takes dstate <= 64 and
    groups of whole backward workgroups).  Returns y, or (y, last_state)."""
    y, ls = _scan_function().apply(u, delta, A, B, C, D, z, delta_bias, initial_state,
                                   bool(delta_softplus))
    return (y, ls) if return_last_state else y


def ssd_state_update(state, x, dt, A, B, C, D, dt_bias, dt_softplus, y, handle=None) -> None:
    """One SSD decode step in place: state [batch, nheads, headdim, dstate]
    float32; x, y [batch, nheads, headdim]; dt [batch, nheads]; B, C
    [batch, ngroups, dstate]; A, D, dt_bias [nheads]."""
    import torch
    sp = _Spec("ssd_state_update")
    ty = sp.in_dtype("x", x)
    sp.ndim("x", x, 3)
    sp.ndim("B", B, 3)
    batch, nheads, headdim = (int(v) for v in x.shape)
    ngroups, dstate = int(B.shape[1]), int(B.shape[2])
    f32 = torch.float32
    sp.tensor("state", state, f32, (batch, nheads, headdim, dstate))
    sp.tensor("dt", dt, ty, (batch, nheads))
    sp.tensor("A", A, f32, (nheads,))
    sp.tensor("B", B, ty, (batch, ngroups, dstate))
    sp.tensor("C", C, ty, (batch, ngroups, dstate))
    sp.tensor("D", D, f32, (nheads,), optional=True)
    sp.tensor("dt_bias", dt_bias, f32, (nheads,), optional=True)
    sp.tensor("y", y, ty, x.shape)
    for name, t, opt in (("state", state, False), ("x", x, False), ("dt", dt, False),
                         ("A", A, False), ("B", B, False), ("C", C, False), ("D", D, True),
                         ("dt_bias", dt_bias, True), ("y", y, False)):
        _need_cuda_contig(name, t, opt)
    batch, nheads, headdim = x.shape
    ngroups, dstate = B.shape[1], B.shape[2]
    dev = x.device.index if x.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    st = load_library().ssd_state_update(
        handle, _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(dt_bias), int(bool(dt_softplus)), _ptr(y), batch, nheads, headdim, dstate,
        ngroups, _dtype_code(x), _stream_ptr(x.device))
    _check("ssd_state_update", st)


def ssd_chunk_scan_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups,
                                  chunk_size, handle=None, device: int = 0) -> int:
    if handle is None:
        handle = get_handle(device)
    n = ctypes.c_size_t()
    st = load_library().ssd_chunk_scan_workspace_size(
        handle, batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, ctypes.byref(n))
    _check("ssd_chunk_scan_workspace_size", st)
    return int(n.value)


def ssd_chunk_scan_fwd(x, dt, A, B, C, D, dt_bias, dt_softplus, y, final_state, workspace,
                       chunk_size, handle=None) -> None:
    """Enqueue the Mamba-2 chunked scan on the current stream (tensor form of
    the C entry point; y, final_state and workspace are caller-allocated)."""
    _ssd_spec("ssd_chunk_scan_fwd", x, dt, A, B, C, D, dt_bias, y, final_state,
              workspace=workspace)
    for name, t, opt in (("x", x, False), ("dt", dt, False), ("A", A, False), ("B", B, False),
                         ("C", C, False), ("D", D, True), ("dt_bias", dt_bias, True),
                         ("y", y, False), ("final_state", final_state, True),
                         ("workspace", workspace, False)):
        _need_cuda_contig(name, t, opt)
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    dev = x.device.index if x.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    st = load_library().ssd_chunk_scan_fwd(
        handle, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
        int(bool(dt_softplus)), _ptr(y), _ptr(final_state), _ptr(workspace),
        workspace.numel() * workspace.element_size(), batch, seqlen, nheads, headdim, dstate,
        ngroups, chunk_size, _dtype_code(x), _stream_ptr(x.device))
    _check("ssd_chunk_scan_fwd", st)


def ssd_chunk_scan_fwd_with_state(x, dt, A, B, C, D, dt_bias, dt_softplus, initial_state, y,
                                  final_state, workspace, chunk_size, handle=None) -> None:
    """ssd_chunk_scan_fwd with an initial state [batch, nheads, headdim,
    dstate] float32 (None = zero; may be final_state itself)."""
    _ssd_spec("ssd_chunk_scan_fwd_with_state", x, dt, A, B, C, D, dt_bias, y, final_state,
              initial_state, workspace=workspace)
    for name, t, opt in (("x", x, False), ("dt", dt, False), ("A", A, False), ("B", B, False),
                         ("C", C, False), ("D", D, True), ("dt_bias", dt_bias, True),
                         ("initial_state", initial_state, True), ("y", y, False),
                         ("final_state", final_state, True), ("workspace", workspace, False)):
        _need_cuda_contig(name, t, opt)
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    dev = x.device.index if x.device.index is not None else 0
    if handle is None:
        handle = get_handle(dev)
    st = load_library().ssd_chunk_scan_fwd_with_state(
        handle, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
        int(bool(dt_softplus)), _ptr(initial_state), _ptr(y), _ptr(final_state), _ptr(workspace),
        workspace.numel() * workspace.element_size(), batch, seqlen, nheads, headdim, dstate,
        ngroups, chunk_size, _dtype_code(x), _stream_ptr(x.device))
    _check("ssd_chunk_scan_fwd_with_state", st)


def ssd_chunk_scan(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True, chunk_size=256,
                   return_final_state=True, initial_state=None) -> Tuple:
    """Allocating form: returns (y, final_state or None)."""
    import torch
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    dev = x.device.index if x.device.index is not None else 0
    nbytes = ssd_chunk_scan_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups,
                                           chunk_size, device=dev)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    y = torch.empty_like(x)
    fs = (torch.empty((batch, nheads, headdim, dstate), dtype=torch.float32, device=x.device)
          if return_final_state else None)
    if initial_state is None:
        ssd_chunk_scan_fwd(x, dt, A, B, C, D, dt_bias, dt_softplus, y, fs, ws, chunk_size)
    else:
        ssd_chunk_scan_fwd_with_state(x, dt, A, B, C, D, dt_bias, dt_softplus, initial_state, y,
                                      fs, ws, chunk_size)
    return y, fs
