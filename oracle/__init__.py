"""fp64 CPU oracle for the Mamba selective scan (Mamba-1) and its SSD form (Mamba-2).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product path (the HIP library and
its Python binding) never imports this package, and this package imports
nothing from the product path.

The arithmetic lives in ``ssm_oracle.c`` (plain C, double precision, one
sequential time loop per independent row).  This module only builds/loads it
and marshals numpy arrays.  Sources are cited in that file's header.

Build: ``python -m oracle.build`` or ``oracle.build_library()`` (gcc, -O2, no
fast-math, so every operation is IEEE double).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build_library() -> str:
    """Compile ssm_oracle.c into libssm_oracle.so next to it (always rebuilds)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build_library()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_selective_scan_f64.restype = ctypes.c_int
    lib.oracle_selective_scan_f64.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        _i64p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
    lib.oracle_selective_scan_h0_f64.restype = ctypes.c_int
    lib.oracle_selective_scan_h0_f64.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int, _f64p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        _i64p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
    lib.oracle_selective_scan_grouped_f64.restype = ctypes.c_int
    lib.oracle_selective_scan_grouped_f64.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int, _f64p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        _i64p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
    lib.oracle_selective_scan_bwd_grouped_f64.restype = ctypes.c_int
    lib.oracle_selective_scan_bwd_grouped_f64.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int,
        _f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64,
        _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int]
    lib.oracle_selective_scan_bwd_f64.restype = ctypes.c_int
    lib.oracle_selective_scan_bwd_f64.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int,
        _f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int]
    lib.oracle_ssd_h0_f64.restype = ctypes.c_int
    lib.oracle_ssd_h0_f64.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int, _f64p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
    lib.oracle_ssd_f64.restype = ctypes.c_int
    lib.oracle_ssd_f64.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
    _lib = lib
    return lib


def _f32(a, shape=None):
    """Contiguous float32 view (values must already be exactly float32)."""
    if a is None:
        return None
    arr = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {arr.shape}")
    return arr


def _p32(a):
    return None if a is None else a.ctypes.data_as(_f32p)


def default_threads() -> int:
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _f64(a, shape):
    if a is None:
        return None
    arr = np.ascontiguousarray(a, dtype=np.float64)
    if arr.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {arr.shape}")
    return arr


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   delta_softplus=True, rows=None, want_y=True,
                   want_state=True, nthreads=None, h0=None):
    """Mamba-1 selective scan in fp64.

    u, delta, z: [batch, dim, seqlen]; A: [dim, dstate]; B, C: [batch, dstate,
    seqlen], or [batch, ngroups, dstate, seqlen] with channel d reading group
    d // (dim // ngroups) (ngroups = dim: per-channel B and C);
    D, delta_bias: [dim]; h0: optional initial state [batch, dim, dstate]
    (float64; zero when None).  ``rows`` optionally restricts the
    work to flat row indices b*dim+d (outputs then follow that order).
    Returns (y [nrows, seqlen] or None, last_state [nrows, dstate] or None),
    both float64; with rows=None, nrows = batch*dim in (b, d) order.
    """
    lib = _load()
    u = _f32(u)
    batch, dim, seqlen = u.shape
    dstate = np.asarray(A).shape[1]
    ngroups = np.asarray(B).shape[1] if np.ndim(B) == 4 else 1
    delta = _f32(delta, (batch, dim, seqlen))
    A = _f32(A, (dim, dstate))
    if np.ndim(B) == 3:
        B = _f32(B, (batch, dstate, seqlen))
        C = _f32(C, (batch, dstate, seqlen))
    else:
        B = _f32(B, (batch, ngroups, dstate, seqlen))
        C = _f32(C, (batch, ngroups, dstate, seqlen))
    D = _f32(D, (dim,))
    z = _f32(z, (batch, dim, seqlen))
    delta_bias = _f32(delta_bias, (dim,))
    if rows is None:
        nrows = batch * dim
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.shape[0]
    y = np.empty((nrows, seqlen), np.float64) if want_y else None
    st = np.empty((nrows, dstate), np.float64) if want_state else None
    h0 = _f64(h0, (batch, dim, dstate))
    rc = lib.oracle_selective_scan_grouped_f64(
        _p32(u), _p32(delta), _p32(A), _p32(B), _p32(C), _p32(D), _p32(z),
        _p32(delta_bias), int(bool(delta_softplus)),
        None if h0 is None else h0.ctypes.data_as(_f64p), batch, dim, dstate, seqlen, ngroups,
        None if rows_arr is None else rows_arr.ctypes.data_as(_i64p), nrows,
        None if y is None else y.ctypes.data_as(_f64p),
        None if st is None else st.ctypes.data_as(_f64p),
        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan_f64 failed with code {rc}")
    return y, st


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, dlast=None, nthreads=None):
    """Gradients of selective_scan (y, last_state) in fp64 by reverse-mode
    differentiation of the sequential loop, for upstream gradients dy
    [batch, dim, seqlen] and dlast [batch, dim, dstate] (None = zero).

    B, C may be [batch, ngroups, dstate, seqlen] (channel d in group
    d // (dim // ngroups)); dB, dC then have that shape too.

    Returns a dict: du, ddelta, dz (None without z) [batch, dim, seqlen];
    dA [dim, dstate]; dB, dC [batch, dstate, seqlen] (or grouped); dD,
    ddelta_bias [dim]; dh0 [batch, dim, dstate].
    """
    lib = _load()
    u = _f32(u)
    batch, dim, seqlen = u.shape
    dstate = np.asarray(A).shape[1]
    grouped = np.ndim(B) == 4
    ngroups = np.asarray(B).shape[1] if grouped else 1
    bc_shape = (batch, ngroups, dstate, seqlen) if grouped else (batch, dstate, seqlen)
    delta = _f32(delta, (batch, dim, seqlen))
    A = _f32(A, (dim, dstate))
    B = _f32(B, bc_shape)
    C = _f32(C, bc_shape)
    D = _f32(D, (dim,))
    z = _f32(z, (batch, dim, seqlen))
    delta_bias = _f32(delta_bias, (dim,))
    h0 = _f64(h0, (batch, dim, dstate))
    dy = _f64(dy, (batch, dim, seqlen))
    dlast = _f64(dlast, (batch, dim, dstate))
    out = {k: np.empty(shape, np.float64) for k, shape in (
        ("du", (batch, dim, seqlen)), ("ddelta", (batch, dim, seqlen)),
        ("dA", (dim, dstate)), ("dB", bc_shape), ("dC", bc_shape),
        ("dD", (dim,)), ("ddelta_bias", (dim,)), ("dh0", (batch, dim, dstate)))}
    out["dz"] = np.empty((batch, dim, seqlen), np.float64) if z is not None else None
    p64 = lambda a: None if a is None else a.ctypes.data_as(_f64p)
    rc = lib.oracle_selective_scan_bwd_grouped_f64(
        _p32(u), _p32(delta), _p32(A), _p32(B), _p32(C), _p32(D), _p32(z), _p32(delta_bias),
        int(bool(delta_softplus)), p64(h0), p64(dy), p64(dlast), batch, dim, dstate, seqlen,
        ngroups,
        p64(out["du"]), p64(out["ddelta"]), p64(out["dA"]), p64(out["dB"]), p64(out["dC"]),
        p64(out["dD"]), p64(out["dz"]), p64(out["ddelta_bias"]), p64(out["dh0"]),
        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan_bwd_f64 failed with code {rc}")
    return out


def ssd_scan(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
             want_y=True, want_state=True, nthreads=None, initial_state=None):
    """Mamba-2 (scalar A per head) recurrence in fp64.

    x: [batch, seqlen, nheads, headdim]; dt: [batch, seqlen, nheads];
    A, D, dt_bias: [nheads]; B, C: [batch, seqlen, ngroups, dstate];
    initial_state: optional [batch, nheads, headdim, dstate] (float64; zero
    when None).
    Returns (y [batch, seqlen, nheads, headdim], final_state [batch, nheads,
    headdim, dstate]) as float64 (either may be None).
    """
    lib = _load()
    x = _f32(x)
    batch, seqlen, nheads, headdim = x.shape
    B = _f32(B)
    ngroups, dstate = B.shape[2], B.shape[3]
    if B.shape[:2] != (batch, seqlen):
        raise ValueError("B shape mismatch")
    dt = _f32(dt, (batch, seqlen, nheads))
    A = _f32(A, (nheads,))
    C = _f32(C, (batch, seqlen, ngroups, dstate))
    D = _f32(D, (nheads,))
    dt_bias = _f32(dt_bias, (nheads,))
    y = np.empty((batch, seqlen, nheads, headdim), np.float64) if want_y else None
    st = np.empty((batch, nheads, headdim, dstate), np.float64) if want_state else None
    init = _f64(initial_state, (batch, nheads, headdim, dstate))
    rc = lib.oracle_ssd_h0_f64(
        _p32(x), _p32(dt), _p32(A), _p32(B), _p32(C), _p32(D), _p32(dt_bias),
        int(bool(dt_softplus)), None if init is None else init.ctypes.data_as(_f64p),
        batch, seqlen, nheads, headdim, dstate, ngroups,
        None if y is None else y.ctypes.data_as(_f64p),
        None if st is None else st.ctypes.data_as(_f64p),
        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_ssd_f64 failed with code {rc}")
    return y, st
