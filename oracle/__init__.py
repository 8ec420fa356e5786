"""Plain CPU oracle for the Mamba-2 SSD forward pass (double precision).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library.  The arithmetic lives in ``ssd_oracle.c`` (see its
header for the definitions and the passages of the pages each function
follows); this module only builds that file with gcc and marshals numpy
arrays into it.

All array arguments are numpy arrays; floating inputs are converted to
contiguous float32 (bfloat16 values widen to float32 exactly) and outputs are
float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compiles ssd_oracle.c into libssd_oracle.so with gcc and OpenMP."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk_size")]


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_chunk_cumsum.argtypes = [ctypes.POINTER(_Dims), P, P, P, P]
        lib.oracle_ssd_recurrence.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P,
                                              ctypes.c_int, P, P, P, P]
        lib.oracle_chunk_local_states.argtypes = [ctypes.POINTER(_Dims), P, P, P, P,
                                                  ctypes.c_int, P, P]
        lib.oracle_state_passing.argtypes = [ctypes.c_int64] * 5 + [P, P, P, P, P]
        lib.oracle_chunk_outputs.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P,
                                             ctypes.c_int, P, P, P]
        lib.oracle_ssd_backward.argtypes = [ctypes.POINTER(_Dims)] + [P] * 16
        lib.oracle_num_threads.restype = ctypes.c_int
        for f in ("oracle_chunk_cumsum", "oracle_ssd_recurrence", "oracle_chunk_local_states",
                  "oracle_state_passing", "oracle_chunk_outputs", "oracle_ssd_backward"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(x, B, chunk_size):
    Bn, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return _Dims(Bn, L, H, P, N, G, int(chunk_size))


def _heads(nheads, heads):
    if heads is None:
        return nheads, None
    h = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    return int(h.size), h


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (rc={rc})")


def chunk_cumsum(dt, A, chunk_size):
    """dA_cs, dt_T, both [B,H,nc,Q] float64 (log2 units for dA_cs)."""
    dt = _f32(dt)
    A = _f32(A)
    Bn, L, H = dt.shape
    nc = -(-L // chunk_size)
    d = _Dims(Bn, L, H, 1, 1, 1, int(chunk_size))
    cs = np.empty((Bn, H, nc, chunk_size), np.float64)
    dtt = np.empty_like(cs)
    _check(_load().oracle_chunk_cumsum(ctypes.byref(d), _ptr(dt), _ptr(A), _ptr(cs), _ptr(dtt)),
           "oracle_chunk_cumsum")
    return cs, dtt


def ssd_recurrence(x, dt, A, B, C, D=None, h0=None, *, chunk_size=64, heads=None,
                   want_final=True, want_hstart=False):
    """Direct recurrence.  Returns (y[B,L,k,P], final[B,k,P,N] or None,
    h_start[B,nc,k,P,N] or None) for the selected heads (all by default)."""
    x, dt, A, B, C, D, h0 = map(_f32, (x, dt, A, B, C, D, h0))
    d = _dims(x, B, chunk_size)
    nsel, hsel = _heads(d.nheads, heads)
    nc = -(-d.seqlen // chunk_size)
    y = np.empty((d.batch, d.seqlen, nsel, d.headdim), np.float64)
    fin = np.empty((d.batch, nsel, d.headdim, d.dstate), np.float64) if want_final else None
    hs = (np.empty((d.batch, nc, nsel, d.headdim, d.dstate), np.float64)
          if want_hstart else None)
    _check(_load().oracle_ssd_recurrence(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                         _ptr(C), _ptr(D), _ptr(h0), nsel, _ptr(hsel), _ptr(y),
                                         _ptr(fin), _ptr(hs)), "oracle_ssd_recurrence")
    return y, fin, hs


def chunk_local_states(x, dt, A, B, *, chunk_size, heads=None):
    """Per-chunk zero-start end states S[B,nc,k,P,N]."""
    x, dt, A, B = map(_f32, (x, dt, A, B))
    d = _dims(x, B, chunk_size)
    nsel, hsel = _heads(d.nheads, heads)
    nc = -(-d.seqlen // chunk_size)
    S = np.empty((d.batch, nc, nsel, d.headdim, d.dstate), np.float64)
    _check(_load().oracle_chunk_local_states(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A),
                                             _ptr(B), nsel, _ptr(hsel), _ptr(S)),
           "oracle_chunk_local_states")
    return S


def state_passing(S, decay, h0=None):
    """h_start[B,nc,H,P,N], final[B,H,P,N] from S[B,nc,H,P,N] and decay[B,H,nc]."""
    S = np.ascontiguousarray(np.asarray(S, np.float64))
    decay = np.ascontiguousarray(np.asarray(decay, np.float64))
    h0 = None if h0 is None else np.ascontiguousarray(np.asarray(h0, np.float64))
    Bn, nc, H, P, N = S.shape
    hs = np.empty_like(S)
    fin = np.empty((Bn, H, P, N), np.float64)
    _check(_load().oracle_state_passing(Bn, nc, H, P, N, _ptr(S), _ptr(decay), _ptr(h0),
                                        _ptr(hs), _ptr(fin)), "oracle_state_passing")
    return hs, fin


def chunk_outputs(x, dt, A, B, C, D, h_start, *, chunk_size, heads=None):
    """y[B,L,k,P] of each chunk restarted from h_start[B,nc,k,P,N]."""
    x, dt, A, B, C, D = map(_f32, (x, dt, A, B, C, D))
    h_start = np.ascontiguousarray(np.asarray(h_start, np.float64))
    d = _dims(x, B, chunk_size)
    nsel, hsel = _heads(d.nheads, heads)
    y = np.empty((d.batch, d.seqlen, nsel, d.headdim), np.float64)
    _check(_load().oracle_chunk_outputs(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                        _ptr(C), _ptr(D), nsel, _ptr(hsel), _ptr(h_start),
                                        _ptr(y)), "oracle_chunk_outputs")
    return y


def ssd_backward(x, dt, A, B, C, D, h0, dy, dfinal=None, *, chunk_size=64):
    """Gradients of sum(dy * y) + sum(dfinal * final) with respect to every
    input of ssd_recurrence, by back-propagation through the recurrence.
    Returns a dict of float64 arrays: dx, ddt, dA, dB, dC (group gradients,
    the heads of each group summed), dD (None when D is None) and dh0 (None
    when h0 is None)."""
    x, dt, A, B, C, D, h0, dy, dfinal = map(_f32, (x, dt, A, B, C, D, h0, dy, dfinal))
    d = _dims(x, B, chunk_size)
    Bn, L, H, P, N, G = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.ngroups
    assert dy.shape == x.shape
    dx = np.empty((Bn, L, H, P), np.float64)
    ddt = np.empty((Bn, L, H), np.float64)
    dBh = np.empty((Bn, L, H, N), np.float64)
    dCh = np.empty((Bn, L, H, N), np.float64)
    dA_part = np.empty((Bn, H), np.float64)
    dD_part = np.empty((Bn, H), np.float64)
    dh0 = np.empty((Bn, H, P, N), np.float64) if h0 is not None else None
    _check(_load().oracle_ssd_backward(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                       _ptr(C), _ptr(D), _ptr(h0), _ptr(dy), _ptr(dfinal),
                                       _ptr(dx), _ptr(ddt), _ptr(dBh), _ptr(dCh), _ptr(dA_part),
                                       _ptr(dD_part), _ptr(dh0)), "oracle_ssd_backward")
    hpg = H // G
    return {"dx": dx, "ddt": ddt, "dA": dA_part.sum(0),
            "dB": dBh.reshape(Bn, L, G, hpg, N).sum(3),
            "dC": dCh.reshape(Bn, L, G, hpg, N).sum(3),
            "dD": dD_part.sum(0) if D is not None else None, "dh0": dh0}
