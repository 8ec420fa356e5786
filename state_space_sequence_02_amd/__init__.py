"""Python binding of the MI355X (gfx950) Mamba-2 SSD forward-pass library.

Thin ctypes marshalling over ``libmamba2_ssd.so`` (C ABI in
``include/mamba2_ssd.h``): every step of the forward pass runs in the HIP
kernels; this module only turns torch tensors into device pointers and the
current torch stream into a ``hipStream_t``.  The functions keep the C names:

    mamba2_validate, mamba2_chunk_cumsum, mamba2_chunk_state,
    mamba2_state_passing, mamba2_chunk_scan, mamba2_ssd_workspace_bytes,
    mamba2_ssd_forward, mamba2_ssd_forward_profile, mamba2_status_string,
    mamba2_last_error

plus ``make_dims`` and ``ssd_forward`` (allocates outputs and workspace with
torch, then calls ``mamba2_ssd_forward``).  Importing fails loudly when the
library has not been built; there is no fallback implementation.

The C ABI receives bare pointers and can only check them for NULL and
alignment, so every wrapper here checks each torch tensor against the sizes
in ``dims`` first: dtype (x, dt, B, C, y and their gradients in the dims
dtype; A, D, states, sums and every state-shaped tensor float32), shape,
contiguity and that it lives on a GPU, raising ``Mamba2Error`` with
``MAMBA2_ERR_DTYPE``, ``MAMBA2_ERR_SHAPE`` or ``MAMBA2_ERR_NULL`` before any
call.  A plain ``int`` is taken as a raw device address and passed as is.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmamba2_ssd.so")

MAMBA2_OK = 0
MAMBA2_ERR_NULL = 1
MAMBA2_ERR_SHAPE = 2
MAMBA2_ERR_DTYPE = 3
MAMBA2_ERR_UNSUPPORTED = 4
MAMBA2_ERR_ALIGN = 5
MAMBA2_ERR_WORKSPACE = 6
MAMBA2_ERR_HIP = 7

MAMBA2_DTYPE_F32 = 0
MAMBA2_DTYPE_BF16 = 1

EXPORTS = (
    "mamba2_validate", "mamba2_chunk_cumsum", "mamba2_chunk_state", "mamba2_state_passing",
    "mamba2_chunk_scan", "mamba2_ssd_workspace_bytes", "mamba2_ssd_forward",
    "mamba2_ssd_forward_profile", "mamba2_fwd_pass_state", "mamba2_ssd_forward_fused",
    "mamba2_decode_step", "mamba2_ssd_backward_workspace_bytes",
    "mamba2_ssd_backward", "mamba2_ssd_backward_profile", "mamba2_status_string",
    "mamba2_last_error", "mamba2_ssd_forward_noalloc",
)

# bytes of the static per-GPU scratch behind mamba2_ssd_forward_noalloc
NOALLOC_SCRATCH_BYTES = 128 << 20


class Mamba2Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("chunk_size", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]

    def __repr__(self):
        return "Mamba2Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class Mamba2Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str | None = None):
        self.status = status
        if detail is None:
            detail = mamba2_last_error()
        super().__init__(f"{where}: {mamba2_status_string(status)} ({detail})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python __graft_entry__.py build` "
            "(or state_space_sequence_02_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(Mamba2Dims)
    sig = {
        "mamba2_validate": ([D], ctypes.c_int),
        "mamba2_chunk_cumsum": ([D, P, P, P, P, P], ctypes.c_int),
        "mamba2_chunk_state": ([D, P, P, P, P, P, P], ctypes.c_int),
        "mamba2_state_passing": ([D, P, P, P, P, P], ctypes.c_int),
        "mamba2_chunk_scan": ([D, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "mamba2_ssd_workspace_bytes": ([D], ctypes.c_size_t),
        "mamba2_ssd_forward": ([D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P], ctypes.c_int),
        "mamba2_ssd_forward_profile": ([D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P,
                                        ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "mamba2_ssd_forward_noalloc": ([D, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "mamba2_decode_step": ([D, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "mamba2_fwd_pass_state": ([D, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "mamba2_ssd_forward_fused": ([D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P],
                                     ctypes.c_int),
        "mamba2_ssd_backward_workspace_bytes": ([D], ctypes.c_size_t),
        "mamba2_ssd_backward": ([D] + [P] * 17 + [ctypes.c_size_t, P], ctypes.c_int),
        "mamba2_ssd_backward_profile": ([D] + [P] * 17 + [ctypes.c_size_t, P, P], ctypes.c_int),
        "mamba2_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "mamba2_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MAMBA2_OK:
        raise Mamba2Error(status, where)


def _io_dtype(dims):
    return torch.float32 if dims.dtype == MAMBA2_DTYPE_F32 else torch.bfloat16


def _nchunks(dims):
    return -(-dims.seqlen // dims.chunk_size)


def _shapes(dims):
    """Expected (shape, dtype) of every tensor role for these dims."""
    b, L, H, P, N, G = (dims.batch, dims.seqlen, dims.nheads, dims.headdim, dims.dstate,
                        dims.ngroups)
    nc, Q, io, f = _nchunks(dims), dims.chunk_size, _io_dtype(dims), torch.float32
    return {
        "x": ((b, L, H, P), io), "y": ((b, L, H, P), io), "dt": ((b, L, H), io),
        "A": ((H,), f), "D": ((H,), f), "B": ((b, L, G, N), io), "C": ((b, L, G, N), io),
        "state": ((b, H, P, N), f), "sums": ((b, H, nc, Q), f),
        "states": ((b, nc, H, P, N), f), "start_bf16": ((b, nc, H, P, N), torch.bfloat16),
        # one-token step: the sequence axis is absent
        "x1": ((b, H, P), io), "dt1": ((b, H), io), "B1": ((b, G, N), io),
    }


def _req(where, dims, role, name, t, optional=False):
    """Checks one argument: None only if optional; an int passes as a raw
    device address; a tensor must match its role's dtype and shape and be
    contiguous (the device is checked for all arguments at once, after)."""
    if t is None:
        if optional:
            return
        raise Mamba2Error(MAMBA2_ERR_NULL, where, f"{name} is None")
    if isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise Mamba2Error(MAMBA2_ERR_SHAPE, where, f"{name} is a {type(t).__name__}, not a tensor")
    shape, dtype = _shapes(dims)[role]
    if t.dtype != dtype:
        raise Mamba2Error(MAMBA2_ERR_DTYPE, where, f"{name} is {t.dtype}, needs {dtype}")
    if tuple(t.shape) != shape:
        raise Mamba2Error(MAMBA2_ERR_SHAPE, where,
                          f"{name} has shape {tuple(t.shape)}, needs {shape}")
    if not t.is_contiguous():
        raise Mamba2Error(MAMBA2_ERR_SHAPE, where,
                          f"{name} is not contiguous (strides {t.stride()})")


def _req_bytes(where, name, t, nbytes):
    """A workspace: raw address, or a contiguous GPU tensor of at least nbytes."""
    if t is None:
        raise Mamba2Error(MAMBA2_ERR_WORKSPACE, where, f"{name} is None")
    if isinstance(t, int):
        return
    if not t.is_contiguous():
        raise Mamba2Error(MAMBA2_ERR_WORKSPACE, where, f"{name} is not contiguous")
    if t.numel() * t.element_size() < int(nbytes):
        raise Mamba2Error(MAMBA2_ERR_WORKSPACE, where,
                          f"{name} holds {t.numel() * t.element_size()} bytes, "
                          f"{int(nbytes)} passed")


def _same_device(where, *ts):
    """After the per-tensor checks: every tensor on one GPU."""
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    off = sorted(str(d) for d in devs if d.type != "cuda")
    if off:
        raise Mamba2Error(MAMBA2_ERR_NULL, where, f"tensors on {off}, not on a GPU")
    if len(devs) > 1:
        raise Mamba2Error(MAMBA2_ERR_NULL, where,
                          f"tensors on different GPUs: {sorted(map(str, devs))}")


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype) -> Mamba2Dims:
    """dtype: torch.float32 / torch.bfloat16 or the MAMBA2_DTYPE_* code."""
    if dtype is torch.float32:
        dtype = MAMBA2_DTYPE_F32
    elif dtype is torch.bfloat16:
        dtype = MAMBA2_DTYPE_BF16
    return Mamba2Dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, int(dtype), 0)


def dims_of(x: torch.Tensor, B: torch.Tensor, chunk_size: int) -> Mamba2Dims:
    """Dims from x[B,L,H,P] and B[B,L,G,N] (the dtype is x's: float32 or
    bfloat16; every other tensor is then checked against these dims)."""
    if x.dim() != 4 or B.dim() != 4:
        raise Mamba2Error(MAMBA2_ERR_SHAPE, "dims_of",
                          f"x {tuple(x.shape)} and B {tuple(B.shape)} must both be 4-d")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise Mamba2Error(MAMBA2_ERR_DTYPE, "dims_of", f"x is {x.dtype}, needs float32 or bfloat16")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(B.shape[:2]) != (b, L):
        raise Mamba2Error(MAMBA2_ERR_SHAPE, "dims_of",
                          f"B {tuple(B.shape)} does not match x {tuple(x.shape)} in batch/seqlen")
    return make_dims(b, L, H, P, N, G, chunk_size, x.dtype)


def mamba2_validate(dims) -> int:
    return int(_lib.mamba2_validate(ctypes.byref(dims)))


def mamba2_status_string(status: int) -> str:
    return _lib.mamba2_status_string(int(status)).decode()


def mamba2_last_error() -> str:
    return _lib.mamba2_last_error().decode()


def mamba2_ssd_workspace_bytes(dims) -> int:
    return int(_lib.mamba2_ssd_workspace_bytes(ctypes.byref(dims)))


def mamba2_chunk_cumsum(dims, dt, A, dA_cs, dt_T, stream=None):
    w = "mamba2_chunk_cumsum"
    for role, name, t in (("dt", "dt", dt), ("A", "A", A), ("sums", "dA_cs", dA_cs),
                          ("sums", "dt_T", dt_T)):
        _req(w, dims, role, name, t)
    _same_device(w, dt, A, dA_cs, dt_T)
    _check(_lib.mamba2_chunk_cumsum(ctypes.byref(dims), _ptr(dt), _ptr(A), _ptr(dA_cs),
                                    _ptr(dt_T), _stream(stream)), "mamba2_chunk_cumsum")


def mamba2_chunk_state(dims, x, B, dA_cs, dt_T, states, stream=None):
    w = "mamba2_chunk_state"
    for role, name, t in (("x", "x", x), ("B", "B", B), ("sums", "dA_cs", dA_cs),
                          ("sums", "dt_T", dt_T), ("states", "states", states)):
        _req(w, dims, role, name, t)
    _same_device(w, x, B, dA_cs, dt_T, states)
    _check(_lib.mamba2_chunk_state(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(dA_cs), _ptr(dt_T),
                                   _ptr(states), _stream(stream)), "mamba2_chunk_state")


def mamba2_state_passing(dims, states, dA_cs, init_state, final_state, stream=None):
    w = "mamba2_state_passing"
    _req(w, dims, "states", "states", states)
    _req(w, dims, "sums", "dA_cs", dA_cs)
    _req(w, dims, "state", "init_state", init_state, optional=True)
    _req(w, dims, "state", "final_state", final_state, optional=True)
    _same_device(w, states, dA_cs, init_state, final_state)
    _check(_lib.mamba2_state_passing(ctypes.byref(dims), _ptr(states), _ptr(dA_cs),
                                     _ptr(init_state), _ptr(final_state), _stream(stream)),
           "mamba2_state_passing")


def mamba2_chunk_scan(dims, x, B, C, dA_cs, dt_T, states, D, y, stream=None):
    w = "mamba2_chunk_scan"
    for role, name, t in (("x", "x", x), ("B", "B", B), ("C", "C", C), ("sums", "dA_cs", dA_cs),
                          ("sums", "dt_T", dt_T), ("states", "states", states), ("y", "y", y)):
        _req(w, dims, role, name, t)
    _req(w, dims, "D", "D", D, optional=True)
    _same_device(w, x, B, C, dA_cs, dt_T, states, D, y)
    _check(_lib.mamba2_chunk_scan(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(C), _ptr(dA_cs),
                                  _ptr(dt_T), _ptr(states), _ptr(D), _ptr(y), _stream(stream)),
           "mamba2_chunk_scan")


def _forward_args(w, dims, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                  workspace_bytes):
    for role, name, t in (("x", "x", x), ("dt", "dt", dt), ("A", "A", A), ("B", "B", B),
                          ("C", "C", C), ("y", "y", y)):
        _req(w, dims, role, name, t)
    _req(w, dims, "D", "D", D, optional=True)
    _req(w, dims, "state", "init_state", init_state, optional=True)
    _req(w, dims, "state", "final_state", final_state, optional=True)
    _req_bytes(w, "workspace", workspace, workspace_bytes)
    _same_device(w, x, dt, A, B, C, D, init_state, y, final_state, workspace)


def mamba2_ssd_forward(dims, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                       workspace_bytes, stream=None):
    _forward_args("mamba2_ssd_forward", dims, x, dt, A, B, C, D, init_state, y, final_state,
                  workspace, workspace_bytes)
    _check(_lib.mamba2_ssd_forward(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                   _ptr(C), _ptr(D), _ptr(init_state), _ptr(y), _ptr(final_state),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "mamba2_ssd_forward")


def mamba2_ssd_forward_noalloc(dims, x, dt, A, B, C, D, init_state, y, final_state,
                               stream=None):
    """mamba2_ssd_forward with the library's static per-GPU scratch as the
    workspace (no allocation; calls that overlap on one GPU race)."""
    w = "mamba2_ssd_forward_noalloc"
    for role, name, t in (("x", "x", x), ("dt", "dt", dt), ("A", "A", A), ("B", "B", B),
                          ("C", "C", C), ("y", "y", y)):
        _req(w, dims, role, name, t)
    _req(w, dims, "D", "D", D, optional=True)
    _req(w, dims, "state", "init_state", init_state, optional=True)
    _req(w, dims, "state", "final_state", final_state, optional=True)
    _same_device(w, x, dt, A, B, C, D, init_state, y, final_state)
    _check(_lib.mamba2_ssd_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A),
                                           _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), _ptr(y),
                                           _ptr(final_state), _stream(stream)), w)


def mamba2_ssd_forward_profile(dims, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                               workspace_bytes, stream=None):
    """Runs mamba2_ssd_forward, waits, and returns the four stage durations in ms
    (chunk_cumsum, chunk_state, state_passing, chunk_scan)."""
    _forward_args("mamba2_ssd_forward_profile", dims, x, dt, A, B, C, D, init_state, y,
                  final_state, workspace, workspace_bytes)
    ms = (ctypes.c_float * 4)()
    _check(_lib.mamba2_ssd_forward_profile(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A),
                                           _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), _ptr(y),
                                           _ptr(final_state), _ptr(workspace),
                                           int(workspace_bytes), _stream(stream), ms),
           "mamba2_ssd_forward_profile")
    return [float(v) for v in ms]


def mamba2_fwd_pass_state(dims, x, B, dA_cs, dt_T, init_state, w_T, chunk_start_states,
                          final_state, stream=None):
    w = "mamba2_fwd_pass_state"
    for role, name, t in (("x", "x", x), ("B", "B", B), ("sums", "dA_cs", dA_cs),
                          ("sums", "dt_T", dt_T), ("sums", "w_T", w_T),
                          ("start_bf16", "chunk_start_states", chunk_start_states),
                          ("state", "final_state", final_state)):
        _req(w, dims, role, name, t)
    _req(w, dims, "state", "init_state", init_state, optional=True)
    _same_device(w, x, B, dA_cs, dt_T, init_state, w_T, chunk_start_states, final_state)
    _check(_lib.mamba2_fwd_pass_state(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(dA_cs),
                                      _ptr(dt_T), _ptr(init_state), _ptr(w_T),
                                      _ptr(chunk_start_states), _ptr(final_state),
                                      _stream(stream)),
           "mamba2_fwd_pass_state")


def mamba2_ssd_forward_fused(dims, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                             workspace_bytes, stream=None):
    _forward_args("mamba2_ssd_forward_fused", dims, x, dt, A, B, C, D, init_state, y,
                  final_state, workspace, workspace_bytes)
    _check(_lib.mamba2_ssd_forward_fused(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                         _ptr(C), _ptr(D), _ptr(init_state), _ptr(y),
                                         _ptr(final_state), _ptr(workspace),
                                         int(workspace_bytes), _stream(stream)),
           "mamba2_ssd_forward_fused")


def mamba2_decode_step(dims, x, dt, A, B, C, D, state, y, stream=None):
    w = "mamba2_decode_step"
    for role, name, t in (("x1", "x", x), ("dt1", "dt", dt), ("A", "A", A), ("B1", "B", B),
                          ("B1", "C", C), ("state", "state", state), ("x1", "y", y)):
        _req(w, dims, role, name, t)
    _req(w, dims, "D", "D", D, optional=True)
    _same_device(w, x, dt, A, B, C, D, state, y)
    _check(_lib.mamba2_decode_step(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                   _ptr(C), _ptr(D), _ptr(state), _ptr(y), _stream(stream)),
           "mamba2_decode_step")


def decode_step(x, dt, A, B, C, D, state, *, chunk_size=64, stream=None):
    """One token per (batch, head): x[B,H,P], dt[B,H], B/C[B,G,N]; updates the
    float32 state[B,H,P,N] in place and returns y[B,H,P] (allocated with torch)."""
    if x.dim() != 3 or B.dim() != 3:
        raise Mamba2Error(MAMBA2_ERR_SHAPE, "decode_step",
                          f"x {tuple(x.shape)} and B {tuple(B.shape)} must both be 3-d")
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dims = make_dims(b, 1, H, P, N, G, chunk_size, x.dtype)
    y = torch.empty_like(x)
    mamba2_decode_step(dims, x, dt, A, B, C, D, state, y, stream)
    return y


def ssd_forward(x, dt, A, B, C, D=None, init_state=None, *, chunk_size=256, workspace=None,
                stream=None):
    """Allocates y, the final state and (unless given) the workspace with torch on x's
    device, runs mamba2_ssd_forward, and returns (y, final_state)."""
    dims = dims_of(x, B, chunk_size)
    y = torch.empty_like(x)
    final = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]), dtype=torch.float32,
                        device=x.device)
    need = mamba2_ssd_workspace_bytes(dims)
    if need == 0:
        _check(mamba2_validate(dims), "ssd_forward")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    mamba2_ssd_forward(dims, x, dt, A, B, C, D, init_state, y, final, workspace,
                       workspace.numel() * workspace.element_size(), stream)
    return y, final


def mamba2_ssd_backward_workspace_bytes(dims) -> int:
    return int(_lib.mamba2_ssd_backward_workspace_bytes(ctypes.byref(dims)))


def _bwd_args(dims, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit,
              workspace, workspace_bytes, where="mamba2_ssd_backward"):
    for role, name, t in (("x", "x", x), ("dt", "dt", dt), ("A", "A", A), ("B", "B", B),
                          ("C", "C", C), ("y", "dy", dy), ("x", "dx", dx), ("dt", "ddt", ddt),
                          ("A", "dA", dA), ("B", "dB", dB), ("C", "dC", dC)):
        _req(where, dims, role, name, t)
    for role, name, t in (("D", "D", D), ("state", "init_state", init_state),
                          ("state", "dfinal", dfinal), ("D", "dD", dD), ("state", "dinit", dinit)):
        _req(where, dims, role, name, t, optional=True)
    _req_bytes(where, "workspace", workspace, workspace_bytes)
    _same_device(where, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit,
                 workspace)
    return (ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(init_state), _ptr(dy), _ptr(dfinal), _ptr(dx), _ptr(ddt), _ptr(dA), _ptr(dB),
            _ptr(dC), _ptr(dD), _ptr(dinit), _ptr(workspace), int(workspace_bytes))


def mamba2_ssd_backward(dims, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC,
                        dD, dinit, workspace, workspace_bytes, stream=None):
    _check(_lib.mamba2_ssd_backward(*_bwd_args(dims, x, dt, A, B, C, D, init_state, dy, dfinal,
                                               dx, ddt, dA, dB, dC, dD, dinit, workspace,
                                               workspace_bytes), _stream(stream)),
           "mamba2_ssd_backward")


def mamba2_ssd_backward_profile(dims, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA,
                                dB, dC, dD, dinit, workspace, workspace_bytes, stream=None):
    """Runs mamba2_ssd_backward, waits, and returns its eight stage durations in ms."""
    ms = (ctypes.c_float * 8)()
    _check(_lib.mamba2_ssd_backward_profile(*_bwd_args(dims, x, dt, A, B, C, D, init_state, dy,
                                                       dfinal, dx, ddt, dA, dB, dC, dD, dinit,
                                                       workspace, workspace_bytes,
                                                       "mamba2_ssd_backward_profile"),
                                            _stream(stream), ms),
           "mamba2_ssd_backward_profile")
    return [float(v) for v in ms]


def ssd_backward(x, dt, A, B, C, D, init_state, dy, dfinal=None, *, chunk_size=256,
                 workspace=None, stream=None):
    """Allocates the gradients (and, unless given, the workspace) with torch on x's
    device, runs mamba2_ssd_backward, and returns a dict with dx, ddt, dA, dB, dC,
    dD (None without D) and dinit."""
    dims = dims_of(x, B, chunk_size)
    need = mamba2_ssd_backward_workspace_bytes(dims)
    if need == 0:
        _check(mamba2_validate(dims), "ssd_backward")
        raise Mamba2Error(MAMBA2_ERR_UNSUPPORTED, "ssd_backward")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    dev = x.device
    g = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt),
         "dA": torch.empty_like(A), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
         "dD": torch.empty_like(D) if D is not None else None,
         "dinit": torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]),
                              dtype=torch.float32, device=dev)}
    mamba2_ssd_backward(dims, x, dt, A, B, C, D, init_state, dy, dfinal, g["dx"], g["ddt"],
                        g["dA"], g["dB"], g["dC"], g["dD"], g["dinit"], workspace,
                        workspace.numel() * workspace.element_size(), stream)
    return g


def stage_buffers(dims, device):
    """Allocates the per-stage intermediates: dA_cs, dt_T [B,H,nc,Q] and states
    [B,nc,H,P,N], all float32."""
    nc = -(-dims.seqlen // dims.chunk_size)
    cs = torch.empty((dims.batch, dims.nheads, nc, dims.chunk_size), dtype=torch.float32,
                     device=device)
    dtt = torch.empty_like(cs)
    st = torch.empty((dims.batch, nc, dims.nheads, dims.headdim, dims.dstate),
                     dtype=torch.float32, device=device)
    return cs, dtt, st
