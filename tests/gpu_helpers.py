"""Shared helpers of the GPU parity tests: moving seeded inputs to the GPU,
running the HIP stages through the C ABI, and the error measures."""
from __future__ import annotations

import sys

import numpy as np
import torch

import ssd_inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}
CUMSUM_TOL = 1e-6


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def normwise(got, ref):
    """max |got - ref| / max |ref| (absolute when ref is all zeros)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref).max() if got.size else 0.0
    scale = np.abs(ref).max() if ref.size else 0.0
    return float(err / scale) if scale > 0 else float(err)


def headwise(got, ref, head_axis):
    """The largest normwise error over (batch, head) slices: batch is axis 0,
    the head axis is given (y [B,L,H,P]: 2; final state [B,H,P,N]: 1; chunk
    states [B,nc,H,P,N]: 2).  A head whose values are much smaller than the
    tensor's largest is held to the same relative bar as the rest."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[head_axis]):
            gs = np.take(got[b], h, axis=head_axis - 1)
            rs = np.take(ref[b], h, axis=head_axis - 1)
            worst = max(worst, normwise(gs, rs))
    return worst


HEAD_AXIS = {"y": 2, "final_state": 1, "local_states": 2, "start_states": 2}


def errors(pairs):
    """{name: (tensor normwise, worst (batch, head) normwise)} for
    name -> (got, ref) pairs whose names are keys of HEAD_AXIS."""
    return {k: (normwise(g, r), headwise(g, r, HEAD_AXIS[k])) for k, (g, r) in pairs.items()}


def assert_within(errs, tol):
    """Every tensor and every (batch, head) slice of it within tol."""
    for k, (e_all, e_head) in errs.items():
        assert e_all <= tol, (k, "tensor", e_all, tol)
        assert e_head <= tol, (k, "worst head", e_head, tol)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def f32(t):
    return None if t is None else t.detach().float().cpu().numpy()


def to_gpu(inp):
    return {k: (None if v is None else v.cuda()) for k, v in inp.items()}


def oracle_inputs(inp):
    """float32 numpy views of the (dtype-rounded) inputs for the oracle."""
    return {k: f32(v) for k, v in inp.items()}


def workload_inputs(w: ssd_inputs.Workload, *, init_state=None):
    inp = ssd_inputs.make_inputs(w)
    if init_state is False:
        inp["init_state"] = None
    return inp


def run_forward(m2, inp_gpu, chunk_size):
    y, fin = m2.ssd_forward(inp_gpu["x"], inp_gpu["dt"], inp_gpu["A"], inp_gpu["B"],
                            inp_gpu["C"], inp_gpu["D"], inp_gpu["init_state"],
                            chunk_size=chunk_size)
    torch.cuda.synchronize()
    return y, fin


def run_stages(m2, inp_gpu, chunk_size):
    """Runs the four stage entry points; returns (dims, dA_cs, dt_T, local_states,
    start_states, final, y) with the states snapshot taken before state_passing."""
    x = inp_gpu["x"]
    dims = m2.dims_of(x, inp_gpu["B"], chunk_size)
    cs, dtt, st = m2.stage_buffers(dims, x.device)
    m2.mamba2_chunk_cumsum(dims, inp_gpu["dt"], inp_gpu["A"], cs, dtt)
    m2.mamba2_chunk_state(dims, x, inp_gpu["B"], cs, dtt, st)
    local = st.clone()
    fin = torch.empty((x.shape[0], x.shape[2], x.shape[3], inp_gpu["B"].shape[3]),
                      dtype=torch.float32, device=x.device)
    m2.mamba2_state_passing(dims, st, cs, inp_gpu["init_state"], fin)
    y = torch.empty_like(x)
    m2.mamba2_chunk_scan(dims, x, inp_gpu["B"], inp_gpu["C"], cs, dtt, st, inp_gpu["D"], y)
    torch.cuda.synchronize()
    return dims, cs, dtt, local, st, fin, y
