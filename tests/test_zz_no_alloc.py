"""mamba2_ssd_forward_noalloc (workspace in the library's static per-GPU
scratch, no allocation) against mamba2_ssd_forward with a caller workspace:
two calls in a row on one stream, the second with a smaller input, so the
second runs over what the first left in the scratch.  The same kernels run
in both, so the outputs must agree bit for bit; both are also held to the
oracle at the bfloat16 bar (2e-2 normwise, per tensor and per head)."""
import ctypes

import pytest
import torch

import oracle
import ssd_inputs
from gpu_helpers import TOL, assert_within, errors, f64, oracle_inputs, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m2():
    import state_space_sequence_02_amd as lib
    return lib


CALLS = [
    # span path (span states in the scratch; span_scan at this state size),
    # then the smaller split path
    ssd_inputs.custom(name="noalloc_span_L1000_N64", batch=1, seqlen=1000, nheads=64,
                      headdim=64, dstate=64, ngroups=2, chunk_size=64, init_state=True, seed=111),
    ssd_inputs.WORKLOADS["small_L1k_N64"],
]


def _outputs(w, g):
    y = torch.full_like(g["x"], 5.0)
    fin = torch.full((w.batch, w.nheads, w.headdim, w.dstate), 5.0, dtype=torch.float32,
                     device="cuda")
    return y, fin


def test_noalloc_matches_forward_on_two_calls(m2):
    from test_gpu_span_state import span_chunks
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert span_chunks(CALLS[0], cus) > 0 and span_chunks(CALLS[1], cus) == 0
    dev_stream = torch.cuda.current_stream()
    runs = []
    for w in CALLS:
        inp = ssd_inputs.make_inputs(w)
        g = to_gpu(inp)
        dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
        need = m2.mamba2_ssd_workspace_bytes(dims)
        say(f"[noalloc] {w} workspace {need} bytes of {m2.NOALLOC_SCRATCH_BYTES}")
        assert 0 < need <= m2.NOALLOC_SCRATCH_BYTES
        y, fin = _outputs(w, g)
        m2.mamba2_ssd_forward_noalloc(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                                      g["init_state"], y, fin, dev_stream)
        runs.append((w, inp, g, dims, need, y, fin))
    # the first call's sizes need more scratch than the second's
    assert runs[0][4] > runs[1][4]
    torch.cuda.synchronize()
    for w, inp, g, dims, need, y, fin in runs:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        y2, fin2 = _outputs(w, g)
        m2.mamba2_ssd_forward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                              g["init_state"], y2, fin2, ws, need, dev_stream)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), w.name
        assert torch.equal(fin, fin2), w.name
        o = oracle_inputs(inp)
        oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                            o["init_state"], chunk_size=w.chunk_size)
        errs = errors({"y": (f64(y), oy), "final_state": (f64(fin), ofin)})
        say(f"  {w.name}: identical to mamba2_ssd_forward; oracle errors {errs}")
        assert_within(errs, TOL["bf16"])


def test_noalloc_rejects_sizes_beyond_the_scratch(m2):
    """The long workload needs more workspace than the scratch holds: refused
    before any launch, outputs untouched."""
    w = ssd_inputs.WORKLOADS["long_L64k_N256"]
    dims = m2.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                        w.chunk_size, torch.bfloat16)
    assert m2.mamba2_ssd_workspace_bytes(dims) > m2.NOALLOC_SCRATCH_BYTES
    y = torch.full((1 << 12,), 3.0, dtype=torch.float32, device="cuda")
    p = y.data_ptr()
    rc = m2._lib.mamba2_ssd_forward_noalloc(ctypes.byref(dims), p, p, p, p, p, None, None, p,
                                            None, None)
    assert rc == m2.MAMBA2_ERR_WORKSPACE and "scratch" in m2.mamba2_last_error()
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
