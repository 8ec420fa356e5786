"""Parity at the two long workloads (L = 65536, N = 256 and L = 262144,
N = 512, G = 4), in the launch configuration the benchmark times
(mamba2_ssd_forward).  The oracle recomputes whole heads (every token, every
headdim row) for a sample of heads that covers every B/C group (at G = 4: heads
0, 9, 17, 25, 31 of groups 0, 1, 2, 3, 3), plus the chunk-start states of those
heads through the stage entry points."""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs
from gpu_helpers import TOL, f32, f64, normwise, run_forward, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m2():
    import state_space_sequence_02_amd as lib
    return lib


def _head_slice(inp, h, G, H):
    g = h // (H // G)
    s = lambda t, dim, i: None if t is None else t.narrow(dim, i, 1).contiguous()
    return {
        "x": f32(s(inp["x"], 2, h)), "dt": f32(s(inp["dt"], 2, h)), "A": f32(s(inp["A"], 0, h)),
        "B": f32(s(inp["B"], 2, g)), "C": f32(s(inp["C"], 2, g)), "D": f32(s(inp["D"], 0, h)),
        "init_state": f32(s(inp["init_state"], 1, h)),
    }


@pytest.mark.parametrize("name", ["long_L64k_N256", "longest_L256k_N512"])
def test_full_size_forward_sampled_heads(m2, name):
    w = ssd_inputs.WORKLOADS[name]
    say(f"[fullsize] {w}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    y, fin = run_forward(m2, g, w.chunk_size)
    # stage path for chunk-start states at the same size
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    cs, dtt, st = m2.stage_buffers(dims, g["x"].device)
    m2.mamba2_chunk_cumsum(dims, g["dt"], g["A"], cs, dtt)
    m2.mamba2_chunk_state(dims, g["x"], g["B"], cs, dtt, st)
    m2.mamba2_state_passing(dims, st, cs, g["init_state"], None)
    torch.cuda.synchronize()
    H, G = w.nheads, w.ngroups
    HG = H // G
    heads = sorted({0, H // 2 + 1, H - 1} | {g * HG + 1 for g in range(1, G)})
    assert {h // HG for h in heads} == set(range(G))
    for h in heads:
        o = _head_slice(inp, h, G, H)
        oy, ofin, ohs = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                              o["init_state"], chunk_size=w.chunk_size,
                                              want_hstart=True)
        ey = normwise(f64(y[:, :, h:h + 1]), oy)
        ef = normwise(f64(fin[:, h:h + 1]), ofin)
        eh = normwise(f64(st[:, :, h:h + 1]), ohs)
        say(f"  head {h}: y {ey:.3e} final {ef:.3e} start_states {eh:.3e}")
        assert ey <= TOL["bf16"]
        assert ef <= TOL["bf16"]
        assert eh <= TOL["bf16"]
    del st, cs, dtt
