"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every comparison runs the GPU and the oracle on the same seeded inputs.
Tolerances: float32 workloads 1e-4 and bfloat16 workloads 2e-2, both as the
normwise relative error max|gpu - oracle| / max|oracle| per output tensor;
the cumulative sum 1e-6 per element relative to the float64 value (exact
where that value is 0).  Stage tests feed the GPU stage with oracle values of
its inputs where the stage is tested in isolation, so that a stage's error is
measured alone.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs
from gpu_helpers import (CUMSUM_TOL, TOL, assert_within, errors, f32, f64, normwise,
                         oracle_inputs, run_forward, run_stages, say, to_gpu)

pytestmark = pytest.mark.gpu

SMALL = ["tiny_fp32_L256_N16", "small_L1k_N64", "mid_L8k_N128"]


@pytest.fixture(scope="module")
def m2():
    import state_space_sequence_02_amd as lib
    return lib


def _custom(**kw):
    return ssd_inputs.custom(**kw)


# Ragged and multi-tile shapes beyond the five workloads: L not a multiple of Q,
# L shorter than one chunk, several groups, initial state, every chunk size,
# every supported headdim and a range of state sizes.
EDGE = [
    _custom(name="ragged_G2", batch=2, seqlen=1000, nheads=4, headdim=64, dstate=128, ngroups=2,
            chunk_size=256, init_state=True, seed=21),
    _custom(name="short_L100", batch=1, seqlen=100, nheads=2, headdim=64, dstate=64, ngroups=1,
            chunk_size=256, seed=22),
    _custom(name="q64_P32", batch=1, seqlen=700, nheads=3, headdim=32, dstate=192, ngroups=1,
            chunk_size=64, init_state=True, seed=23),
    _custom(name="q128_P128", batch=1, seqlen=600, nheads=2, headdim=128, dstate=64, ngroups=2,
            chunk_size=128, seed=24),
    _custom(name="N512_G4", batch=1, seqlen=520, nheads=8, headdim=64, dstate=512, ngroups=4,
            chunk_size=256, init_state=True, seed=25),
    _custom(name="f32_ragged", batch=2, seqlen=333, nheads=3, headdim=24, dstate=20, ngroups=3,
            chunk_size=32, dtype="f32", init_state=True, seed=26),
    # float32 chunks too large for the LDS-staged kernels (the plain fallbacks)
    _custom(name="f32_q256_fallback", batch=1, seqlen=600, nheads=2, headdim=32, dstate=64,
            ngroups=1, chunk_size=256, dtype="f32", init_state=True, seed=28),
    _custom(name="L1", batch=1, seqlen=1, nheads=2, headdim=64, dstate=64, ngroups=1,
            chunk_size=64, init_state=True, seed=27),
]


def _wl(name):
    return ssd_inputs.WORKLOADS[name]


def _all_small():
    return [_wl(n) for n in SMALL] + EDGE


@pytest.mark.parametrize("w", _all_small(), ids=lambda w: w.name)
def test_chunk_cumsum(m2, w):
    say(f"[cumsum] {w}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    dims, cs, dtt, *_ = run_stages(m2, g, w.chunk_size)
    ocs, odt = oracle.chunk_cumsum(f32(inp["dt"]), f32(inp["A"]), w.chunk_size)
    got = f64(cs)
    rel = np.abs(got - ocs) / np.where(ocs == 0, 1.0, np.abs(ocs))
    assert np.all(got[ocs == 0] == 0)
    assert rel.max() <= CUMSUM_TOL, rel.max()
    np.testing.assert_array_equal(f64(dtt), odt)


# Long sequences of many chunks for chunk_cumsum, with a ragged last chunk
# and a last head tile of 4 heads, through the scalar (H % 8 != 0, bfloat16)
# and the vector (float32) dt loads.
CUMSUM_WIDE = [
    _custom(name="cumsum_long_bf16_H36", batch=1, seqlen=1022 * 64 + 17, nheads=36, headdim=16,
            dstate=16, ngroups=1, chunk_size=64, seed=29),
    _custom(name="cumsum_long_f32_H12", batch=2, seqlen=300 * 32 + 5, nheads=12, headdim=16,
            dstate=16, ngroups=1, chunk_size=32, dtype="f32", seed=30),
]


@pytest.mark.parametrize("w", CUMSUM_WIDE, ids=lambda w: w.name)
def test_chunk_cumsum_long_ragged(m2, w):
    say(f"[cumsum wide] {w}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    cs, dtt, _ = m2.stage_buffers(dims, g["x"].device)
    m2.mamba2_chunk_cumsum(dims, g["dt"], g["A"], cs, dtt)
    torch.cuda.synchronize()
    ocs, odt = oracle.chunk_cumsum(f32(inp["dt"]), f32(inp["A"]), w.chunk_size)
    got = f64(cs)
    rel = np.abs(got - ocs) / np.where(ocs == 0, 1.0, np.abs(ocs))
    assert np.all(got[ocs == 0] == 0)
    assert rel.max() <= CUMSUM_TOL, rel.max()
    np.testing.assert_array_equal(f64(dtt), odt)


@pytest.mark.parametrize("w", _all_small(), ids=lambda w: w.name)
def test_stages_and_forward(m2, w):
    """Chained stages and the whole forward against the oracle's definitions:
    local chunk states, chunk-start states, final state and y."""
    say(f"[stages] {w}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    o = oracle_inputs(inp)
    dims, cs, dtt, local, st, fin, y = run_stages(m2, g, w.chunk_size)
    oy, ofin, ohs = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                          o["init_state"], chunk_size=w.chunk_size,
                                          want_hstart=True)
    oS = oracle.chunk_local_states(o["x"], o["dt"], o["A"], o["B"], chunk_size=w.chunk_size)
    tol = TOL[w.dtype]
    errs = errors({"local_states": (f64(local), oS), "start_states": (f64(st), ohs),
                   "final_state": (f64(fin), ofin), "y": (f64(y), oy)})
    say(f"  errors (tensor, worst head) {errs}")
    assert_within(errs, tol)
    # the fused entry point (its own kernels for some sizes) agrees with the
    # chained stages and with the oracle
    y2, fin2 = run_forward(m2, g, w.chunk_size)
    assert normwise(f64(y2), f64(y)) <= tol
    assert normwise(f64(fin2), f64(fin)) <= tol
    errs2 = errors({"y": (f64(y2), oy), "final_state": (f64(fin2), ofin)})
    say(f"  forward errors {errs2}")
    assert_within(errs2, tol)


@pytest.mark.parametrize("w", [_wl("small_L1k_N64"), _wl("tiny_fp32_L256_N16"), EDGE[0], EDGE[3]],
                         ids=lambda w: w.name)
def test_state_passing_isolated(m2, w):
    """state_passing fed with the oracle's local states and cumulative sums."""
    say(f"[state_passing] {w}")
    inp = ssd_inputs.make_inputs(w)
    o = oracle_inputs(inp)
    oS = oracle.chunk_local_states(o["x"], o["dt"], o["A"], o["B"], chunk_size=w.chunk_size)
    ocs, _ = oracle.chunk_cumsum(o["dt"], o["A"], w.chunk_size)
    cs32 = torch.from_numpy(ocs.astype(np.float32)).cuda()
    st = torch.from_numpy(oS.astype(np.float32)).cuda()
    h0 = None if inp["init_state"] is None else inp["init_state"].cuda()
    dims = m2.dims_of(inp["x"], inp["B"], w.chunk_size)
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
    m2.mamba2_state_passing(dims, st, cs32, h0, fin)
    torch.cuda.synchronize()
    decay = np.exp2(ocs.astype(np.float32).astype(np.float64)[..., -1])
    ohs, ofin = oracle.state_passing(oS.astype(np.float32), decay, o["init_state"])
    assert normwise(f64(st), ohs) <= 1e-5
    assert normwise(f64(fin), ofin) <= 1e-5


@pytest.mark.parametrize("w", [_wl("small_L1k_N64"), _wl("tiny_fp32_L256_N16"), EDGE[0], EDGE[2],
                               EDGE[3], EDGE[4]], ids=lambda w: w.name)
def test_chunk_scan_isolated(m2, w):
    """chunk_scan fed with the oracle's chunk-start states and cumulative sums."""
    say(f"[chunk_scan] {w}")
    inp = ssd_inputs.make_inputs(w)
    o = oracle_inputs(inp)
    g = to_gpu(inp)
    _, _, ohs = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                      o["init_state"], chunk_size=w.chunk_size, want_final=False,
                                      want_hstart=True)
    ocs, odt = oracle.chunk_cumsum(o["dt"], o["A"], w.chunk_size)
    dims = m2.dims_of(inp["x"], inp["B"], w.chunk_size)
    y = torch.empty_like(g["x"])
    m2.mamba2_chunk_scan(dims, g["x"], g["B"], g["C"],
                         torch.from_numpy(ocs.astype(np.float32)).cuda(),
                         torch.from_numpy(odt.astype(np.float32)).cuda(),
                         torch.from_numpy(ohs.astype(np.float32)).cuda(), g["D"], y)
    torch.cuda.synchronize()
    oy = oracle.chunk_outputs(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"], ohs,
                              chunk_size=w.chunk_size)
    errs = errors({"y": (f64(y), oy)})
    say(f"  y error (tensor, worst head) {errs['y']}")
    assert_within(errs, TOL[w.dtype])


def test_chunk_state_without_decay_is_BXt(m2):
    """A = 0: each chunk's local state is (dt X)^T B (the no-decay jump)."""
    w = _custom(name="a0", batch=1, seqlen=512, nheads=2, headdim=64, dstate=128, chunk_size=256,
                seed=31)
    inp = ssd_inputs.make_inputs(w)
    inp["A"] = torch.zeros_like(inp["A"])
    g = to_gpu(inp)
    _, _, _, local, *_ = run_stages(m2, g, w.chunk_size)
    x, dt, B = f64(inp["x"]), f64(inp["dt"]), f64(inp["B"])
    for c in range(2):
        sl = slice(256 * c, 256 * (c + 1))
        for h in range(2):
            ref = (x[0, sl, h] * dt[0, sl, h][:, None]).T @ B[0, sl, 0]
            assert normwise(f64(local[0, c, h]), ref) <= 2e-2


def test_zero_input_pure_decay(m2):
    """x = 0 with an initial state: y_t = 2^{cs_t} C_t . h0 across chunks and
    final = exp(A sum dt) h0."""
    w = _custom(name="x0", batch=1, seqlen=640, nheads=2, headdim=64, dstate=64, chunk_size=128,
                init_state=True, seed=32)
    inp = ssd_inputs.make_inputs(w)
    inp["x"] = torch.zeros_like(inp["x"])
    inp["A"] = 0.02 * inp["A"]  # keep exp(A sum dt) well inside float32 over 640 steps
    g = to_gpu(inp)
    y, fin = run_forward(m2, g, w.chunk_size)
    dt, A, C, h0 = f64(inp["dt"]), f64(inp["A"]), f64(inp["C"]), f64(inp["init_state"])
    for h in range(2):
        decay = np.exp(A[h] * np.cumsum(dt[0, :, h]))
        ref = decay[:, None] * (C[0, :, 0] @ h0[0, h].T)
        assert normwise(f64(y[0, :, h]), ref) <= 2e-2
        assert normwise(f64(fin[0, h]), decay[-1] * h0[0, h]) <= 1e-4


@pytest.mark.parametrize("Q", [64, 128, 256])
def test_chunk_size_invariance(m2, Q):
    w = _custom(name="qinv", batch=1, seqlen=1536, nheads=4, headdim=64, dstate=128, ngroups=2,
                chunk_size=Q, init_state=True, seed=33)
    inp = ssd_inputs.make_inputs(w)
    o = oracle_inputs(inp)
    y, fin = run_forward(m2, to_gpu(inp), Q)
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                        o["init_state"], chunk_size=Q)
    assert_within(errors({"y": (f64(y), oy), "final_state": (f64(fin), ofin)}), 2e-2)


def test_split_sequence_resume(m2):
    """Running [0, s) then [s, L) from the first part's final state matches one run.

    On a chunk boundary (s = 512) both runs perform the same chunks, so the
    final states agree to float32 accumulation order.  Off a boundary
    (s = 700) the second part is chunked differently, so its weighted inputs
    round to bfloat16 differently: both runs must meet the oracle at the
    bfloat16 tolerance and differ from each other by no more than about one
    bfloat16 rounding of the state's inputs (2^-8)."""
    w = _custom(name="split", batch=1, seqlen=1280, nheads=4, headdim=64, dstate=64, ngroups=1,
                chunk_size=256, init_state=True, seed=34)
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    o = oracle_inputs(inp)
    _, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                       o["init_state"], chunk_size=256)
    y, fin = run_forward(m2, g, 256)
    for s, tol in ((512, 1e-5), (700, 2.0 ** -8)):
        a = {k: (v[:, :s].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in g.items()}
        b = {k: (v[:, s:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in g.items()}
        ya, fa = run_forward(m2, a, 256)
        b["init_state"] = fa
        yb, fb = run_forward(m2, b, 256)
        assert normwise(f64(torch.cat([ya, yb], 1)), f64(y)) <= 1e-2
        assert normwise(f64(fb), f64(fin)) <= tol, s
        assert normwise(f64(fb), ofin) <= TOL["bf16"], s


def test_bitwise_deterministic(m2):
    w = _wl("mid_L8k_N128")
    g = to_gpu(ssd_inputs.make_inputs(w))
    y1, f1 = run_forward(m2, g, w.chunk_size)
    y2, f2 = run_forward(m2, g, w.chunk_size)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_outputs_stay_in_bounds(m2):
    """Guard bands around every output: nothing is written outside y, the final
    state, or (for the ragged tail) rows t >= L."""
    w = EDGE[0]
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    pad = 4096
    ybuf = torch.full((g["x"].numel() + 2 * pad,), 7.0, dtype=g["x"].dtype, device="cuda")
    y = ybuf[pad:pad + g["x"].numel()].view_as(g["x"])
    fn = w.batch * w.nheads * w.headdim * w.dstate
    fbuf = torch.full((fn + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    fin = fbuf[pad:pad + fn].view(w.batch, w.nheads, w.headdim, w.dstate)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    wbuf = torch.full((need + 2 * 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = wbuf[4096:4096 + need]
    m2.mamba2_ssd_forward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"],
                          y, fin, ws, need)
    torch.cuda.synchronize()
    assert torch.all(ybuf[:pad] == 7.0) and torch.all(ybuf[-pad:] == 7.0)
    assert torch.all(fbuf[:pad] == 7.0) and torch.all(fbuf[-pad:] == 7.0)
    assert torch.all(wbuf[:4096] == 0x5A) and torch.all(wbuf[-4096:] == 0x5A)
    y2, _ = run_forward(m2, g, w.chunk_size)
    assert torch.equal(y, y2)


def test_bad_workspace_is_rejected_without_launch(m2):
    w = EDGE[1]
    g = to_gpu(ssd_inputs.make_inputs(w))
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    y = torch.full_like(g["x"], 3.0)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(m2.Mamba2Error) as ei:
        m2.mamba2_ssd_forward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, y, None,
                              ws, need - 256)
    assert ei.value.status == m2.MAMBA2_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)


# The fused forward's grouped output stage serves several heads per workgroup;
# these shapes give several head slices per group, a short last slice, G > 1,
# every state size it supports (512 in two column-half passes), every chunk
# size, and a ragged last chunk.
GROUPED = [
    _custom(name="grp_N64_slices", batch=1, seqlen=16384 - 100, nheads=10, headdim=64, dstate=64,
            ngroups=2, chunk_size=256, init_state=True, seed=41),
    _custom(name="grp_N256_slices", batch=1, seqlen=8192, nheads=16, headdim=64, dstate=256,
            ngroups=1, chunk_size=256, seed=42),
    _custom(name="grp_N128_q64", batch=2, seqlen=4096 + 33, nheads=8, headdim=64, dstate=128,
            ngroups=4, chunk_size=64, init_state=True, seed=43),
    _custom(name="grp_N256_q128", batch=1, seqlen=6000, nheads=12, headdim=64, dstate=256,
            ngroups=3, chunk_size=128, seed=44),
    # state size 512: two passes over column halves, float32 y in between
    _custom(name="grp_N512_slices", batch=1, seqlen=8192 - 37, nheads=16, headdim=64,
            dstate=512, ngroups=2, chunk_size=256, init_state=True, seed=45),
    _custom(name="grp_N512_q64", batch=2, seqlen=2048 + 5, nheads=8, headdim=64, dstate=512,
            ngroups=4, chunk_size=64, seed=46),
    _custom(name="grp_N512_q128", batch=1, seqlen=3000, nheads=6, headdim=64, dstate=512,
            ngroups=1, chunk_size=128, init_state=True, seed=47),
]


@pytest.mark.parametrize("w", GROUPED, ids=lambda w: w.name)
def test_forward_grouped_heads(m2, w):
    say(f"[grouped] {w}")
    inp = ssd_inputs.make_inputs(w)
    o = oracle_inputs(inp)
    y, fin = run_forward(m2, to_gpu(inp), w.chunk_size)
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                        o["init_state"], chunk_size=w.chunk_size)
    errs = errors({"y": (f64(y), oy), "final_state": (f64(fin), ofin)})
    say(f"  errors (tensor, worst head) {errs}")
    assert_within(errs, TOL["bf16"])


def _zero_dt_tokens(L, Q):
    """Interior tokens whose dt is set to 0: the first and last step of a
    chunk, neighbours of chunk edges, a run of 40 steps across a chunk edge,
    and the last token."""
    ts = {0, 1, Q - 1, Q, Q + 5, 2 * Q - 1, L - 1}
    ts |= set(range(3 * Q - 20, 3 * Q + 20))
    return sorted(t for t in ts if t < L)


# Shapes whose forward takes each kind of kernel: per-head bfloat16 (headdim
# 32), the split form with the grouped output stage, the span path (heads
# sharing B, and state size 512 over column halves), span_scan, and float32.
DT_ZERO = [
    _custom(name="dt0_P32_split", batch=1, seqlen=1000, nheads=3, headdim=32, dstate=64,
            ngroups=1, chunk_size=64, init_state=True, seed=61),
    _custom(name="dt0_grouped_split", batch=2, seqlen=1100, nheads=4, headdim=64, dstate=128,
            ngroups=2, chunk_size=128, init_state=True, seed=62),
    _custom(name="dt0_span_N256", batch=1, seqlen=8155, nheads=64, headdim=64, dstate=256,
            ngroups=1, chunk_size=64, init_state=True, seed=63),
    _custom(name="dt0_span_N512", batch=4, seqlen=4096 - 19, nheads=32, headdim=64, dstate=512,
            ngroups=4, chunk_size=64, seed=64),
    # span_scan (the span replay fused with the output stage)
    _custom(name="dt0_span_scan_N128", batch=2, seqlen=8192 - 45, nheads=32, headdim=64,
            dstate=128, ngroups=2, chunk_size=64, init_state=True, seed=60),
    _custom(name="dt0_f32", batch=1, seqlen=700, nheads=2, headdim=16, dstate=16, ngroups=1,
            chunk_size=64, dtype="f32", init_state=True, seed=65),
]


@pytest.mark.parametrize("w", DT_ZERO, ids=lambda w: w.name)
def test_zero_dt_inside_sequence(m2, w):
    """dt = 0 at chosen interior tokens (decay 1, no input: the in-chunk
    weight exponent cs_j - log2(dt_j) is +inf there) and for all of one head's
    second chunk; y and the final state against the oracle, per head."""
    say(f"[dt=0] {w}")
    inp = ssd_inputs.make_inputs(w)
    Q = w.chunk_size
    ts = _zero_dt_tokens(w.seqlen, Q)
    inp["dt"][:, ts, :] = 0
    inp["dt"][:, Q:2 * Q, 0] = 0
    o = oracle_inputs(inp)
    g = to_gpu(inp)
    y, fin = run_forward(m2, g, Q)
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                        o["init_state"], chunk_size=Q)
    errs = errors({"y": (f64(y), oy), "final_state": (f64(fin), ofin)})
    say(f"  errors (tensor, worst head) {errs}")
    assert_within(errs, TOL[w.dtype])
    assert np.isfinite(f64(y)).all() and np.isfinite(f64(fin)).all()
    # the cumulative sum holds still across the zeroed steps
    cs, _ = oracle.chunk_cumsum(o["dt"], o["A"], Q)
    dims = m2.dims_of(g["x"], g["B"], Q)
    gcs, gdt, _ = m2.stage_buffers(dims, g["x"].device)
    m2.mamba2_chunk_cumsum(dims, g["dt"], g["A"], gcs, gdt)
    torch.cuda.synchronize()
    got = f64(gcs)
    rel = np.abs(got - cs) / np.where(cs == 0, 1.0, np.abs(cs))
    assert np.all(got[cs == 0] == 0) and rel.max() <= CUMSUM_TOL


MEMORYLESS = [
    _custom(name="memoryless_Q64_grouped", batch=1, seqlen=640, nheads=4, headdim=64, dstate=128,
            ngroups=2, chunk_size=64, init_state=True, seed=66),
    _custom(name="memoryless_Q256_span", batch=1, seqlen=8192, nheads=64, headdim=64, dstate=256,
            ngroups=1, chunk_size=256, init_state=True, seed=67),
    _custom(name="memoryless_span_scan_N64", batch=1, seqlen=4096 - 5, nheads=64, headdim=64,
            dstate=64, ngroups=2, chunk_size=128, init_state=True, seed=70),
    _custom(name="memoryless_Q64_f32", batch=1, seqlen=300, nheads=2, headdim=16, dstate=16,
            ngroups=1, chunk_size=64, dtype="f32", init_state=True, seed=68),
]


@pytest.mark.parametrize("w", MEMORYLESS, ids=lambda w: w.name)
def test_memoryless_limit(m2, w):
    """A dt = -200 at every step (dt held at 0.05): the state forgets
    everything but the current step, so y_t = dt_t (C_t . B_t) x_t + D x_t
    (the initial state has decayed by e^-200 after one step) and the final
    state is dt_L x_L (outer) B_L.  Checked against the oracle and against
    this closed form."""
    say(f"[memoryless] {w}")
    inp = ssd_inputs.make_inputs(w)
    inp["dt"] = torch.full_like(inp["dt"], 0.05)
    dtv = float(inp["dt"].flatten()[0])
    inp["A"] = torch.full_like(inp["A"], -200.0 / dtv)
    o = oracle_inputs(inp)
    g = to_gpu(inp)
    y, fin = run_forward(m2, g, w.chunk_size)
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                        o["init_state"], chunk_size=w.chunk_size)
    tol = TOL[w.dtype]
    errs = errors({"y": (f64(y), oy), "final_state": (f64(fin), ofin)})
    say(f"  errors (tensor, worst head) {errs}")
    assert_within(errs, tol)
    x, Bm, C, D = f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["D"])
    HG = w.nheads // w.ngroups
    for h in range(w.nheads):
        gg = h // HG
        cb = np.einsum("bln,bln->bl", C[:, :, gg], Bm[:, :, gg])
        ref = (dtv * cb)[..., None] * x[:, :, h] + D[h] * x[:, :, h]
        assert normwise(f64(y[:, :, h]), ref) <= tol, h
        fref = dtv * x[:, -1, h][:, :, None] * Bm[:, -1, gg][:, None, :]
        assert normwise(f64(fin[:, h]), fref) <= tol, h


def test_span_path_outputs_stay_in_bounds(m2):
    """Guard bands around y, the final state and the workspace on a shape that
    takes the span path (state size 512 over column halves, ragged tail,
    several groups and batches): nothing is written outside them."""
    from test_gpu_span_state import span_chunks
    w = _custom(name="guard_span_N512", batch=4, seqlen=4096 - 19, nheads=32, headdim=64,
                dstate=512, ngroups=4, chunk_size=64, init_state=True, seed=69)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert span_chunks(w, cus) > 0
    say(f"[guard span] {w}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    pad = 4096
    ybuf = torch.full((g["x"].numel() + 2 * pad,), 7.0, dtype=g["x"].dtype, device="cuda")
    y = ybuf[pad:pad + g["x"].numel()].view_as(g["x"])
    fn = w.batch * w.nheads * w.headdim * w.dstate
    fbuf = torch.full((fn + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    fin = fbuf[pad:pad + fn].view(w.batch, w.nheads, w.headdim, w.dstate)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    wbuf = torch.full((need + 2 * 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = wbuf[4096:4096 + need]
    m2.mamba2_ssd_forward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"],
                          y, fin, ws, need)
    torch.cuda.synchronize()
    assert torch.all(ybuf[:pad] == 7.0) and torch.all(ybuf[-pad:] == 7.0)
    assert torch.all(fbuf[:pad] == 7.0) and torch.all(fbuf[-pad:] == 7.0)
    assert torch.all(wbuf[:4096] == 0x5A) and torch.all(wbuf[-4096:] == 0x5A)
    y2, f2 = run_forward(m2, g, w.chunk_size)
    assert torch.equal(y, y2) and torch.equal(fin, f2)


# bfloat16 head and state sizes that are multiples of 16 but none of 32/64/128
# or of 64: the per-head kernels with a zero-padded last column block and odd
# p-tile counts.
ODD_SIZES = [
    _custom(name="bf16_P16_N16", batch=1, seqlen=700, nheads=3, headdim=16, dstate=16,
            ngroups=1, chunk_size=64, init_state=True, seed=71),
    _custom(name="bf16_P48_N48", batch=2, seqlen=600, nheads=4, headdim=48, dstate=48,
            ngroups=2, chunk_size=128, seed=72),
    _custom(name="bf16_P96_N80", batch=1, seqlen=1000, nheads=2, headdim=96, dstate=80,
            ngroups=1, chunk_size=256, init_state=True, seed=73),
    _custom(name="bf16_P80_N192", batch=1, seqlen=513, nheads=2, headdim=80, dstate=192,
            ngroups=2, chunk_size=64, seed=74),
    _custom(name="bf16_P112_N496", batch=1, seqlen=300, nheads=2, headdim=112, dstate=496,
            ngroups=1, chunk_size=128, init_state=True, seed=75),
    _custom(name="bf16_P64_N208", batch=1, seqlen=777, nheads=4, headdim=64, dstate=208,
            ngroups=1, chunk_size=256, seed=76),
]


@pytest.mark.parametrize("w", ODD_SIZES, ids=lambda w: w.name)
def test_bf16_sizes_multiple_of_16(m2, w):
    """Every stage and the whole forward at these sizes against the oracle
    (per tensor and per head), like the workloads above."""
    say(f"[odd sizes] {w}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    o = oracle_inputs(inp)
    dims, cs, dtt, local, st, fin, y = run_stages(m2, g, w.chunk_size)
    oy, ofin, ohs = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                          o["init_state"], chunk_size=w.chunk_size,
                                          want_hstart=True)
    oS = oracle.chunk_local_states(o["x"], o["dt"], o["A"], o["B"], chunk_size=w.chunk_size)
    errs = errors({"local_states": (f64(local), oS), "start_states": (f64(st), ohs),
                   "final_state": (f64(fin), ofin), "y": (f64(y), oy)})
    say(f"  stage errors (tensor, worst head) {errs}")
    assert_within(errs, TOL["bf16"])
    y2, fin2 = run_forward(m2, g, w.chunk_size)
    errs2 = errors({"y": (f64(y2), oy), "final_state": (f64(fin2), ofin)})
    say(f"  forward errors {errs2}")
    assert_within(errs2, TOL["bf16"])
