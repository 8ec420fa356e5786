"""Parity of the one-kernel fwd_pass_state (mamba2_fwd_pass_state) and of the
forward that runs through it (mamba2_ssd_forward_fused) with the oracle.

mamba2_fwd_pass_state is fed the oracle's cumulative sums and dt, so its
outputs are measured alone: the weights w_j = 2^(cs[Q-1] - cs[j]) dt_j
(float32, per element against float64 within the rounding of the float32
exponent difference), the bfloat16
chunk-start states and the float32 final state (2e-2 normwise, the bfloat16
bar: the kernel rounds the weighted x to bfloat16 before the contraction).
The fused forward is compared with the oracle's y and final state at the same
bar.  Shapes cover every supported (chunk size, state size) pair, ragged last
chunks, a sequence shorter than one chunk, one token, one and several groups,
with and without the initial state, and enough chunks to cycle the kernel's
three LDS buffers many times; the long workload is checked on sampled heads."""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs
from gpu_helpers import (TOL, assert_within, errors, f32, f64, normwise, oracle_inputs,
                         run_forward, say, to_gpu)

pytestmark = pytest.mark.gpu

BT = TOL["bf16"]


@pytest.fixture(scope="module")
def m2():
    import state_space_sequence_02_amd as lib
    return lib


def _w(name, L, H, N, G, Q, Bn=1, init=True, seed=0):
    return ssd_inputs.custom(name=name, batch=Bn, seqlen=L, nheads=H, headdim=64, dstate=N,
                             ngroups=G, chunk_size=Q, init_state=init, seed=seed)


SHAPES = [
    _w("fps_Q64_N64_ragged_B2", 1000, 4, 64, 2, 64, Bn=2, seed=81),
    _w("fps_Q64_N256_many_chunks", 4096, 2, 256, 1, 64, seed=82),
    _w("fps_Q128_N128_G4", 700, 8, 128, 4, 128, init=False, seed=83),
    _w("fps_Q128_N64_short", 100, 3, 64, 1, 128, seed=84),
    _w("fps_Q256_N256_ragged", 1300, 4, 256, 2, 256, seed=85),
    _w("fps_Q256_N128_H9", 512, 9, 128, 3, 256, Bn=2, seed=86),
    _w("fps_Q256_N64_one_token", 1, 2, 64, 1, 256, seed=87),
    _w("fps_Q64_N128_two_chunks", 128, 16, 128, 1, 64, init=False, seed=88),
]


def _oracle_sums(o, Q):
    ocs, odt = oracle.chunk_cumsum(o["dt"], o["A"], Q)
    return ocs.astype(np.float32), odt.astype(np.float32)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_fwd_pass_state_isolated(m2, w):
    say(f"[fwd_pass_state] {w}")
    inp = ssd_inputs.make_inputs(w)
    o = oracle_inputs(inp)
    g = to_gpu(inp)
    ocs, odt = _oracle_sums(o, w.chunk_size)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    nc = ocs.shape[2]
    cs = torch.from_numpy(ocs).cuda()
    dtt = torch.from_numpy(odt).cuda()
    wT = torch.full_like(cs, float("nan"))
    hst = torch.empty((w.batch, nc, w.nheads, w.headdim, w.dstate), dtype=torch.bfloat16,
                      device="cuda")
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                      device="cuda")
    m2.mamba2_fwd_pass_state(dims, g["x"], g["B"], cs, dtt, g["init_state"], wT, hst, fin)
    torch.cuda.synchronize()
    # weights: the definition in float64 on the float32 inputs.  The kernel
    # forms d = cs[Q-1] - cs[j] in float32 (rounding error up to |d| 2^-24,
    # which exp2 turns into a relative error of ln 2 |d| 2^-24), then exp2 and
    # the product add a few ulps; the bound allows twice that.  Below the
    # float32 normal range (strong decay over a long chunk) exp2 flushes to
    # zero, so there only the absolute error is bounded.
    c64 = ocs.astype(np.float64)
    d = c64[..., -1:] - c64
    want = np.exp2(d) * odt.astype(np.float64)
    got = f64(wT)
    tiny = 2.0 ** -126
    normal = np.abs(want) >= tiny
    rel = np.abs(got - want) / np.where(normal, np.abs(want), 1.0)
    bound = 2.0 ** -21 + np.log(2.0) * np.abs(d) * 2.0 ** -23
    assert np.all(got[want == 0] == 0)
    assert np.all(rel[normal] <= bound[normal]), (rel[normal] / bound[normal]).max()
    assert np.abs(got - want)[~normal].max(initial=0.0) <= tiny
    # states: the token-by-token recurrence
    _, ofin, ohs = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                         o["init_state"], chunk_size=w.chunk_size,
                                         want_hstart=True)
    errs = errors({"start_states": (f64(hst), ohs), "final_state": (f64(fin), ofin)})
    say(f"  errors (tensor, worst head) {errs}")
    assert_within(errs, BT)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_forward_fused_matches_oracle(m2, w):
    say(f"[forward_fused] {w}")
    inp = ssd_inputs.make_inputs(w)
    o = oracle_inputs(inp)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(g["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                      device="cuda")
    m2.mamba2_ssd_forward_fused(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                                g["init_state"], y, fin, ws, need)
    torch.cuda.synchronize()
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                        o["init_state"], chunk_size=w.chunk_size)
    errs = errors({"y": (f64(y), oy), "final_state": (f64(fin), ofin)})
    say(f"  errors (tensor, worst head) {errs}")
    assert_within(errs, BT)
    # and with the default state path (chunk_state + state_passing)
    y2, fin2 = run_forward(m2, g, w.chunk_size)
    assert normwise(f64(y), f64(y2)) <= BT
    assert normwise(f64(fin), f64(fin2)) <= BT


def test_forward_fused_rejects_unsupported_sizes(m2):
    w = ssd_inputs.custom(name="fps_P32", batch=1, seqlen=300, nheads=2, headdim=32, dstate=64,
                          ngroups=1, chunk_size=64, seed=89)
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.full_like(g["x"], 3.0)
    fin = torch.empty((1, 2, 32, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(m2.Mamba2Error) as e:
        m2.mamba2_ssd_forward_fused(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None,
                                    y, fin, ws, need)
    assert e.value.status == m2.MAMBA2_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)


def test_forward_fused_full_size_sampled_heads(m2):
    """L = 65536, H = 32, P = 64, N = 256, G = 1, Q = 256: whole heads of the
    fused forward's y and final state against the oracle for three heads."""
    w = ssd_inputs.WORKLOADS["long_L64k_N256"]
    say(f"[forward_fused full] {w}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(g["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                      device="cuda")
    m2.mamba2_ssd_forward_fused(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                                g["init_state"], y, fin, ws, need)
    torch.cuda.synchronize()
    H, G = w.nheads, w.ngroups
    for h in sorted({0, H // 2 + 1, H - 1}):
        gi = h // (H // G)
        s = lambda t, dim, i: None if t is None else f32(t.narrow(dim, i, 1).contiguous())
        oy, ofin, _ = oracle.ssd_recurrence(
            s(inp["x"], 2, h), s(inp["dt"], 2, h), s(inp["A"], 0, h), s(inp["B"], 2, gi),
            s(inp["C"], 2, gi), s(inp["D"], 0, h), s(inp["init_state"], 1, h),
            chunk_size=w.chunk_size)
        ey = normwise(f64(y[:, :, h:h + 1]), oy)
        ef = normwise(f64(fin[:, h:h + 1]), ofin)
        say(f"  head {h}: y {ey:.3e} final {ef:.3e}")
        assert ey <= BT
        assert ef <= BT
