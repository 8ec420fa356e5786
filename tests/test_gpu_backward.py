"""Parity of the backward pass (mamba2_ssd_backward) with the oracle.

The oracle's gradients (oracle.ssd_backward: back-propagation through the
token-by-token recurrence in float64, pinned by finite differences) are the
reference.  Every gradient is compared normwise (max |err| / max |ref|)
against 2e-2, the bfloat16 bar of the forward pass: the kernels compute in
float32 from bfloat16 operands and write dx, ddt, dB, dC in bfloat16.
Shapes cover every supported (chunk size, state size) pair, ragged last
chunks, a sequence shorter than one chunk, one and several groups, with and
without D, the initial state and the final-state gradient.  Full-size runs
check properties that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs
from gpu_helpers import TOL, f64, normwise, oracle_inputs, say, to_gpu

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
    _w("bwd_Q64_N64_G2_ragged", 200, 4, 64, 2, 64, Bn=2, seed=61),
    _w("bwd_Q64_N256_short", 17, 2, 256, 1, 64, seed=62),
    _w("bwd_Q128_N128_G1", 300, 4, 128, 1, 128, seed=63),
    _w("bwd_Q128_N64_G4", 256, 4, 64, 4, 128, Bn=2, seed=64),
    _w("bwd_Q256_N256_G2_ragged", 600, 4, 256, 2, 256, seed=65),
    _w("bwd_Q256_N64_H8_G1", 512, 8, 64, 1, 256, init=False, seed=66),
    _w("bwd_Q256_N128_H6_G3", 700, 6, 128, 3, 256, seed=67),
    _w("bwd_Q64_N128_G1_H8", 333, 8, 128, 1, 64, seed=68),
    _w("bwd_one_token", 1, 4, 128, 2, 128, Bn=2, seed=72),
    _w("bwd_Q128_N256_heads_eq_groups", 257, 3, 256, 3, 128, Bn=3, seed=73),
    # state size 512 (chunk 256): the state term of dU formed by its own
    # kernel, ragged last chunk, two batches, heads in two and four groups
    _w("bwd_Q256_N512_G2", 600, 4, 512, 2, 256, seed=85),
    _w("bwd_Q256_N512_G4_B2_ragged", 777, 8, 512, 4, 256, Bn=2, seed=92),
    _w("bwd_Q256_N512_short", 100, 2, 512, 1, 256, init=False, seed=93),
]

NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")


def _run(m2, w, *, with_D=True, with_dfinal=True):
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    if not with_D:
        inp["D"] = None
    g = to_gpu(inp)
    dy = cot["dy"].cuda()
    dfin = cot["dfinal"].cuda() if with_dfinal else None
    got = m2.ssd_backward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], dy,
                          dfin, chunk_size=w.chunk_size)
    torch.cuda.synchronize()
    o = oracle_inputs(inp)
    ref = oracle.ssd_backward(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"], o["init_state"],
                              cot["dy"].float().numpy(),
                              cot["dfinal"].numpy() if with_dfinal else None,
                              chunk_size=w.chunk_size)
    return got, ref


def _compare(got, ref, tol=BT):
    errs = {}
    for k in NAMES:
        r = ref[k if k != "dinit" else "dh0"]
        if r is None:
            assert k in ("dD", "dinit"), k
            continue
        errs[k] = normwise(f64(got[k]), r)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (bad, errs)
    return errs


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_backward_matches_oracle(m2, w):
    say(f"backward {w.name}")
    got, ref = _run(m2, w)
    errs = _compare(got, ref)
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_backward_without_D_or_final_gradient(m2):
    w = SHAPES[0]
    got, ref = _run(m2, w, with_D=False, with_dfinal=False)
    assert got["dD"] is None
    _compare(got, ref)


def test_backward_without_initial_state_still_gives_its_gradient(m2):
    # init_state = None means a zero start; its gradient is still defined
    w = _w("bwd_noinit", 300, 4, 128, 2, 128, init=False, seed=69)
    got, ref = _run(m2, w)
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    o = oracle_inputs(inp)
    zero = np.zeros((w.batch, w.nheads, w.headdim, w.dstate), np.float32)
    ref0 = oracle.ssd_backward(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"], zero,
                               cot["dy"].float().numpy(), cot["dfinal"].numpy(),
                               chunk_size=w.chunk_size)
    assert normwise(f64(got["dinit"]), ref0["dh0"]) <= BT
    _compare(got, ref)


def test_backward_multichunk_long(m2):
    """16 chunks of 256, 8 heads in one group, N = 256: the full-size head and
    state shape on a shorter sequence, so the gradient crosses many chunk
    boundaries in the reverse state pass."""
    w = _w("bwd_long_L4096", 4096, 8, 256, 1, 256, seed=70)
    say(f"backward {w.name}")
    got, ref = _run(m2, w)
    errs = _compare(got, ref)
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_backward_recompute_over_spans(m2):
    """A shape whose forward runs fwd_pass_state over spans of chunks (the
    span-end states, the jump across spans and the replay): the backward
    recomputes its chunk-start states the same way."""
    from test_gpu_span_state import span_chunks
    w = _w("bwd_span_L8192_N128", 8192, 32, 128, 2, 128, seed=74)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert span_chunks(w, cus, forward=False) > 0
    say(f"backward {w.name}")
    got, ref = _run(m2, w)
    errs = _compare(got, ref)
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("w", [SHAPES[4], SHAPES[-2]], ids=lambda w: w.name)
def test_backward_writes_only_its_outputs(m2, w):
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    pad = 4096
    bufs, views = {}, {}
    for k, like in (("dx", g["x"]), ("ddt", g["dt"]), ("dB", g["B"]), ("dC", g["C"])):
        n = like.numel()
        bufs[k] = torch.full((n + 2 * pad,), 5.0, dtype=like.dtype, device="cuda")
        views[k] = bufs[k][pad:pad + n].view(like.shape)
    need = m2.mamba2_ssd_backward_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dA = torch.empty(w.nheads, dtype=torch.float32, device="cuda")
    dD = torch.empty_like(dA)
    m2.mamba2_ssd_backward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                           g["init_state"], cot["dy"].cuda(), cot["dfinal"].cuda(), views["dx"],
                           views["ddt"], dA, views["dB"], views["dC"], dD, None, ws, need)
    torch.cuda.synchronize()
    for k, b in bufs.items():
        assert torch.all(b[:pad] == 5.0) and torch.all(b[-pad:] == 5.0), k
        assert torch.isfinite(views[k].float()).all(), k


def _wg(name, L, H, P, N, G, Q, Bn=1, init=True, seed=0, dtype="bf16"):
    return ssd_inputs.custom(name=name, batch=Bn, seqlen=L, nheads=H, headdim=P, dstate=N,
                             ngroups=G, chunk_size=Q, dtype=dtype, init_state=init, seed=seed)


# Sizes the MFMA backward does not cover run the generic backward (float32
# arithmetic on the vector ALU): float32 inputs, head sizes other than 64,
# state sizes other than 64/128/256/512 and state size 512 with chunks
# shorter than 256.  The shapes put 1 to 4
# output tiles of 64 along the chunk, the head size and the state size, with
# ragged tiles, ragged last chunks, a sequence shorter than one chunk and a
# single token.
GENERIC = [
    _wg("gbwd_f32_Q64_P16_N32_G2_ragged", 200, 4, 16, 32, 2, 64, Bn=2, dtype="f32", seed=81),
    _wg("gbwd_f32_Q16_P32_N16", 70, 2, 32, 16, 1, 16, dtype="f32", seed=82),
    _wg("gbwd_f32_Q256_P80_N100", 300, 2, 80, 100, 1, 256, dtype="f32", init=False, seed=83),
    _wg("gbwd_bf16_P32_N64", 300, 4, 32, 64, 2, 128, seed=84),
    _wg("gbwd_bf16_P64_N512_G2_Q128", 600, 4, 64, 512, 2, 128, seed=85),
    _wg("gbwd_bf16_P64_N512_Q64", 333, 4, 64, 512, 4, 64, Bn=2, seed=86),
    _wg("gbwd_bf16_P128_N96", 257, 2, 128, 96, 1, 128, seed=87),
    _wg("gbwd_bf16_P48_N208_short", 40, 3, 48, 208, 3, 64, seed=88),
    _wg("gbwd_bf16_one_token_N512", 1, 2, 64, 512, 1, 64, seed=89),
]
GTOL = {"bf16": BT, "f32": TOL["f32"]}


@pytest.mark.parametrize("w", GENERIC, ids=lambda w: w.name)
def test_generic_backward_matches_oracle(m2, w):
    say(f"backward (generic) {w.name}")
    got, ref = _run(m2, w)
    errs = _compare(got, ref, GTOL[w.dtype])
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_generic_backward_without_D_or_final_gradient(m2):
    for w in (GENERIC[0], GENERIC[4]):  # float32; bf16 at N = 512, chunk 128
        got, ref = _run(m2, w, with_D=False, with_dfinal=False)
        assert got["dD"] is None
        _compare(got, ref, GTOL[w.dtype])


@pytest.mark.parametrize("w", [GENERIC[2], GENERIC[5]], ids=lambda w: w.name)
def test_generic_backward_writes_only_its_outputs(m2, w):
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    pad = 4096
    bufs, views = {}, {}
    for k, like in (("dx", g["x"]), ("ddt", g["dt"]), ("dB", g["B"]), ("dC", g["C"])):
        n = like.numel()
        bufs[k] = torch.full((n + 2 * pad,), 5.0, dtype=like.dtype, device="cuda")
        views[k] = bufs[k][pad:pad + n].view(like.shape)
    hw = w.nheads * w.headdim * w.dstate * w.batch
    dinit_buf = torch.full((hw + 2 * pad,), 5.0, dtype=torch.float32, device="cuda")
    dinit = dinit_buf[pad:pad + hw].view(w.batch, w.nheads, w.headdim, w.dstate)
    need = m2.mamba2_ssd_backward_workspace_bytes(dims)
    ws_buf = torch.full((need + 2 * pad,), 7, dtype=torch.uint8, device="cuda")
    ws = ws_buf[pad:pad + need]
    dA = torch.empty(w.nheads, dtype=torch.float32, device="cuda")
    dD = torch.empty_like(dA)
    m2.mamba2_ssd_backward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                           g["init_state"], cot["dy"].cuda(), cot["dfinal"].cuda(), views["dx"],
                           views["ddt"], dA, views["dB"], views["dC"], dD, dinit, ws, need)
    torch.cuda.synchronize()
    for k, b in list(bufs.items()) + [("dinit", dinit_buf)]:
        assert torch.all(b[:pad] == 5.0) and torch.all(b[-pad:] == 5.0), k
    assert torch.all(ws_buf[:pad] == 7) and torch.all(ws_buf[-pad:] == 7)
    for k, v in list(views.items()) + [("dinit", dinit)]:
        assert torch.isfinite(v.float()).all(), k


def test_generic_backward_multichunk_N512(m2):
    """16 chunks of 128 at the largest state (N = 512), 8 heads in 2 groups:
    the generic backward across many chunk boundaries."""
    w = _wg("gbwd_long_L2048_N512_Q128", 2048, 8, 64, 512, 2, 128, seed=90)
    say(f"backward (generic) {w.name}")
    got, ref = _run(m2, w)
    errs = _compare(got, ref)
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_backward_multichunk_N512(m2):
    """16 chunks of 256 at the largest state (N = 512), 8 heads in 2 groups:
    the MFMA backward with the separate state-term kernel across many chunk
    boundaries (over spans of chunks in the recompute)."""
    w = _wg("bwd_long_L4096_N512", 4096, 8, 64, 512, 2, 256, seed=90)
    say(f"backward {w.name}")
    got, ref = _run(m2, w)
    errs = _compare(got, ref)
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_backward_N512_takes_the_mfma_path(m2):
    """At N = 512 with chunk 256 every stage of the profile entry runs (the
    generic path reports its whole time as stage 0 and 0 for the others)."""
    w = SHAPES[-3]
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    g = to_gpu(inp)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    need = m2.mamba2_ssd_backward_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = {k: torch.empty_like(g[s]) for k, s in (("dx", "x"), ("ddt", "dt"), ("dB", "B"),
                                                  ("dC", "C"))}
    dA = torch.empty(w.nheads, dtype=torch.float32, device="cuda")
    dD = torch.empty_like(dA)
    dinit = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=torch.float32, device="cuda")
    ms = m2.mamba2_ssd_backward_profile(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                                        g["init_state"], cot["dy"].cuda(), cot["dfinal"].cuda(),
                                        out["dx"], out["ddt"], dA, out["dB"], out["dC"], dD, dinit,
                                        ws, need)
    assert len(ms) == 8 and all(v > 0 for v in ms[1:7]), ms


def test_backward_fullsize_properties_N512(m2):
    """L = 262144, H = 32, P = 64, N = 512, G = 4, Q = 256 (the largest-state
    workload) through the MFMA backward: finite gradients, dD equal to
    sum(dy * x), and gradients homogeneous in the upstream gradient."""
    w = ssd_inputs.custom(name="bwd_full_N512", batch=1, seqlen=262144, nheads=32, headdim=64,
                          dstate=512, ngroups=4, chunk_size=256, init_state=False, seed=91)
    say(f"backward {w.name}")
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    g = to_gpu(inp)
    dy = cot["dy"].cuda()
    dfin = cot["dfinal"].cuda()
    a = m2.ssd_backward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, dy, dfin,
                        chunk_size=256)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.isfinite(a[k].float()).all(), k
    dD_ref = (dy.double() * g["x"].double()).sum(dim=(0, 1, 3))
    assert normwise(f64(a["dD"]), dD_ref.cpu().numpy()) <= 1e-4
    b2 = m2.ssd_backward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, 2 * dy, 2 * dfin,
                         chunk_size=256)
    torch.cuda.synchronize()
    for k in NAMES:
        diff = (b2[k].float() != 2 * a[k].float()).sum().item()
        assert diff <= 1e-6 * a[k].numel() + 1, (k, diff)


def test_backward_fullsize_properties(m2):
    """L = 65536, H = 32, P = 64, N = 256, G = 1, Q = 256 (the long-sequence
    workload): gradients are finite; dD equals sum(dy * x) over the batch and
    sequence; the gradients are linear in the upstream gradient (dy, dfinal)."""
    w = ssd_inputs.custom(name="bwd_full", batch=1, seqlen=65536, nheads=32, headdim=64,
                          dstate=256, ngroups=1, chunk_size=256, init_state=False, seed=71)
    say(f"backward {w.name}")
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    g = to_gpu(inp)
    dy = cot["dy"].cuda()
    dfin = cot["dfinal"].cuda()
    a = m2.ssd_backward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, dy, dfin,
                        chunk_size=256)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.isfinite(a[k].float()).all(), k
    dD_ref = (dy.double() * g["x"].double()).sum(dim=(0, 1, 3))
    assert normwise(f64(a["dD"]), dD_ref.cpu().numpy()) <= 1e-4
    # doubling the upstream gradient doubles every gradient: every step is
    # homogeneous in it and scaling by 2 is exact in binary floating point, so
    # only values at the edge of the float32 underflow range may differ
    b2 = m2.ssd_backward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, 2 * dy, 2 * dfin,
                         chunk_size=256)
    torch.cuda.synchronize()
    for k in NAMES:
        diff = (b2[k].float() != 2 * a[k].float()).sum().item()
        assert diff <= 1e-6 * a[k].numel() + 1, (k, diff)
        assert normwise(f64(b2[k]), 2 * f64(a[k])) <= 1e-2, k
