"""Parity of the one-token recurrent step (mamba2_decode_step) with the oracle.

The oracle's token-by-token recurrence is the definition: T decode steps from
a state are the recurrence over those T tokens from that state, so the
decode outputs y_t and the state after the last step are compared with the
oracle's y and final state (normwise, 2e-2 bfloat16 / 1e-4 float32, as for
the forward pass).  Also checked: the steps agree with the chunked forward
over the same tokens, nothing outside the outputs is written, D = NULL, and
sampled rows of a serving-sized batch."""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs
from gpu_helpers import TOL, f64, normwise, oracle_inputs, run_forward, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m2():
    import state_space_sequence_02_amd as lib
    return lib


SHAPES = [
    ssd_inputs.custom(name="dec_bf16_N64", batch=3, seqlen=6, nheads=8, headdim=64, dstate=64,
                      ngroups=1, chunk_size=64, init_state=True, seed=41),
    ssd_inputs.custom(name="dec_bf16_N256_G2", batch=2, seqlen=6, nheads=8, headdim=64,
                      dstate=256, ngroups=2, chunk_size=64, init_state=True, seed=42),
    ssd_inputs.custom(name="dec_bf16_P32_N192", batch=2, seqlen=6, nheads=4, headdim=32,
                      dstate=192, ngroups=1, chunk_size=64, init_state=True, seed=43),
    ssd_inputs.custom(name="dec_bf16_P128_N512_G4", batch=1, seqlen=6, nheads=8, headdim=128,
                      dstate=512, ngroups=4, chunk_size=64, init_state=True, seed=44),
    ssd_inputs.custom(name="dec_f32_odd", batch=2, seqlen=6, nheads=3, headdim=5, dstate=7,
                      ngroups=3, chunk_size=16, dtype="f32", init_state=True, seed=45),
    ssd_inputs.custom(name="dec_f32_N100", batch=1, seqlen=6, nheads=2, headdim=16, dstate=100,
                      ngroups=1, chunk_size=16, dtype="f32", init_state=True, seed=46),
    # state size 128: two rows per wavefront pass; a row count that leaves
    # the last wavefront partly idle
    ssd_inputs.custom(name="dec_bf16_N128_G2", batch=3, seqlen=6, nheads=6, headdim=48,
                      dstate=128, ngroups=2, chunk_size=64, init_state=True, seed=48),
    ssd_inputs.custom(name="dec_f32_N128", batch=2, seqlen=6, nheads=4, headdim=16, dstate=128,
                      ngroups=1, chunk_size=16, dtype="f32", init_state=True, seed=49),
]


def _decode_all(m2, g, w, D=True):
    """Runs one decode step per token of g; returns (y[B,L,H,P], final state)."""
    state = g["init_state"].clone()
    ys = []
    for t in range(w.seqlen):
        ys.append(m2.decode_step(g["x"][:, t].clone(), g["dt"][:, t].clone(), g["A"],
                                 g["B"][:, t].clone(), g["C"][:, t].clone(),
                                 g["D"] if D else None, state, chunk_size=w.chunk_size))
    torch.cuda.synchronize()
    return torch.stack(ys, 1), state


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_decode_steps_match_recurrence(m2, w):
    say(f"decode {w.name}")
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    o = oracle_inputs(inp)
    y, fin = _decode_all(m2, g, w)
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                        o["init_state"], chunk_size=w.chunk_size)
    tol = TOL[w.dtype]
    assert normwise(f64(y), oy) <= tol
    assert normwise(f64(fin), ofin) <= tol
    # the first step alone is the recurrence over one token
    o1 = {k: (v[:, :1] if k in ("x", "dt", "B", "C") else v) for k, v in o.items()}
    oy1, ofin1, _ = oracle.ssd_recurrence(o1["x"], o1["dt"], o1["A"], o1["B"], o1["C"], o1["D"],
                                          o1["init_state"], chunk_size=w.chunk_size)
    assert normwise(f64(y[:, :1]), oy1) <= tol


def test_decode_without_skip_term(m2):
    w = SHAPES[1]
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    o = oracle_inputs(inp)
    y, fin = _decode_all(m2, g, w, D=False)
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], None,
                                        o["init_state"], chunk_size=w.chunk_size)
    assert normwise(f64(y), oy) <= TOL["bf16"]
    assert normwise(f64(fin), ofin) <= TOL["bf16"]


@pytest.mark.parametrize("w", [SHAPES[0], SHAPES[4]], ids=lambda w: w.name)
def test_decode_agrees_with_forward(m2, w):
    """Token-by-token steps and the chunked forward over the same tokens are two
    evaluations of the same recurrence."""
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    y, fin = _decode_all(m2, g, w)
    yf, finf = run_forward(m2, g, w.chunk_size)
    tol = TOL[w.dtype]
    assert normwise(f64(y), f64(yf)) <= tol
    assert normwise(f64(fin), f64(finf)) <= tol


def test_decode_writes_only_its_outputs(m2):
    w = SHAPES[0]
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    Bn, H, P, N = g["init_state"].shape
    pad = 4096
    sbuf = torch.full((Bn * H * P * N + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    ybuf = torch.full((Bn * H * P + 2 * pad,), 3.0, dtype=torch.bfloat16, device="cuda")
    state = sbuf[pad:pad + Bn * H * P * N].view(Bn, H, P, N)
    state.copy_(g["init_state"])
    y = ybuf[pad:pad + Bn * H * P].view(Bn, H, P)
    dims = m2.make_dims(Bn, 1, H, P, N, w.ngroups, w.chunk_size, torch.bfloat16)
    m2.mamba2_decode_step(dims, g["x"][:, 0].clone(), g["dt"][:, 0].clone(), g["A"],
                          g["B"][:, 0].clone(), g["C"][:, 0].clone(), g["D"], state, y)
    torch.cuda.synchronize()
    assert torch.all(sbuf[:pad] == 7.0) and torch.all(sbuf[-pad:] == 7.0)
    assert torch.all(ybuf[:pad] == 3.0) and torch.all(ybuf[-pad:] == 3.0)
    assert torch.isfinite(state).all() and torch.isfinite(y.float()).all()


def test_decode_rejects_more_than_one_token(m2):
    w = SHAPES[0]
    dims = m2.make_dims(1, 2, w.nheads, w.headdim, w.dstate, 1, 64, torch.bfloat16)
    # raw device addresses: the library's own size check, not the binding's
    t = torch.zeros(1 << 16, dtype=torch.float32, device="cuda").data_ptr()
    with pytest.raises(m2.Mamba2Error) as e:
        m2.mamba2_decode_step(dims, t, t, t, t, t, None, t, t)
    assert e.value.status == m2.MAMBA2_ERR_SHAPE


SERVING = [
    # batch 64, H = 32, P = 64, N = 256: a 128 MiB state, four rows per wavefront
    ssd_inputs.custom(name="dec_serving", batch=64, seqlen=1, nheads=32, headdim=64,
                      dstate=256, ngroups=1, chunk_size=64, init_state=True, seed=47),
    # 2^20 state rows (batch 256, H = 64, P = 64, N = 64): the two-pass form
    ssd_inputs.custom(name="dec_serving_1M_rows", batch=256, seqlen=1, nheads=64, headdim=64,
                      dstate=64, ngroups=2, chunk_size=64, init_state=True, seed=50),
]


@pytest.mark.parametrize("w", SERVING, ids=lambda w: w.name)
def test_decode_serving_batch_sampled(m2, w):
    """One step at a serving batch size, checked against the oracle on sampled
    heads (of every group) of sampled batch rows."""
    inp = ssd_inputs.make_inputs(w)
    g = to_gpu(inp)
    y, fin = _decode_all(m2, g, w)
    heads = [0, w.nheads // 2 + 1, w.nheads - 1]
    for b in (0, w.batch // 2 - 3, w.batch - 1):
        o = oracle_inputs({k: (None if v is None else v[b:b + 1]) if k != "A" and k != "D" else v
                           for k, v in inp.items()})
        oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                            o["init_state"], chunk_size=64, heads=heads)
        assert normwise(f64(y[b:b + 1][:, :, heads]), oy) <= TOL["bf16"], b
        assert normwise(f64(fin[b:b + 1][:, heads]), ofin) <= TOL["bf16"], b
