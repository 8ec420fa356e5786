"""Pins of the CPU oracle against facts other than itself.

Every check here compares the oracle with something it does not share code
or formula with: hand-worked examples (``tests/golden``), closed forms that
hold for special inputs, a textbook first-order IIR filter (scipy), an
explicit-product brute force, an independent chunked ("dual") evaluation, and
structural invariants.  Each is chosen so that a plausible slip in the oracle
(a dropped term, a wrong sign, a transposed operand, an exclusive instead of
an inclusive sum, a wrong head-to-group index) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.signal
import torch

import oracle
import ssd_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LOG2E = math.log2(math.e)


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            vals[k] = np.array([float(t) for t in v], dtype=np.float64)
    return vals


def _rand_case(seed, Bn=2, L=37, H=4, P=3, N=5, G=2, h0=True, D=True, a_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bn, L, H, P)).astype(np.float32)
    dt = rng.uniform(0.01, 0.6, (Bn, L, H)).astype(np.float32)
    A = (-a_scale * rng.uniform(0.5, 4.0, (H,))).astype(np.float32)
    B = rng.standard_normal((Bn, L, G, N)).astype(np.float32)
    C = rng.standard_normal((Bn, L, G, N)).astype(np.float32)
    Dv = rng.standard_normal((H,)).astype(np.float32) if D else None
    h = (0.5 * rng.standard_normal((Bn, H, P, N))).astype(np.float32) if h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=Dv, h0=h)


def _group(H, G):
    return np.arange(H) // (H // G)


# ----------------------------------------------------------------------------
# Independent formulations used as pins (numpy, float64)
# ----------------------------------------------------------------------------

def brute_force(x, dt, A, B, C, D, h0):
    """y_t = (prod_{r<=t} a_r) C_t.h0 + sum_{s<=t} (prod_{s<r<=t} a_r)(C_t.B_s) dt_s x_s + D x_t
    with explicit products of per-step decays (no recurrence, no log space)."""
    x, dt, A, B, C = (np.asarray(v, np.float64) for v in (x, dt, A, B, C))
    Bn, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    grp = _group(H, G)
    y = np.zeros((Bn, L, H, P))
    fin = np.zeros((Bn, H, P, N))
    for b in range(Bn):
        for h in range(H):
            g = grp[h]
            a = np.exp(dt[b, :, h] * A[h])
            for t in range(L):
                acc = np.zeros(P)
                if h0 is not None:
                    acc += np.prod(a[: t + 1]) * (np.asarray(h0[b, h], np.float64) @ C[b, t, g])
                for s in range(t + 1):
                    w = np.prod(a[s + 1: t + 1]) * (C[b, t, g] @ B[b, s, g]) * dt[b, s, h]
                    acc += w * x[b, s, h]
                if D is not None:
                    acc += float(D[h]) * x[b, t, h]
                y[b, t, h] = acc
            st = np.zeros((P, N))
            if h0 is not None:
                st += np.prod(a) * np.asarray(h0[b, h], np.float64)
            for s in range(L):
                st += np.prod(a[s + 1:]) * dt[b, s, h] * np.outer(x[b, s, h], B[b, s, g])
            fin[b, h] = st
    return y, fin


def chunked_dual(x, dt, A, B, C, D, h0, Q):
    """Independent chunked evaluation: natural-log cumulative sums per chunk,
    per-chunk local states (X scaled by the decay to the chunk end)^T B,
    the jump across chunks, and the masked quadratic form inside each chunk."""
    x, dt, A, B, C = (np.asarray(v, np.float64) for v in (x, dt, A, B, C))
    Bn, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    grp = _group(H, G)
    nc = -(-L // Q)
    y = np.zeros((Bn, L, H, P))
    fin = np.zeros((Bn, H, P, N))
    hstart = np.zeros((Bn, nc, H, P, N))
    local = np.zeros((Bn, nc, H, P, N))
    for b in range(Bn):
        for h in range(H):
            g = grp[h]
            run = np.zeros((P, N)) if h0 is None else np.asarray(h0[b, h], np.float64).copy()
            for c in range(nc):
                t0, t1 = c * Q, min(L, (c + 1) * Q)
                X = x[b, t0:t1, h]
                Bc, Cc, dtc = B[b, t0:t1, g], C[b, t0:t1, g], dt[b, t0:t1, h]
                cs = np.cumsum(A[h] * dtc)
                hstart[b, c, h] = run
                Sc = (X * (np.exp(cs[-1] - cs) * dtc)[:, None]).T @ Bc
                local[b, c, h] = Sc
                seg = np.exp(cs[:, None] - cs[None, :])
                M = np.tril(Cc @ Bc.T * seg) * dtc[None, :]
                yc = np.exp(cs)[:, None] * (Cc @ run.T) + M @ X
                if D is not None:
                    yc += float(D[h]) * X
                y[b, t0:t1, h] = yc
                run = np.exp(cs[-1]) * run + Sc
            fin[b, h] = run
    return y, fin, hstart, local


def _oracle(case, Q=8, **kw):
    return oracle.ssd_recurrence(case["x"], case["dt"], case["A"], case["B"], case["C"],
                                 case["D"], case["h0"], chunk_size=Q, **kw)


def _close(a, b, rtol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() <= rtol * scale


# ----------------------------------------------------------------------------
# Hand-worked goldens
# ----------------------------------------------------------------------------

def test_golden_scalar_two_step():
    g = _read_golden("scalar_two_step.txt")
    f = lambda v: np.asarray(v, np.float32)
    y, fin, _ = oracle.ssd_recurrence(
        f(g["x"]).reshape(1, 2, 1, 1), f(g["dt"]).reshape(1, 2, 1), f(g["A"]),
        f(g["B"]).reshape(1, 2, 1, 1), f(g["C"]).reshape(1, 2, 1, 1), f(g["D"]),
        f(g["h0"]).reshape(1, 1, 1, 1), chunk_size=2)
    np.testing.assert_allclose(y.ravel(), g["y"], rtol=1e-7)
    np.testing.assert_allclose(fin.ravel(), g["final"], rtol=1e-7)


def test_golden_orientation_P2_N2():
    g = _read_golden("orientation_P2_N2.txt")
    f = lambda v: np.asarray(v, np.float32)
    y, fin, _ = oracle.ssd_recurrence(
        f(g["x"]).reshape(1, 1, 1, 2), np.ones((1, 1, 1), np.float32), np.zeros(1, np.float32),
        f(g["B"]).reshape(1, 1, 1, 2), f(g["C"]).reshape(1, 1, 1, 2), np.zeros(1, np.float32),
        f(g["h0"]).reshape(1, 1, 2, 2), chunk_size=1)
    np.testing.assert_array_equal(y.ravel(), g["y"])
    np.testing.assert_array_equal(fin.ravel(), g["final"])


def test_golden_cumsum_ragged():
    g = _read_golden("cumsum_ragged.txt")
    Q = int(g["chunk_size"][0])
    cs, dtt = oracle.chunk_cumsum(np.asarray(g["dt"], np.float32).reshape(1, 3, 1),
                                  np.asarray(g["A"], np.float32), Q)
    np.testing.assert_allclose(cs.ravel(), g["dA_cs"], rtol=1e-15)
    np.testing.assert_array_equal(dtt.ravel(), g["dt_T"])


# ----------------------------------------------------------------------------
# Closed forms and textbook routines
# ----------------------------------------------------------------------------

def test_zero_decay_is_causal_linear_attention():
    """A = 0: y = tril(C B^T) (dt * X) + C h0^T + D X per (b, h): unnormalised
    causal linear attention, i.e. the no-decay jump h(t+T) = h(t) + B X^T."""
    case = _rand_case(1)
    case["A"] = np.zeros_like(case["A"])
    y, fin, _ = _oracle(case)
    x, dt, B, C = (case[k].astype(np.float64) for k in ("x", "dt", "B", "C"))
    Bn, L, H, P = x.shape
    grp = _group(H, B.shape[2])
    for b in range(Bn):
        for h in range(H):
            g = grp[h]
            X = x[b, :, h] * dt[b, :, h][:, None]
            h0 = case["h0"][b, h].astype(np.float64)
            ref = np.tril(C[b, :, g] @ B[b, :, g].T) @ X + C[b, :, g] @ h0.T + case["D"][h] * x[b, :, h]
            assert _close(y[b, :, h], ref)
            assert _close(fin[b, h], h0 + X.T @ B[b, :, g])


def test_zero_input_pure_decay():
    """x = 0 with an initial state: y_t = exp(A sum_{s<=t} dt_s) C_t . h0 and the
    final state is exp(A sum dt) h0."""
    case = _rand_case(2)
    case["x"] = np.zeros_like(case["x"])
    y, fin, _ = _oracle(case)
    dt, C = case["dt"].astype(np.float64), case["C"].astype(np.float64)
    Bn, L, H = dt.shape
    grp = _group(H, C.shape[2])
    for b in range(Bn):
        for h in range(H):
            h0 = case["h0"][b, h].astype(np.float64)
            decay = np.exp(float(case["A"][h]) * np.cumsum(dt[b, :, h]))
            ref = decay[:, None] * (C[b, :, grp[h]] @ h0.T)
            assert _close(y[b, :, h], ref, 1e-11)
            assert _close(fin[b, h], decay[-1] * h0, 1e-11)


def test_skip_term_is_D_times_x():
    case = _rand_case(3)
    y1, f1, _ = _oracle(case)
    case0 = dict(case, D=None)
    y0, f0, _ = _oracle(case0)
    np.testing.assert_allclose(y1 - y0, case["D"][None, None, :, None] * case["x"].astype(np.float64),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(f1, f0)


def test_first_order_iir_filter():
    """P = N = H = 1 with constant dt, b, c: the state is a first-order IIR
    filter of x, y = c * lfilter([dt b], [1, -e^{dt A}], x, zi=[e^{dt A} h0]) + D x."""
    L = 200
    rng = np.random.default_rng(4)
    x = rng.standard_normal(L).astype(np.float32)
    dtv, bv, cv, Av, Dv, h0v = 0.3, 1.7, -0.8, -0.9, 0.25, 2.0
    f32 = lambda v: np.float32(v)
    y, fin, _ = oracle.ssd_recurrence(
        x.reshape(1, L, 1, 1), np.full((1, L, 1), f32(dtv)), np.array([Av], np.float32),
        np.full((1, L, 1, 1), f32(bv)), np.full((1, L, 1, 1), f32(cv)), np.array([Dv], np.float32),
        np.full((1, 1, 1, 1), f32(h0v)), chunk_size=16)
    dt64, b64, c64, A64 = (float(f32(v)) for v in (dtv, bv, cv, Av))
    a = math.exp(dt64 * A64)
    s, _ = scipy.signal.lfilter([dt64 * b64], [1.0, -a], x.astype(np.float64), zi=[a * float(f32(h0v))])
    ref = c64 * s + float(f32(Dv)) * x.astype(np.float64)
    assert _close(y.ravel(), ref, 1e-12)
    assert _close(fin.ravel(), s[-1:], 1e-12)


def test_memoryless_limit():
    """A dt << 0: every step forgets the past, y_t = dt_t (C_t . B_t) x_t + D x_t."""
    case = _rand_case(5, a_scale=1e4)
    y, fin, _ = _oracle(case)
    x, dt, B, C = (case[k].astype(np.float64) for k in ("x", "dt", "B", "C"))
    grp = _group(x.shape[2], B.shape[2])
    Bg, Cg = B[:, :, grp], C[:, :, grp]
    ref = (dt * np.einsum("blhn,blhn->blh", Cg, Bg))[..., None] * x + case["D"][None, None, :, None] * x
    assert _close(y, ref, 1e-12)


# ----------------------------------------------------------------------------
# Brute force and the independent chunked evaluation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed,L", [(6, 1), (7, 9), (8, 23)])
def test_brute_force_quadratic(seed, L):
    case = _rand_case(seed, L=L)
    y, fin, _ = _oracle(case, Q=4)
    yb, fb = brute_force(case["x"], case["dt"], case["A"], case["B"], case["C"], case["D"], case["h0"])
    assert _close(y, yb, 1e-11)
    assert _close(fin, fb, 1e-11)


@pytest.mark.parametrize("Q", [1, 4, 7, 16, 64])
def test_chunked_dual_form(Q):
    case = _rand_case(9, L=45)
    y, fin, hs = _oracle(case, Q=Q, want_hstart=True)
    yd, fd, hd, ld = chunked_dual(case["x"], case["dt"], case["A"], case["B"], case["C"],
                                  case["D"], case["h0"], Q)
    assert _close(y, yd, 1e-11)
    assert _close(fin, fd, 1e-11)
    assert _close(hs, hd, 1e-11)
    S = oracle.chunk_local_states(case["x"], case["dt"], case["A"], case["B"], chunk_size=Q)
    assert _close(S, ld, 1e-11)


def test_local_states_without_decay_are_BXt():
    """A = 0: each chunk's local state is (dt X)^T B over the chunk, the jump
    formula's B X^T matrix product."""
    case = _rand_case(10, L=40)
    case["A"] = np.zeros_like(case["A"])
    Q = 16
    S = oracle.chunk_local_states(case["x"], case["dt"], case["A"], case["B"], chunk_size=Q)
    x, dt, B = (case[k].astype(np.float64) for k in ("x", "dt", "B"))
    grp = _group(x.shape[2], B.shape[2])
    for b in range(x.shape[0]):
        for c in range(S.shape[1]):
            sl = slice(c * Q, min(40, (c + 1) * Q))
            for h in range(x.shape[2]):
                ref = (x[b, sl, h] * dt[b, sl, h][:, None]).T @ B[b, sl, grp[h]]
                assert _close(S[b, c, h], ref)


# ----------------------------------------------------------------------------
# Stage functions reproduce the recurrence
# ----------------------------------------------------------------------------

def test_state_passing_and_chunk_outputs_reproduce_recurrence():
    case = _rand_case(11, L=50)
    Q = 8
    y, fin, hs = _oracle(case, Q=Q, want_hstart=True)
    S = oracle.chunk_local_states(case["x"], case["dt"], case["A"], case["B"], chunk_size=Q)
    nc = S.shape[1]
    dt = case["dt"].astype(np.float64)
    Bn, L, H = dt.shape
    decay = np.ones((Bn, H, nc))
    for c in range(nc):
        sl = slice(c * Q, min(L, (c + 1) * Q))
        decay[:, :, c] = np.prod(np.exp(dt[:, sl, :] * case["A"].astype(np.float64)), axis=1)
    hs2, fin2 = oracle.state_passing(S, decay, case["h0"])
    assert _close(hs2, hs, 1e-12)
    assert _close(fin2, fin, 1e-12)
    y2 = oracle.chunk_outputs(case["x"], case["dt"], case["A"], case["B"], case["C"], case["D"],
                              hs, chunk_size=Q)
    assert _close(y2, y, 1e-12)


def test_cumsum_matches_decay_products_and_is_monotone():
    case = _rand_case(12, L=50)
    Q = 16
    cs, dtt = oracle.chunk_cumsum(case["dt"], case["A"], Q)
    dt = case["dt"].astype(np.float64)
    Bn, L, H = dt.shape
    nc = cs.shape[2]
    for c in range(nc):
        sl = slice(c * Q, min(L, (c + 1) * Q))
        prod = np.prod(np.exp(dt[:, sl, :] * case["A"].astype(np.float64)), axis=1)  # [B,H]
        np.testing.assert_allclose(np.exp2(cs[:, :, c, -1]), prod, rtol=1e-13)
    assert np.all(np.diff(cs, axis=-1) <= 0)
    # ragged tail: padded steps add nothing and carry dt = 0
    tail = L - (nc - 1) * Q
    np.testing.assert_array_equal(cs[:, :, -1, tail:], np.repeat(cs[:, :, -1, tail - 1:tail], Q - tail, -1))
    np.testing.assert_array_equal(dtt[:, :, -1, tail:], 0.0)
    np.testing.assert_array_equal(dtt[:, :, 0, :], np.transpose(dt[:, :Q, :], (0, 2, 1)))


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------

def test_chunk_size_does_not_change_results():
    case = _rand_case(13, L=64)
    y1, f1, _ = _oracle(case, Q=4)
    y2, f2, _ = _oracle(case, Q=64)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(f1, f2)


@pytest.mark.parametrize("split", [16, 21])
def test_split_sequence_resume(split):
    case = _rand_case(14, L=48)
    y, fin, _ = _oracle(case, Q=8)
    first = {k: (v[:, :split] if k in ("x", "dt", "B", "C") else v) for k, v in case.items()}
    y1, f1, _ = _oracle(first, Q=8)
    second = {k: (v[:, split:] if k in ("x", "dt", "B", "C") else v) for k, v in case.items()}
    second["h0"] = f1.astype(np.float32)
    y2, f2, _ = _oracle(second, Q=8)
    # the resumed state is rounded to float32 at the split; compare to that precision
    assert _close(np.concatenate([y1, y2], axis=1), y, 1e-6)
    assert _close(f2, fin, 1e-6)


def test_linearity_in_x_and_h0():
    case = _rand_case(15)
    c2 = dict(case, D=None)
    ya, fa, _ = _oracle(c2)
    cb = dict(c2, x=(2.0 * c2["x"]).astype(np.float32), h0=(2.0 * c2["h0"]).astype(np.float32))
    yb, fb, _ = _oracle(cb)
    assert _close(yb, 2.0 * ya, 1e-13)
    assert _close(fb, 2.0 * fa, 1e-13)


def test_gauge_scaling_leaves_y_unchanged():
    case = _rand_case(16)
    y, fin, _ = _oracle(case)
    alpha = np.float32(4.0)  # power of two keeps the float32 inputs exact
    c2 = dict(case, B=case["B"] * alpha, C=case["C"] / alpha, h0=case["h0"] * alpha)
    y2, f2, _ = _oracle(c2)
    assert _close(y2, y, 1e-13)
    assert _close(f2, alpha * fin, 1e-13)


def test_group_expansion_matches_per_head_groups():
    case = _rand_case(17, H=6, G=3)
    y, fin, _ = _oracle(case)
    rep = case["x"].shape[2] // case["B"].shape[2]
    c2 = dict(case, B=np.repeat(case["B"], rep, axis=2), C=np.repeat(case["C"], rep, axis=2))
    y2, f2, _ = _oracle(c2)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(fin, f2)


def test_batch_independence_and_head_selection():
    case = _rand_case(18, Bn=3, H=4, G=2)
    y, fin, hs = _oracle(case, want_hstart=True)
    one = {k: (v[1:2] if (v is not None and k in ("x", "dt", "B", "C", "h0")) else v)
           for k, v in case.items()}
    y1, f1, _ = _oracle(one)
    np.testing.assert_array_equal(y1, y[1:2])
    np.testing.assert_array_equal(f1, fin[1:2])
    ys, fs, hss = _oracle(case, heads=[3, 0], want_hstart=True)
    np.testing.assert_array_equal(ys, y[:, :, [3, 0]])
    np.testing.assert_array_equal(fs, fin[:, [3, 0]])
    np.testing.assert_array_equal(hss, hs[:, :, [3, 0]])


def test_bad_arguments_are_rejected():
    case = _rand_case(19, H=3, G=2)  # H not a multiple of G
    with pytest.raises(ValueError):
        _oracle(case)


# ----------------------------------------------------------------------------
# Input generator
# ----------------------------------------------------------------------------

def test_input_generator_is_deterministic_and_in_domain():
    w = ssd_inputs.WORKLOADS["small_L1k_N64"]
    a = ssd_inputs.make_inputs(w)
    b = ssd_inputs.make_inputs(w)
    for k in a:
        if a[k] is None:
            assert b[k] is None
        else:
            assert torch.equal(a[k], b[k])
    assert a["x"].dtype == torch.bfloat16 and a["A"].dtype == torch.float32
    assert (a["A"] <= -1.0).all() and (a["A"] >= -16.0).all()
    assert (a["dt"].float() > 0).all() and (a["dt"].float() < 2.0).all()
    assert a["init_state"] is not None and a["init_state"].shape == (1, 8, 64, 64)
    t = ssd_inputs.make_inputs(ssd_inputs.WORKLOADS["tiny_fp32_L256_N16"])
    assert t["x"].dtype == torch.float32 and torch.equal(t["D"], torch.ones(2))
    assert t["init_state"] is None
