"""Pins of the oracle's gradients (oracle.ssd_backward) against facts other
than its own adjoint recursion.

The scalar differentiated is loss = sum(dy * y) + sum(dfinal * final_state).
  * Central finite differences of the forward oracle, one input element at a
    time, for every input.  The loss is affine in each single element of x,
    B, C, D and h0 (the recurrence is linear in each of them), so there a
    central difference is exact up to rounding.  In dt and A it is not (they
    enter through exp), so two step sizes are combined by Richardson
    extrapolation (error of order eps^4).  Inputs are multiples of 2^-10 and
    steps are powers of two, so every perturbed float32 input is exact.
  * The gradient is linear in (dy, dfinal).
  * One token from a zero state: the gradients have a closed form.
Shapes have two heads per group and two groups, so a wrong head-to-group
index or a missing sum over a group's heads fails the B and C checks.
"""
import numpy as np
import pytest

import oracle

Q = 1 << 10  # input quantum 2^-10


def _case(seed, Bn=2, L=5, H=4, P=2, N=3, G=2, D=True, h0=True):
    rng = np.random.default_rng(seed)
    q = lambda a: np.round(a * Q) / Q
    c = {
        "x": q(rng.standard_normal((Bn, L, H, P))),
        "dt": q(rng.uniform(0.05, 0.6, (Bn, L, H))),
        "A": q(-rng.uniform(0.3, 2.0, H)),
        "B": q(rng.standard_normal((Bn, L, G, N))),
        "C": q(rng.standard_normal((Bn, L, G, N))),
        "D": q(rng.standard_normal(H)) if D else None,
        "h0": q(rng.standard_normal((Bn, H, P, N))) if h0 else None,
    }
    dy = q(rng.standard_normal((Bn, L, H, P)))
    dfin = q(rng.standard_normal((Bn, H, P, N)))
    return {k: (None if v is None else v.astype(np.float32)) for k, v in c.items()}, dy, dfin


def _loss(c, dy, dfin):
    y, fin, _ = oracle.ssd_recurrence(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["h0"],
                                      chunk_size=4)
    s = float(np.sum(dy.astype(np.float64) * y))
    if dfin is not None:
        s += float(np.sum(dfin.astype(np.float64) * fin))
    return s


def _fd(c, dy, dfin, name, idx, eps):
    base = c[name][idx]
    vals = []
    for sgn in (1, -1):
        c[name][idx] = base + sgn * eps
        vals.append(_loss(c, dy, dfin))
    c[name][idx] = base
    return (vals[0] - vals[1]) / (2 * eps)


def _grads(c, dy, dfin):
    return oracle.ssd_backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["h0"], dy,
                               dfin, chunk_size=4)


AFFINE = {"x": "dx", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}
CURVED = {"dt": "ddt", "A": "dA"}


@pytest.mark.parametrize("seed,with_final", [(101, True), (102, False)])
def test_gradients_match_finite_differences(seed, with_final):
    c, dy, dfin = _case(seed)
    dfin = dfin if with_final else None
    g = _grads(c, dy, dfin)
    for name, gname in AFFINE.items():
        fd = np.zeros(c[name].shape)
        for idx in np.ndindex(*c[name].shape):
            fd[idx] = _fd(c, dy, dfin, name, idx, 2.0 ** -4)
        scale = max(1.0, np.abs(fd).max())
        assert np.abs(g[gname] - fd).max() <= 1e-9 * scale, name
    for name, gname in CURVED.items():
        fd = np.zeros(c[name].shape)
        for idx in np.ndindex(*c[name].shape):
            d1 = _fd(c, dy, dfin, name, idx, 2.0 ** -6)
            d2 = _fd(c, dy, dfin, name, idx, 2.0 ** -7)
            fd[idx] = (4 * d2 - d1) / 3
        scale = max(1.0, np.abs(fd).max())
        assert np.abs(g[gname] - fd).max() <= 2e-6 * scale, name


def test_gradients_without_skip_or_initial_state():
    c, dy, dfin = _case(103, L=4, H=2, G=1, D=False, h0=False)
    g = _grads(c, dy, dfin)
    assert g["dD"] is None and g["dh0"] is None
    for name, gname in (("x", "dx"), ("B", "dB"), ("C", "dC")):
        for idx in np.ndindex(*c[name].shape):
            assert abs(g[gname][idx] - _fd(c, dy, dfin, name, idx, 2.0 ** -4)) <= 1e-9, name
    for idx in np.ndindex(*c["dt"].shape):
        d1 = _fd(c, dy, dfin, "dt", idx, 2.0 ** -6)
        d2 = _fd(c, dy, dfin, "dt", idx, 2.0 ** -7)
        assert abs(g["ddt"][idx] - (4 * d2 - d1) / 3) <= 2e-6 * max(1.0, abs(d2))


def test_gradient_is_linear_in_upstream():
    c, dy, dfin = _case(104, L=9)
    rng = np.random.default_rng(5)
    dy2 = rng.standard_normal(dy.shape).astype(np.float32)
    df2 = rng.standard_normal(dfin.shape).astype(np.float32)
    g1, g2 = _grads(c, dy, dfin), _grads(c, dy2, df2)
    a, b = 0.75, -2.5
    g3 = _grads(c, (a * dy + b * dy2).astype(np.float32), (a * dfin + b * df2).astype(np.float32))
    for k in g1:
        ref = a * g1[k] + b * g2[k]
        assert np.allclose(g3[k], ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max()), k


def test_single_token_from_zero_state_closed_form():
    """L = 1, h0 = 0: y = dt x (B . C) + D x and final = dt x B^T, so every
    gradient is a one-line product."""
    c, dy, dfin = _case(105, Bn=1, L=1, H=2, P=3, N=4, G=1, h0=False)
    g = _grads(c, dy, dfin)
    x, dt, B, C, D = (c[k].astype(np.float64) for k in ("x", "dt", "B", "C", "D"))
    dy64, df64 = dy.astype(np.float64), dfin.astype(np.float64)
    for h in range(2):
        xv, dtv, Bv, Cv = x[0, 0, h], dt[0, 0, h], B[0, 0, 0], C[0, 0, 0]
        u = dy64[0, 0, h]                                   # [P]
        gs = u[:, None] * Cv[None, :] + df64[0, h]          # d loss / d final row, [P, N]
        np.testing.assert_allclose(g["dx"][0, 0, h], D[h] * u + dtv * gs @ Bv, rtol=1e-12)
        np.testing.assert_allclose(g["ddt"][0, 0, h], np.sum(xv * (gs @ Bv)), rtol=1e-12)
        # from a zero state the decay multiplies nothing: no gradient reaches A
        assert g["dA"][h] == 0.0
    gs_all = dy64[0, 0][:, :, None] * C[0, 0, 0][None, None, :] + df64[0]      # [H, P, N]
    wx = dt[0, 0][:, None] * x[0, 0]                                            # [H, P]
    np.testing.assert_allclose(g["dB"][0, 0, 0], np.einsum("hp,hpn->n", wx, gs_all), rtol=1e-12)
    np.testing.assert_allclose(g["dC"][0, 0, 0],
                               np.einsum("hp,hp,n->n", dy64[0, 0], wx, B[0, 0, 0]), rtol=1e-12)
