"""Pins of the backward oracle (oracle/backward.py, float64 vector-Jacobian
product of the recurrence) against facts that do not come from it:

 - central finite differences of the forward oracle (the C loop of oracle.scan)
   for every input, with rotation, incoming state and previous write, R = 1, 2;
 - adjoint identities: with zero incoming state Y and h_out are linear in X and
   in C, so <dY, Y> + <dH, h_out> = <dX, X> = <dC, C> exactly;
 - zero angles and no angles give the same gradients (the real-valued SSM);
 - the scalar LTI case (N = P = R = 1, constant coefficients, no rotation):
   y = L x with the explainer's causal matrix L_ts = gamma alpha^(t-s) +
   [s < t] beta alpha^(t-s-1), so dx = L^T dy, built here from the closed form;
 - an empty sequence passes dh_out to h0;
 - planted slips in a copy of the VJP each fail one of these pins.
"""
import inspect

import numpy as np
import pytest

import oracle
from oracle import backward
from oracle.backward import scan_vjp


def _problem(seed, R=2, theta=True, carry=True, L=6, H=2, P=3, N=4, b=1):
    rng = np.random.default_rng(seed)
    d = dict(x=rng.standard_normal((b, L, H, R, P)), B=rng.standard_normal((b, L, H, R, N)),
             C=rng.standard_normal((b, L, H, R, N)), dt=rng.uniform(0.1, 0.6, (b, L, H)),
             A=-rng.uniform(0.3, 2.0, (H,)), lam=rng.uniform(0.15, 0.85, (b, L, H)),
             theta=rng.uniform(-1.2, 1.2, (b, L, H, N // 2)) if theta else None,
             h0=rng.standard_normal((b, H, N, P)) if carry else None,
             B_prev=rng.standard_normal((b, H, R, N)) if carry else None,
             x_prev=rng.standard_normal((b, H, R, P)) if carry else None)
    cot = dict(dy=rng.standard_normal((b, L, H, R, P)), dh_out=rng.standard_normal((b, H, N, P)))
    return d, cot


def _loss(d, cot):
    y, ho = oracle.scan(**d)
    return float(np.sum(y * cot["dy"]) + np.sum(ho * cot["dh_out"]))


def _fd_check(vjp, d, cot, eps=1e-6, tol=1e-6):
    g = vjp(**d, **cot)
    for k, v in d.items():
        if v is None:
            assert g[k] is None
            continue
        for idx in np.ndindex(v.shape):
            hi = {kk: (None if vv is None else vv.copy()) for kk, vv in d.items()}
            lo = {kk: (None if vv is None else vv.copy()) for kk, vv in d.items()}
            hi[k][idx] += eps
            lo[k][idx] -= eps
            fd = (_loss(hi, cot) - _loss(lo, cot)) / (2 * eps)
            assert abs(fd - g[k][idx]) <= tol * (1.0 + abs(fd)), (k, idx, fd, g[k][idx])


@pytest.mark.parametrize("seed,R,theta,carry", [(0, 2, True, True), (1, 1, True, True), (2, 2, False, True),
                                                (3, 1, True, False)])
def test_finite_differences(seed, R, theta, carry):
    d, cot = _problem(seed, R=R, theta=theta, carry=carry)
    _fd_check(scan_vjp, d, cot)


@pytest.mark.parametrize("seed", [4, 5])
def test_adjoint_identities(seed):
    d, cot = _problem(seed, R=2, carry=False, L=9, P=5, N=6)
    y, ho = oracle.scan(**d)
    lhs = np.sum(y * cot["dy"]) + np.sum(ho * cot["dh_out"])
    g = scan_vjp(**d, **cot)
    assert np.isclose(np.sum(g["x"] * d["x"]), lhs, rtol=1e-12, atol=1e-12)
    assert np.isclose(np.sum(g["C"] * d["C"]), np.sum(y * cot["dy"]), rtol=1e-12, atol=1e-12)


def test_zero_angles_equal_no_rotation():
    d, cot = _problem(6, R=2)
    d0 = dict(d, theta=np.zeros_like(d["theta"]))
    dn = dict(d, theta=None)
    g0, gn = scan_vjp(**d0, **cot), scan_vjp(**dn, **cot)
    for k in ("x", "B", "C", "dt", "A", "lam", "h0", "B_prev", "x_prev"):
        np.testing.assert_allclose(g0[k], gn[k], rtol=0, atol=1e-13)


def test_scalar_lti_transpose():
    L, dtv, Av, lv = 12, 0.3, -1.1, 0.35
    alpha = np.exp(dtv * Av)
    beta, gamma = (1 - lv) * dtv * alpha, lv * dtv
    Lm = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            Lm[t, s] = gamma * alpha ** (t - s) + (beta * alpha ** (t - s - 1) if s < t else 0.0)
    rng = np.random.default_rng(7)
    xs, dys = rng.standard_normal(L), rng.standard_normal(L)
    one = np.ones((1, L, 1, 1, 1))
    g = scan_vjp(x=xs.reshape(1, L, 1, 1, 1), B=one, C=one, dt=np.full((1, L, 1), dtv), A=np.array([Av]),
                 lam=np.full((1, L, 1), lv), dy=dys.reshape(1, L, 1, 1, 1))
    np.testing.assert_allclose(g["x"].ravel(), Lm.T @ dys, rtol=1e-12, atol=1e-14)


def test_empty_sequence():
    d, cot = _problem(8, L=0)
    g = scan_vjp(**d, **cot)
    np.testing.assert_array_equal(g["h0"], cot["dh_out"])
    assert not g["B_prev"].any() and not g["x_prev"].any()


MUTANTS = [
    ("ga[t] * G + b_n * Qn", "ga[t] * G + 0.0 * Qn"),                  # delayed write's gradient dropped
    ("G[1::2] * K[0::2] - G[0::2] * K[1::2]", "G[0::2] * K[1::2] - G[1::2] * K[0::2]"),   # angle sign
    ("a_n * _rot(Gn, phi_n, -1)", "a_n * _rot(Gn, phi_n, +1)"),       # carried gradient turned the wrong way
    ("g[\"h0\"][bi, h] = a_n * Qn", "g[\"h0\"][bi, h] = Qn"),           # alpha_0 missing in dh0
    ("db * (1.0 - l_) * d_ * d_ * al", "db * (1.0 - l_) * d_ * al"),     # dA's beta term
    ("dg[t] = np.sum(G * Vt)", "dg[t] = np.sum(Q * Vt)"),              # gamma's gradient against Q
    ("Ht, Hp, Vt, Vp = Hs[t + 1], Hs[t], Vs[t + 1], Vs[t]", "Ht, Hp, Vt, Vp = Hs[t + 1], Hs[t + 1], Vs[t + 1], Vs[t]"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_slips_fail_a_pin(old, new):
    src = inspect.getsource(backward)
    assert src.count(old) == 1, old
    ns = {}
    exec(compile(src.replace(old, new), "mutant", "exec"), ns)
    mutant = ns["scan_vjp"]
    d, cot = _problem(9, R=2)
    with pytest.raises(AssertionError):
        _fd_check(mutant, d, cot)
