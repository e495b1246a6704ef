"""Float64 vector-Jacobian product of the Mamba-3 recurrence -- TEST
INFRASTRUCTURE ONLY (imported by tests/, the benchmark's cpu_baseline leg).

The forward map is the one `oracle.scan` computes, per (batch, head), t = 0..L-1
(Mamba-3 explainer, panels 1, 3, 4; paper page, Table 1 caption):

    alpha_t = exp(dt_t A), beta_t = (1 - lam_t) dt_t alpha_t, gamma_t = lam_t dt_t
    V_t = B_t X_t^T                                       (N x P)
    H_t = R(phi_t) [alpha_t H_{t-1} + beta_t V_{t-1}] + gamma_t V_t
    Y_t = H_t^T C_t                                       (P x R)

with H_{-1} = h0, V_{-1} = B_prev X_prev^T and R(phi) turning each row pair
(2k, 2k+1) by phi[k].  Given the cotangents dY (all t) and dH = d h_out, this
module returns the gradients of <dY, Y> + <dH, H_{L-1}> with respect to every
input, by the chain rule taken backwards through the same loop (plain loops
over time, NumPy over the N x P state):

    G_t  = C_t dY_t^T + alpha_{t+1} R(phi_{t+1})^T G_{t+1}    (G_{L-1} adds dH)
    Q_t  = R(phi_t)^T G_t                  (the gradient of the bracket above)
    dV_t = gamma_t G_t + beta_{t+1} Q_{t+1}
    dC_t = H_t dY_t,  dB_t = dV_t X_t,  dX_t = dV_t^T B_t
    d alpha_t = <Q_t, H_{t-1}>,  d beta_t = <Q_t, V_{t-1}>,  d gamma_t = <G_t, V_t>
    d phi_t[k] = sum_p (G_t[2k+1, p] K_t[2k, p] - G_t[2k, p] K_t[2k+1, p]),
                 K_t = H_t - gamma_t V_t = R(phi_t)[...]  (d/dphi R(phi) = R(phi) J)
    d h0 = alpha_0 Q_0,   dV_{-1} = beta_0 Q_0 -> d B_prev, d x_prev as for dV_t
    d dt_t  = d alpha A alpha + d beta (1 - lam) alpha (1 + dt A) + d gamma lam
    d lam_t = -d beta dt alpha + d gamma dt
    d A     = sum_t d alpha dt alpha + d beta (1 - lam) dt^2 alpha
    d theta_t = d phi_t   (theta holds the per-step angle itself)
"""
from __future__ import annotations

import numpy as np


def _rot(M, phi, sign):
    """R(sign * phi) applied to the row pairs of M [N, P] (phi [N/2]; None: no
    rotation)."""
    if phi is None:
        return M
    c = np.cos(phi)[:, None]
    s = sign * np.sin(phi)[:, None]
    out = np.empty_like(M)
    out[0::2] = c * M[0::2] - s * M[1::2]
    out[1::2] = s * M[0::2] + c * M[1::2]
    return out


def scan_vjp(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None, dy=None, dh_out=None):
    """Gradients of <dy, Y> + <dh_out, h_out> for the recurrence of oracle.scan.

    Shapes as oracle.scan (x [b,L,H,R,P], B/C [b,L,H,R,N], dt/lam [b,L,H], A [H],
    theta [b,L,H,N/2] or None, h0 [b,H,N,P] or None, B_prev [b,H,R,N] /
    x_prev [b,H,R,P] or None); dy [b,L,H,R,P] or None (zeros); dh_out
    [b,H,N,P] or None (zeros).  Returns a dict with the gradient of every
    input (None for the inputs that were None)."""
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    x, B, C, dt, A, lam = map(f, (x, B, C, dt, A, lam))
    theta, h0, B_prev, x_prev, dy, dh_out = map(f, (theta, h0, B_prev, x_prev, dy, dh_out))
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    if dy is None:
        dy = np.zeros_like(x)
    g = {k: np.zeros_like(v) for k, v in dict(x=x, B=B, C=C, dt=dt, A=A, lam=lam).items()}
    g["theta"] = None if theta is None else np.zeros_like(theta)
    g["h0"] = None if h0 is None else np.zeros_like(h0)
    g["B_prev"] = None if B_prev is None else np.zeros_like(B_prev)
    g["x_prev"] = None if x_prev is None else np.zeros_like(x_prev)
    for bi in range(b):
        for h in range(H):
            # ---- forward, keeping every state and write ----
            Hs = np.zeros((L + 1, N, P))           # Hs[t + 1] = H_t
            Vs = np.zeros((L + 1, N, P))           # Vs[t + 1] = V_t
            if h0 is not None:
                Hs[0] = h0[bi, h]
            if B_prev is not None:
                Vs[0] = B_prev[bi, h].T @ x_prev[bi, h]
            al = np.exp(dt[bi, :, h] * A[h])
            be = (1.0 - lam[bi, :, h]) * dt[bi, :, h] * al
            ga = lam[bi, :, h] * dt[bi, :, h]
            phis = [theta[bi, t, h] if theta is not None else None for t in range(L)]
            for t in range(L):
                Vs[t + 1] = B[bi, t, h].T @ x[bi, t, h]
                Hs[t + 1] = _rot(al[t] * Hs[t] + be[t] * Vs[t], phis[t], +1) + ga[t] * Vs[t + 1]
            # ---- backward ----
            Gn = np.zeros((N, P))
            Qn = np.zeros((N, P))
            a_n = b_n = 0.0
            phi_n = None
            da, db, dg = np.zeros(L), np.zeros(L), np.zeros(L)
            for t in range(L - 1, -1, -1):
                G = C[bi, t, h].T @ dy[bi, t, h] + a_n * _rot(Gn, phi_n, -1)
                if t == L - 1 and dh_out is not None:
                    G = G + dh_out[bi, h]
                Q = _rot(G, phis[t], -1)
                dV = ga[t] * G + b_n * Qn
                Ht, Hp, Vt, Vp = Hs[t + 1], Hs[t], Vs[t + 1], Vs[t]
                g["C"][bi, t, h] = (Ht @ dy[bi, t, h].T).T
                g["B"][bi, t, h] = (dV @ x[bi, t, h].T).T
                g["x"][bi, t, h] = B[bi, t, h] @ dV
                da[t] = np.sum(Q * Hp)
                db[t] = np.sum(Q * Vp)
                dg[t] = np.sum(G * Vt)
                if theta is not None:
                    K = Ht - ga[t] * Vt
                    g["theta"][bi, t, h] = np.sum(G[1::2] * K[0::2] - G[0::2] * K[1::2], axis=1)
                Gn, Qn, a_n, b_n, phi_n = G, Q, al[t], be[t], phis[t]
            if L == 0:
                Gn = np.zeros((N, P)) if dh_out is None else dh_out[bi, h]
                Qn, a_n, b_n = Gn, 1.0, 0.0
            if h0 is not None:
                g["h0"][bi, h] = a_n * Qn
            if B_prev is not None:
                dVp = b_n * Qn
                g["B_prev"][bi, h] = (dVp @ x_prev[bi, h].T).T
                g["x_prev"][bi, h] = B_prev[bi, h] @ dVp
            d_, l_ = dt[bi, :, h], lam[bi, :, h]
            g["dt"][bi, :, h] = da * A[h] * al + db * (1.0 - l_) * al * (1.0 + d_ * A[h]) + dg * l_
            g["lam"][bi, :, h] = -db * d_ * al + dg * d_
            g["A"][h] += np.sum(da * d_ * al + db * (1.0 - l_) * d_ * d_ * al)
    return g
