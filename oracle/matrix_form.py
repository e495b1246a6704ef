"""Independent NumPy derivations that pin the C oracle -- TEST INFRASTRUCTURE ONLY.

Neither function calls the C loop; each one reaches the recurrence's result by
another route the Mamba-3 pages describe.

`dual_form`: the explicit causal operator.  The paper page's Figure 1 caption
and the explainer's section 3.1.2-3.1.3 (Eq. 7) describe the exponential-
trapezoidal recurrence as a decay operator times a lower two-band operator:
    D[t, k] = prod_{j=k+1..t} alpha_j            (k <= t)
    T[k, k] = gamma_k,  T[k, k-1] = beta_k       (lower bidiagonal)
    L = D @ T
The rotation enters in the data-dependent RoPE form (explainer Prop. 3, Prop. 4
and Eq. 11): with the absolute cumulative phase Phi_t = sum_{i<=t} phi_i,
B~_s = R(-Phi_s) B_s and C~_t = R(-Phi_t) C_t, and the delayed write keeps the
phase of the token that made it.  Then
    Y_t = sum_s L[t, s] X_s (B~_s^T C~_t)
plus the incoming state decayed to t.  The state itself is the transformed-frame
sum rotated back by Phi_t.

`rotating_frame`: the explainer's transformed-frame loop (panel 3, Prop. 3/4):
a scalar decay on an unrotated state, writes rotated by -Phi_t, readout with
C~_t.

Index convention: column s = -1 stands for the previous token's write carried
into the call (B_prev, x_prev), stored as column 0 of the (L+1)-column arrays.
"""
from __future__ import annotations

import numpy as np


def _rot(ang: np.ndarray) -> np.ndarray:
    """Block-diagonal rotation matrices: ang [..., K] -> [..., 2K, 2K]."""
    K = ang.shape[-1]
    out = np.zeros(ang.shape[:-1] + (2 * K, 2 * K))
    c, s = np.cos(ang), np.sin(ang)
    idx = np.arange(K)
    out[..., 2 * idx, 2 * idx] = c
    out[..., 2 * idx, 2 * idx + 1] = -s
    out[..., 2 * idx + 1, 2 * idx] = s
    out[..., 2 * idx + 1, 2 * idx + 1] = c
    return out


def causal_operator(dt: np.ndarray, a: float, lam: np.ndarray) -> np.ndarray:
    """L = D @ T with the extra leading column for the carried previous write.

    dt, lam: [L].  Returns [L, L+1]: column 0 is the carried write (s = -1),
    column s+1 is token s.  Also returns the decay of the incoming state,
    prod_{j<=t} alpha_j, as a second value.
    """
    Lq = dt.shape[0]
    alpha = np.exp(dt * a)
    beta = (1.0 - lam) * dt * alpha
    gamma = lam * dt
    D = np.zeros((Lq, Lq))
    for t in range(Lq):
        for k in range(t + 1):
            D[t, k] = np.prod(alpha[k + 1:t + 1])
    T = np.zeros((Lq, Lq + 1))          # rows k = 0..L-1, columns s = -1..L-1
    for k in range(Lq):
        T[k, k + 1] = gamma[k]          # diagonal: current write
        T[k, k] = beta[k]               # sub-diagonal: previous write
    init_decay = np.array([np.prod(alpha[:t + 1]) for t in range(Lq)])
    return D @ T, init_decay


def dual_form(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None):
    """Brute-force matrix form; same arguments and shapes as `oracle.scan`."""
    x, B, C, dt, A, lam = (np.asarray(v, dtype=np.float64) for v in (x, B, C, dt, A, lam))
    b, Lq, H, R, P = x.shape
    N = B.shape[-1]
    y = np.zeros((b, Lq, H, R, P))
    h_out = np.zeros((b, H, N, P))
    for bi in range(b):
        for h in range(H):
            Lmat, init_decay = causal_operator(dt[bi, :, h], float(A[h]), lam[bi, :, h])
            if theta is not None:
                Phi = np.cumsum(np.asarray(theta, dtype=np.float64)[bi, :, h, :], axis=0)  # [L, N/2]
                Rneg = _rot(-Phi)                                  # [L, N, N]
            else:
                Phi = np.zeros((Lq, N // 2))
                Rneg = np.broadcast_to(np.eye(N), (Lq, N, N))
            # transformed B and C; column 0 = carried write (phase 0, physical)
            Bt = np.einsum("tij,trj->tri", Rneg, B[bi, :, h])     # [L, R, N]
            Ct = np.einsum("tij,trj->tri", Rneg, C[bi, :, h])
            Ball = np.zeros((Lq + 1, R, N))
            Xall = np.zeros((Lq + 1, R, P))
            Ball[1:] = Bt
            Xall[1:] = x[bi, :, h]
            if B_prev is not None:
                Ball[0] = np.asarray(B_prev, dtype=np.float64)[bi, h]
                Xall[0] = np.asarray(x_prev, dtype=np.float64)[bi, h]
            H0 = np.zeros((N, P)) if h0 is None else np.asarray(h0, dtype=np.float64)[bi, h]
            # score[t, s, r, r'] = C~_t[:, r] . B~_s[:, r']
            score = np.einsum("trn,sqn->tsrq", Ct, Ball)
            # Y_t[r, p] = sum_s L[t, s] sum_r' score[t, s, r, r'] X_s[r', p]
            Ymat = np.einsum("ts,tsrq,sqp->trp", Lmat, score, Xall)
            Ymat += init_decay[:, None, None] * np.einsum("trn,np->trp", Ct, H0)
            y[bi, :, h] = Ymat
            # state at the last token, transformed frame then rotated back by Phi_{L-1}
            if Lq > 0:
                G = np.einsum("s,sqn,sqp->np", Lmat[-1], Ball, Xall) + init_decay[-1] * H0
                Rpos = _rot(Phi[-1]) if theta is not None else np.eye(N)
                h_out[bi, h] = Rpos @ G
            else:
                h_out[bi, h] = H0
    return y, h_out


def rotating_frame(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None):
    """Transformed-frame sequential loop; same arguments as `oracle.scan`."""
    x, B, C, dt, A, lam = (np.asarray(v, dtype=np.float64) for v in (x, B, C, dt, A, lam))
    b, Lq, H, R, P = x.shape
    N = B.shape[-1]
    y = np.zeros((b, Lq, H, R, P))
    h_out = np.zeros((b, H, N, P))
    for bi in range(b):
        for h in range(H):
            G = np.zeros((N, P)) if h0 is None else np.array(np.asarray(h0, dtype=np.float64)[bi, h])
            if B_prev is not None:
                Vprev = np.asarray(B_prev, dtype=np.float64)[bi, h].T @ np.asarray(x_prev, dtype=np.float64)[bi, h]
            else:
                Vprev = np.zeros((N, P))
            Phi = np.zeros(N // 2)
            for t in range(Lq):
                alpha = np.exp(dt[bi, t, h] * A[h])
                beta = (1.0 - lam[bi, t, h]) * dt[bi, t, h] * alpha
                gamma = lam[bi, t, h] * dt[bi, t, h]
                if theta is not None:
                    Phi = Phi + np.asarray(theta, dtype=np.float64)[bi, t, h]
                Rn = _rot(-Phi)
                Vcur = (Rn @ B[bi, t, h].T) @ x[bi, t, h]          # rotated current write
                G = alpha * G + beta * Vprev + gamma * Vcur       # scalar transition
                y[bi, t, h] = ((Rn @ C[bi, t, h].T).T @ G)         # C~_t^T G -> [R, P]
                Vprev = Vcur                                       # keeps its own phase
            h_out[bi, h] = _rot(Phi) @ G
    return y, h_out

