"""CPU oracle for the Mamba-3 SSM recurrence -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the benchmark's `cpu_baseline` leg
may import this package.  It shares no code with the HIP library.

`scan` wraps the float64 C library (`m3ref.c`: the plain sequential recurrence
in the physical frame).  `matrix_form` holds two independent NumPy derivations
(the decay x two-band matrix form with data-dependent RoPE, and the rotating-
frame loop) that pin the C loop.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("M3REF_LIB") or os.path.join(_HERE, "libm3ref.so")
_lib = None

ERRORS = {
    1: "bad dimensions",
    2: "non-finite input",
    3: "dt < 0",
    4: "A > 0",
    5: "lambda outside [0, 1]",
    6: "dstate must be even when angles are given",
    7: "missing required input",
    8: "out of memory",
}


class OracleError(ValueError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.m3ref_scan.restype = ctypes.c_int
    lib.m3ref_scan.argtypes = [ctypes.c_int] * 6 + [dp] * 6 + [dp] * 4 + [dp, dp, ctypes.c_int]
    lib.m3ref_validate.restype = ctypes.c_int
    lib.m3ref_validate.argtypes = [ctypes.c_int] * 6 + [dp] * 10
    lib.m3ref_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _as64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().m3ref_max_threads())


def scan(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None,
         nthreads: int = 0):
    """Runs the float64 recurrence.

    Shapes: x [b,L,H,R,P], B/C [b,L,H,R,N], dt/lam [b,L,H], A [H],
    theta [b,L,H,N/2] or None, h0 [b,H,N,P] or None, B_prev [b,H,R,N] and
    x_prev [b,H,R,P] or both None.  Returns (y [b,L,H,R,P], h_out [b,H,N,P]) as
    float64 arrays.  Raises OracleError on a violated precondition.
    """
    x, B, C, dt, A, lam = map(_as64, (x, B, C, dt, A, lam))
    theta, h0, B_prev, x_prev = map(_as64, (theta, h0, B_prev, x_prev))
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    if B.shape != (b, L, H, R, N) or C.shape != B.shape:
        raise OracleError("B/C shape mismatch")
    if dt.shape != (b, L, H) or lam.shape != (b, L, H) or A.shape != (H,):
        raise OracleError("dt/lam/A shape mismatch")
    if theta is not None and theta.shape != (b, L, H, N // 2):
        raise OracleError("theta shape mismatch")
    if h0 is not None and h0.shape != (b, H, N, P):
        raise OracleError("h0 shape mismatch")
    if (B_prev is None) != (x_prev is None):
        raise OracleError("B_prev and x_prev must be given together")
    if B_prev is not None and (B_prev.shape != (b, H, R, N) or x_prev.shape != (b, H, R, P)):
        raise OracleError("B_prev/x_prev shape mismatch")
    y = np.zeros((b, L, H, R, P), dtype=np.float64)
    h_out = np.zeros((b, H, N, P), dtype=np.float64)
    rc = _load().m3ref_scan(b, L, H, P, N, R, _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A),
                            _ptr(lam), _ptr(theta), _ptr(h0), _ptr(B_prev), _ptr(x_prev),
                            _ptr(y), _ptr(h_out), int(nthreads))
    if rc:
        raise OracleError(ERRORS.get(rc, f"error {rc}"))
    return y, h_out


def decode_steps(h0, x, B, C, dt, A, lam, theta=None, B_prev=None, x_prev=None,
                 nthreads: int = 0):
    """Successive single-token steps: x [S,b,H,R,P] etc. (step axis first).

    The same recurrence as `scan` with the steps as the time axis.  Returns
    (y [S,b,H,R,P], h_final [b,H,N,P]).
    """
    def tok_major(a):
        if a is None:
            return None
        a = _as64(a)
        return np.ascontiguousarray(np.moveaxis(a, 0, 1))  # [b,S,H,...]
    y, h = scan(tok_major(x), tok_major(B), tok_major(C), tok_major(dt), A, tok_major(lam),
                tok_major(theta), h0, B_prev, x_prev, nthreads=nthreads)
    return np.ascontiguousarray(np.moveaxis(y, 1, 0)), h


def round_bf16(a) -> np.ndarray:
    """Each value rounded to the nearest bfloat16 number, ties to even, returned
    as float64.  bfloat16 keeps 8 significant bits with float32's exponent
    range: a normal number's spacing is 2^(e-8) for a value in [2^(e-1), 2^e),
    and below the smallest normal, 2^-126, the spacing is 2^-133.  numpy's
    `round` rounds halves to even."""
    v = _as64(a)
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133).astype(np.float64)
    return np.round(np.ldexp(v, (-q).astype(np.int64))) * np.exp2(q)


def decode_steps_bf16_state(h0, x, B, C, dt, A, lam, theta=None, B_prev=None, x_prev=None,
                            nthreads: int = 0):
    """Successive single-token steps with the state held in bfloat16 between
    steps (the paper page's Table 6 benchmarks decode with an FP32 or a BF16
    state): each step is the float64 recurrence of `scan` (explainer panel 3's
    physical-frame loop, one token) from the stored state, y is read from the
    updated state before it is stored, and the stored state is the updated state
    rounded to bfloat16.  h0 is rounded the same way before the first step.
    Shapes as `decode_steps`; returns (y [S,b,H,R,P], h_final [b,H,N,P])."""
    x, B, C, dt, lam = map(_as64, (x, B, C, dt, lam))
    theta, B_prev, x_prev = map(_as64, (theta, B_prev, x_prev))
    S = x.shape[0]
    h = round_bf16(h0)
    ys = []
    for s in range(S):
        bp, xp = (B[s - 1], x[s - 1]) if s else (B_prev, x_prev)
        th = None if theta is None else theta[s][:, None]
        y, h_new = scan(x[s][:, None], B[s][:, None], C[s][:, None], dt[s][:, None], A, lam[s][:, None],
                        th, h, bp, xp, nthreads=nthreads)
        ys.append(y[:, 0])
        h = round_bf16(h_new)
    return np.stack(ys), h


def silu(v) -> np.ndarray:
    """v * sigmoid(v) = v / (1 + exp(-v)), in float64."""
    v = _as64(v)
    return v / (1.0 + np.exp(-v))


def gated_readout(y, z=None, w_y=None, w_z=None) -> np.ndarray:
    """Rank contraction of the outputs with an elementwise rank-expanded gate.

    The explainer's remark on MIMO training cost (its sec. 3.3 / 4.1.1 note)
    says the architecture replaces dense rank projections of x, y and the gate
    by learned elementwise rank expansion, printing no formula; the paper page's
    Tables 11 and 12 fuse the gate into the SSM kernel (prefill and decode).
    Reading used here: the gate z_t (one value per head column p) is expanded to
    Z_t[p, r] = w_z[h, r, p] z_t[p], applied to each rank's output through SiLU,
    and the ranks are contracted with w_y:
        out_t[p] = sum_r w_y[h, r, p] * Y_t[p, r] * silu(Z_t[p, r]).
    y [..., H, R, P]; z [..., H, P] or None (no gate); w_y, w_z [H, R, P] or
    None (all ones).  Returns out [..., H, P] in float64."""
    y = _as64(y)
    H, R, P = y.shape[-3:]
    wy = np.ones((H, R, P)) if w_y is None else _as64(w_y)
    g = np.ones(y.shape)
    if z is not None:
        wz = np.ones((H, R, P)) if w_z is None else _as64(w_z)
        g = silu(wz * _as64(z)[..., None, :])
    return (wy * y * g).sum(axis=-2)


def scan_gated(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None,
               z=None, w_y=None, w_z=None, nthreads: int = 0):
    """`scan` followed by `gated_readout` of its outputs: (out [b,L,H,P], h)."""
    y, h = scan(x, B, C, dt, A, lam, theta, h0, B_prev, x_prev, nthreads=nthreads)
    return gated_readout(y, z, w_y, w_z), h


def prologue(B, C, dt, theta_raw=None, B_prev=None, eps: float = 1e-6, bias_B=None, bias_C=None):
    """The inputs' pre-processing the explainer describes for Mamba-3 (its
    sec. 3.4 note: B and C get RMS normalization, then learned head-specific
    channel biases) and the per-step angle as dt times a raw angle (the
    complex transition generator of its Prop. 2 discretized over the step, as
    A becomes exp(dt A)).  Reading:
    each (token, head, rank) column of B and C (N values) is divided by
    sqrt(mean of its squares + eps), then bias [H, R, N] is added; B_prev (the
    token before the sequence, [b, H, R, N]) is treated as a B column; the
    angle of pair k at step t is dt_t * theta_raw[t, k].
    B, C [b, L, H, R, N]; dt [b, L, H]; theta_raw [b, L, H, N/2] or None.
    Returns (B_hat, C_hat, phi, B_prev_hat) in float64."""
    def norm(v, bias):
        v = _as64(v)
        out = v / np.sqrt((v * v).mean(axis=-1, keepdims=True) + eps)
        return out if bias is None else out + _as64(bias)
    Bh, Ch = norm(B, bias_B), norm(C, bias_C)
    phi = None if theta_raw is None else _as64(dt)[..., None] * _as64(theta_raw)
    Bp = None if B_prev is None else norm(B_prev, bias_B)
    return Bh, Ch, phi, Bp


def scan_prologue(x, B, C, dt, A, lam, theta_raw=None, h0=None, B_prev=None, x_prev=None,
                  eps: float = 1e-6, bias_B=None, bias_C=None, nthreads: int = 0):
    """`prologue` followed by `scan`: (y, h)."""
    Bh, Ch, phi, Bp = prologue(B, C, dt, theta_raw, B_prev, eps, bias_B, bias_C)
    return scan(x, Bh, Ch, dt, A, lam, phi, h0, Bp, x_prev, nthreads=nthreads)
