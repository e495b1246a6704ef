"""Shared helpers for GPU-vs-oracle parity tests.

Tolerances: relative 2e-2 for bf16 inputs/outputs and 1e-4 for fp32, as a
Frobenius norm per (batch, head) block (and per decode step), plus an
elementwise check |err| <= ELEM_FACTOR[dtype] * tol * (|ref| + scale).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"bf16": 2e-2, "fp32": 1e-4}
# The stated tolerance gates the relative Frobenius error of every (batch, head)
# block.  Single elements are additionally held to ELEM_FACTOR x the tolerance
# times (|ref| + scale), scale the block's or token's rms: a localized slip (a
# wrong token, a missing term) is off by ~100% of the output scale and fails
# either check.
#  - bf16: the path rounds four intermediates to bf16 for the MFMA (rotated B
#    and C, the masked score tile, the entering state), so an element's error
#    is a sum of many independent roundings: near-Gaussian, block rms about
#    3e-3 of the output rms (measured).  Over the ~10^7 elements of a full-size
#    case the largest of n such errors is about sqrt(2 ln n) ~ 5.7 times their
#    rms, i.e. ~0.017 x the scale, within 1x the tolerance; but where a token's
#    output nearly cancels, |ref| is tiny and the token rms carries the bound,
#    and measured tails there reached 1.7x.  4x leaves room for that tail and
#    stays 25x below a slip's size.
#  - fp32: fp32 MFMA operands and accumulation, errors ~1e-6 relative: held to
#    1x the tolerance.
ELEM_FACTOR = {"bf16": 4.0, "fp32": 1.0}


def note(msg: str):
    """Names the case about to run on the GPU (unbuffered, bypasses capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def to64(t) -> np.ndarray:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


def check_blocks(got: np.ndarray, ref: np.ndarray, tol: float, block_axes, what: str,
                 elem_axes=None, elem_scale=None):
    """Relative Frobenius error over each block (block_axes = axes reduced), then
    an elementwise bound ELEM_FACTOR * tol * (|ref| + scale).  The scale is the
    larger of the block's rms and, when elem_axes is given, the rms over
    elem_axes (one token's rank x column outputs for y): a token whose outputs
    are far larger than the block average (an incoming state that decays away)
    is judged at its own magnitude, and a token whose outputs nearly cancel
    (C_t . B_t ~ 0 after the state has decayed) at the block's.  elem_scale,
    when given, replaces that scale (same shape as ref): the gated readout
    passes gate_scale(), which carries y's own scale through the gains, so the
    bound on out is never looser than y's bound carried through the readout."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    err = got - ref
    num = np.sqrt((err ** 2).sum(axis=block_axes))
    den = np.sqrt((ref ** 2).sum(axis=block_axes))
    rel = num / np.maximum(den, 1e-30)
    small = den < 1e-20
    assert (num[small] < 1e-12).all(), f"{what}: nonzero output where reference is zero"
    worst = float(rel[~small].max()) if (~small).any() else 0.0
    assert worst <= tol, f"{what}: worst block relative error {worst:.3e} > {tol:g}"
    if elem_scale is not None:
        scale = np.asarray(elem_scale, dtype=np.float64)
    else:
        scale = np.sqrt((ref ** 2).mean(axis=tuple(block_axes), keepdims=True))
        if elem_axes is not None:
            scale = np.maximum(scale, np.sqrt((ref ** 2).mean(axis=tuple(elem_axes), keepdims=True)))
    bound = elem_factor(tol) * tol * (np.abs(ref) + scale) + 1e-30
    ratio = np.abs(err) / bound
    assert ratio.max() <= 1.0, f"{what}: elementwise error {ratio.max():.2f}x the bound"
    return worst


def elem_factor(tol: float) -> float:
    """ELEM_FACTOR of the dtype whose tolerance is `tol`."""
    return ELEM_FACTOR["bf16"] if tol >= TOL["bf16"] else ELEM_FACTOR["fp32"]


def y_elem_bound(y, tol, block_axes, elem_axes):
    """The elementwise bound check_blocks holds y [.., H, R, P] to (float64
    reference): ELEM_FACTOR * tol * (|y| + max(block rms, token rms))."""
    y = np.asarray(y, dtype=np.float64)
    scale = np.maximum(np.sqrt((y ** 2).mean(axis=tuple(block_axes), keepdims=True)),
                       np.sqrt((y ** 2).mean(axis=tuple(elem_axes), keepdims=True)))
    return elem_factor(tol) * tol * (np.abs(y) + scale)


def gate_scale(y, z=None, w_y=None, w_z=None, block_axes=None) -> np.ndarray:
    """Per-element scale of a gated readout out[.., h, p] = sum_r g[r, p] y[.., h, r, p]
    (g = w_y silu(w_z z)): sum_r |g[r, p]| times the scale y itself is judged
    at (the larger of the token's rms over its ranks and columns and, with
    block_axes, the block's rms), so out's bound is y's carried through the
    gains.  y [.., H, R, P] float64 (the reference outputs)."""
    import oracle
    y = np.asarray(y, dtype=np.float64)
    H, R, P = y.shape[-3:]
    wy = np.ones((H, R, P)) if w_y is None else np.asarray(w_y, dtype=np.float64)
    g = np.abs(wy) * np.ones(y.shape)
    if z is not None:
        wz = np.ones((H, R, P)) if w_z is None else np.asarray(w_z, dtype=np.float64)
        g = g * np.abs(oracle.silu(wz * np.asarray(z, dtype=np.float64)[..., None, :]))
    ys = np.sqrt((y ** 2).mean(axis=(-2, -1), keepdims=True))
    if block_axes is not None:
        ys = np.maximum(ys, np.sqrt((y ** 2).mean(axis=tuple(block_axes), keepdims=True)))
    return g.sum(axis=-2) * ys[..., 0, :]


def taken_chunk(w, chunk, variant="plain") -> int:
    """The chunk the library takes for workload `w` at the requested chunk and
    entry point ("plain", "gated", "prologue"), or 0 when it refuses the shape
    on the host (an unsupported size, or a kernel variant that would use
    scratch memory): the call then raises M3_ERR_SHAPE and launches nothing."""
    import state_space_sequence_02_amd as m3
    code = m3.M3_BF16 if w.dtype == "bf16" else m3.M3_FP32
    s = m3.make_shape(w.batch, max(w.seqlen, 1), w.nheads, w.headdim, w.dstate, w.rank, chunk, code)
    return m3.prefill_chunk_used(s, variant)


def dev_inputs(d: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def oracle_inputs(d: dict, heads=None) -> dict:
    """Float64 copies of a prefill input dict, optionally restricted to heads."""
    out = {}
    for k, v in d.items():
        if v is None:
            out[k] = None
            continue
        t = v.detach().to("cpu")
        if heads is not None:
            if k == "A":
                t = t[heads]
            elif k in ("h0", "B_prev", "x_prev"):
                t = t[:, heads]
            else:
                t = t[:, :, heads]
        out[k] = t.double().numpy().copy()
    return out
