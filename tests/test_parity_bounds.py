"""CPU checks of the parity tests' own bounds (tests/_parity.py): the gated
readout's elementwise bound is never looser than y's bound carried through the
readout, and the per-dtype elementwise factors are the ones the tests state."""
import numpy as np
import pytest

import oracle
from _parity import ELEM_FACTOR, TOL, elem_factor, gate_scale, y_elem_bound


def test_factors():
    assert ELEM_FACTOR == {"bf16": 4.0, "fp32": 1.0}
    assert elem_factor(TOL["bf16"]) == 4.0 and elem_factor(TOL["fp32"]) == 1.0


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_gated_bound_not_looser_than_carried_y_bound(seed, dtype):
    """out[.., p] = sum_r g[r, p] y[.., r, p] with g = w_y silu(w_z z).  If every
    y element is within its bound e_r, out is within sum_r |g_r| e_r (triangle
    inequality); the bound the gated tests apply, F tol (|out| + gate_scale),
    must not exceed that -- elementwise, on shapes with cancelling ranks,
    tiny and huge gains, and tokens of very different sizes."""
    rng = np.random.default_rng(seed)
    b, L, H, R, P = 2, 9, 3, (1, 2, 4, 8)[seed % 4], 16
    y = rng.standard_normal((b, L, H, R, P)) * np.exp(rng.uniform(-4, 4, (b, L, 1, 1, 1)))
    if seed % 2:
        y[..., 1:, :] = -y[..., :1, :] * rng.uniform(0.9, 1.1, (b, L, H, R - 1, P)) if R > 1 else y[..., 1:, :]
    z = rng.standard_normal((b, L, H, P)) * 3
    w_y = rng.standard_normal((H, R, P)) * np.exp(rng.uniform(-3, 3, (H, R, P)))
    w_z = rng.uniform(0.1, 2.0, (H, R, P))
    tol = TOL[dtype]
    out = oracle.gated_readout(y, z, w_y, w_z)
    bound_out = elem_factor(tol) * tol * (np.abs(out) + gate_scale(y, z, w_y, w_z, block_axes=(1, 3, 4)))
    g = w_y * oracle.silu(w_z * z[..., None, :])
    carried = (np.abs(g) * y_elem_bound(y, tol, (1, 3, 4), (3, 4))).sum(axis=-2)
    assert np.all(bound_out <= carried * (1 + 1e-12) + 1e-300)
    # and without gate or weights (a plain rank sum)
    out1 = oracle.gated_readout(y, None, None, None)
    b1 = elem_factor(tol) * tol * (np.abs(out1) + gate_scale(y, block_axes=(1, 3, 4)))
    c1 = y_elem_bound(y, tol, (1, 3, 4), (3, 4)).sum(axis=-2)
    assert np.all(b1 <= c1 * (1 + 1e-12) + 1e-300)
