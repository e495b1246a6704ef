"""GPU parity of the fused prologue (BCNorm + head-specific B/C biases + angle
= dt x raw angle) against the float64 oracle's `prologue` followed by its
plain recurrence: every rank, both dtypes, several state and head sizes, with
and without biases, the previous write carried from step to step.
"""
import math

import pytest
import torch

import oracle
import state_space_sequence_02_amd as m3
from state_space_sequence_02_amd import inputs

from _parity import TOL, check_blocks, dev_inputs, note, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m3.load_library()


def _np(t):
    return None if t is None else t.double().numpy()


def _pro_inputs(w, seed, lead, biases):
    """Raw angles U(-pi, pi) per pair and [H, R, N] biases (or None)."""
    g = torch.Generator().manual_seed(seed)
    th = (torch.rand((*lead, w.nheads, w.dstate // 2), generator=g) * 2 - 1) * math.pi
    bb = torch.randn((w.nheads, w.rank, w.dstate), generator=g) * 0.5 if biases else None
    bc = torch.randn((w.nheads, w.rank, w.dstate), generator=g) * 0.5 if biases else None
    return th, bb, bc


@pytest.mark.parametrize("shape", [
    dict(batch=3, nheads=2, headdim=64, dstate=128, rank=4, dtype="bf16"),
    dict(batch=2, nheads=3, headdim=64, dstate=64, rank=1, dtype="bf16"),
    dict(batch=2, nheads=2, headdim=32, dstate=16, rank=2, dtype="fp32"),
    dict(batch=2, nheads=2, headdim=16, dstate=128, rank=8, dtype="bf16"),    # more items than 2 x threads
    dict(batch=1, nheads=2, headdim=128, dstate=256, rank=8, dtype="bf16"),
])
@pytest.mark.parametrize("biases", [True, False])
def test_decode_prologue(shape, biases):
    w = inputs.workload("decode", **shape)
    steps, seed, eps = 4, 600 + w.rank + w.dstate, 1e-5
    d = inputs.make_decode_inputs(w, seed=seed, steps=steps)
    th, bb, bc = _pro_inputs(w, seed + 1, (steps, w.batch), biases)
    dg = dev_inputs(d)
    h0 = torch.randn((w.batch, w.nheads, w.dstate, w.headdim), generator=torch.Generator().manual_seed(seed + 2)) * 0.5
    h = h0.cuda()
    thg = th.cuda()
    note(f"decode prologue {shape} biases={biases}")
    ys = []
    for s in range(steps):
        kw = dict(B_prev=dg["B"][s - 1], x_prev=dg["x"][s - 1]) if s else {}
        ys.append(m3.decode_step_prologue(h, dg["x"][s], dg["B"][s], dg["C"][s], dg["dt"][s], dg["A"], dg["lam"][s],
                                          thg[s], eps=eps, bias_B=None if bb is None else bb.cuda(),
                                          bias_C=None if bc is None else bc.cuda(), **kw))
    torch.cuda.synchronize()
    Bh, Ch, phi, _ = oracle.prologue(d["B"], d["C"], d["dt"], _np(th), eps=eps, bias_B=_np(bb), bias_C=_np(bc))
    yr, hr = oracle.decode_steps(h0, d["x"], Bh, Ch, d["dt"], d["A"], d["lam"], phi)
    tol = TOL[w.dtype]
    check_blocks(to64(torch.stack(ys)), yr, tol, (3, 4), "decode prologue y")
    check_blocks(to64(h), hr, tol, (2, 3), "decode prologue h")
