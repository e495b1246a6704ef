"""GPU parity of the gated readout (m3_scan_prefill_gated, m3_decode_step_gated)
against the float64 oracle's `scan_gated` / `gated_readout`, over every rank,
both dtypes, with and without the gate and its weights, one and several output
tiles per wave, and an incoming state and previous write.
"""
import numpy as np
import pytest
import torch

import oracle
import state_space_sequence_02_amd as m3
from state_space_sequence_02_amd import inputs

from _parity import TOL, check_blocks, dev_inputs, gate_scale, note, oracle_inputs, taken_chunk, to64

pytestmark = pytest.mark.gpu

KEYS = ("x", "B", "C", "dt", "A", "lam", "theta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m3.load_library()


def _gate_inputs(w, seed, lead, gate, weights):
    """z [*lead, H, P] in the input dtype (rounded like the inputs), w_y, w_z [H, R, P] fp32."""
    g = torch.Generator().manual_seed(seed)
    z = (torch.randn((*lead, w.nheads, w.headdim), generator=g) * 2).to(w.torch_dtype) if gate else None
    wy = torch.randn((w.nheads, w.rank, w.headdim), generator=g) if weights else None
    wz = (torch.rand((w.nheads, w.rank, w.headdim), generator=g) + 0.5) if (weights and gate) else None
    return z, wy, wz


def _np(t):
    return None if t is None else t.double().numpy()


CASES = [
    # (workload, overrides, chunk, gate, weights)
    ("siso", dict(batch=2, seqlen=300, nheads=3), 64, True, True),
    ("siso", dict(batch=1, seqlen=333, nheads=2), 256, True, True),          # two tiles per wave
    ("mimo", dict(batch=2, seqlen=130, nheads=2), 64, True, True),
    ("mimo", dict(batch=1, seqlen=150, nheads=2), 32, False, True),          # rank contraction only
    ("mimo", dict(batch=1, seqlen=97, nheads=2), 64, True, False),           # gate, unit weights
    ("mimo", dict(batch=1, seqlen=70, nheads=2, rank=2, dstate=64), 64, True, True),
    # N = 128: the streaming kernel with the gated output stage (R = 4, 2, 1)
    ("mimo", dict(batch=2, seqlen=300, nheads=3), 64, True, True),
    ("mimo", dict(batch=1, seqlen=300, nheads=2, rank=2), 64, True, True),
    ("mimo", dict(batch=1, seqlen=260, nheads=2, rank=1), 128, True, False),
    ("mimo", dict(batch=1, seqlen=90, nheads=2, rank=8, dstate=64), 16, True, True),
    ("mimo", dict(batch=1, seqlen=90, nheads=1, rank=8, headdim=128, dstate=64), 16, True, True),
    ("tiny", dict(batch=1, seqlen=100, nheads=2, rank=4, headdim=32, dstate=32), 32, True, True),   # fp32
    ("tiny", dict(batch=2, seqlen=77, nheads=1), 16, True, True),                                    # fp32 R=1
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-q{c[2]}-g{int(c[3])}w{int(c[4])}")
def test_prefill_gated(case):
    name, kw, chunk, gate, weights = case
    w = inputs.workload(name, **kw)
    seed = 300 + chunk + w.rank
    d = inputs.make_prefill_inputs(w, seed=seed)
    c = inputs.random_carry(w, seed=seed + 1)
    z, wy, wz = _gate_inputs(w, seed + 2, (w.batch, w.seqlen), gate, weights)
    dg, cg = dev_inputs(d), dev_inputs(c)
    assert taken_chunk(w, chunk, "gated") == chunk
    note(f"prefill gated {name} {kw} {w.dtype} chunk={chunk} gate={gate} weights={weights}")
    out, h = m3.scan_prefill_gated(**{k: dg[k] for k in KEYS}, **cg,
                                   z=None if z is None else z.cuda(), w_y=None if wy is None else wy.cuda(),
                                   w_z=None if wz is None else wz.cuda(), chunk=chunk)
    torch.cuda.synchronize()
    assert out.shape == (w.batch, w.seqlen, w.nheads, w.headdim)
    yref, href = oracle.scan(**oracle_inputs({**d, **c}))
    ref = oracle.gated_readout(yref, _np(z), _np(wy), _np(wz))
    tol = TOL[w.dtype]
    check_blocks(to64(out), ref, tol, (1, 3), "gated out", elem_axes=(3,),
                 elem_scale=gate_scale(yref, _np(z), _np(wy), _np(wz), block_axes=(1, 3, 4)))
    check_blocks(to64(h), href, tol, (2, 3), "h_out")
    # the state path is the ungated call's on the same kernel (the streaming
    # or the per-chunk one, whose products run in different orders), equal up
    # to rounding: with few sequences a chunk may compose its predecessors'
    # maps, an order of the products that depends on timing
    code = m3.M3_BF16 if w.dtype == "bf16" else m3.M3_FP32
    kern = m3.prefill_gated_kernel_used(m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank,
                                                      chunk, code))
    m3.debug_set_prefill_kernel(kern)
    try:
        _, h2 = m3.scan_prefill(**{k: dg[k] for k in KEYS}, **cg, chunk=chunk)
        torch.cuda.synchronize()
    finally:
        m3.debug_set_prefill_kernel(0)
    torch.testing.assert_close(h, h2, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("shape", [
    dict(batch=3, nheads=2, headdim=64, dstate=128, rank=4, dtype="bf16"),
    dict(batch=2, nheads=3, headdim=64, dstate=64, rank=1, dtype="bf16"),
    dict(batch=2, nheads=2, headdim=32, dstate=64, rank=2, dtype="fp32"),
    dict(batch=1, nheads=2, headdim=128, dstate=256, rank=8, dtype="bf16"),
])
@pytest.mark.parametrize("gate", [True, False])
def test_decode_gated(shape, gate):
    w = inputs.workload("decode", **shape)
    steps, seed = 4, 400 + w.rank + w.dstate
    d = inputs.make_decode_inputs(w, seed=seed, steps=steps)
    dg = dev_inputs(d)
    z, wy, wz = _gate_inputs(w, seed + 1, (steps, w.batch), gate, True)
    h0 = torch.randn((w.batch, w.nheads, w.dstate, w.headdim), generator=torch.Generator().manual_seed(seed + 2)) * 0.5
    h = h0.cuda()
    note(f"decode gated {shape} gate={gate}")
    outs = []
    for s in range(steps):
        kw = dict(B_prev=dg["B"][s - 1], x_prev=dg["x"][s - 1]) if s else {}
        outs.append(m3.decode_step_gated(h, dg["x"][s], dg["B"][s], dg["C"][s], dg["dt"][s], dg["A"], dg["lam"][s],
                                         dg["theta"][s], z=None if z is None else z[s].cuda(), w_y=wy.cuda(),
                                         w_z=None if wz is None else wz.cuda(), **kw))
    torch.cuda.synchronize()
    yr, hr = oracle.decode_steps(h0, d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"])
    ref = oracle.gated_readout(yr, _np(z), _np(wy), _np(wz))
    tol = TOL[w.dtype]
    check_blocks(to64(torch.stack(outs)), ref, tol, (3,), "decode gated out",
                 elem_scale=gate_scale(yr, _np(z), _np(wy), _np(wz)))
    check_blocks(to64(h), hr, tol, (2, 3), "decode h")


def test_gated_prefill_then_decode_continues():
    """prefill_gated over L - 2 tokens, then two gated decode steps, equals the
    gated readout of the whole sequence."""
    w = inputs.workload("mimo", batch=2, seqlen=70, nheads=2)
    d = inputs.make_prefill_inputs(w, seed=501)
    z, wy, wz = _gate_inputs(w, 502, (w.batch, w.seqlen), True, True)
    dg = dev_inputs(d)
    L0 = w.seqlen - 2
    note("gated prefill then gated decode")
    out0, h = m3.scan_prefill_gated(*(dg[k][:, :L0].contiguous() if dg[k].dim() > 1 else dg[k] for k in KEYS),
                                    z=z[:, :L0].contiguous().cuda(), w_y=wy.cuda(), w_z=wz.cuda(), chunk=32)
    outs = [out0]
    for t in (L0, L0 + 1):
        o = m3.decode_step_gated(h, dg["x"][:, t].contiguous(), dg["B"][:, t].contiguous(), dg["C"][:, t].contiguous(),
                                 dg["dt"][:, t].contiguous(), dg["A"], dg["lam"][:, t].contiguous(),
                                 dg["theta"][:, t].contiguous(), B_prev=dg["B"][:, t - 1].contiguous(),
                                 x_prev=dg["x"][:, t - 1].contiguous(), z=z[:, t].contiguous().cuda(),
                                 w_y=wy.cuda(), w_z=wz.cuda())
        outs.append(o[:, None])
    torch.cuda.synchronize()
    yref, _ = oracle.scan(**oracle_inputs(d))
    ref = oracle.gated_readout(yref, _np(z), _np(wy), _np(wz))
    check_blocks(to64(torch.cat(outs, dim=1)), ref, TOL[w.dtype], (1, 3), "gated out", elem_axes=(3,),
                 elem_scale=gate_scale(yref, _np(z), _np(wy), _np(wz), block_axes=(1, 3, 4)))
    assert np.isfinite(to64(h)).all()


@pytest.mark.parametrize("name,kw", [("mimo", {}), ("long", dict(seqlen=8192, nheads=2))],
                         ids=["mimo-full-size", "long-8192-chain"])
def test_prefill_gated_stream(name, kw):
    """The gated readout in the streaming kernel's output stage: the MIMO
    workload at full size (4 x 4,096 tokens x 32 heads, states only), two heads
    compared with the oracle; and 8,192 tokens of two heads at the long shape
    (maps in use), every head compared."""
    w = inputs.workload(name, **kw)
    shape = m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 64, m3.M3_BF16)
    assert m3.prefill_gated_kernel_used(shape) == m3.M3_KERNEL_STREAM
    d = inputs.make_prefill_inputs(w, seed=901)
    c = inputs.random_carry(w, seed=902)
    z, wy, wz = _gate_inputs(w, 903, (w.batch, w.seqlen), True, True)
    dg, cg = dev_inputs(d), dev_inputs(c)
    note(f"prefill gated stream {name} {kw}")
    out, h = m3.scan_prefill_gated(**{k: dg[k] for k in KEYS}, **cg, z=z.cuda(), w_y=wy.cuda(), w_z=wz.cuda(),
                                   chunk=64)
    torch.cuda.synchronize()
    heads = [0, w.nheads - 1]
    sub = lambda t: None if t is None else t[:, :, heads]
    d2 = {k: (v[heads] if k == "A" else sub(v)) for k, v in d.items()}
    c2 = {k: v[:, heads] for k, v in c.items()}
    yref, href = oracle.scan(**oracle_inputs({**d2, **c2}))
    zn, wyn, wzn = _np(z[:, :, heads]), _np(wy[heads]), _np(wz[heads])
    ref = oracle.gated_readout(yref, zn, wyn, wzn)
    tol = TOL[w.dtype]
    check_blocks(to64(out[:, :, heads]), ref, tol, (1, 3), "gated out", elem_axes=(3,),
                 elem_scale=gate_scale(yref, zn, wyn, wzn, block_axes=(1, 3, 4)))
    check_blocks(to64(h[:, heads]), href, tol, (2, 3), "h_out")
