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

from _parity import TOL, check_blocks, dev_inputs, note, taken_chunk, to64

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


PREFILL = [
    # (workload, overrides, chunk, biases, carry)
    ("siso", dict(batch=2, seqlen=300, nheads=3), 64, True, True),
    # two output tiles per wave: no fused variant is launched (the prologue's
    # variants with more than one tile per wave spilled to scratch, and one of
    # them made a GPU memory fault whose cause was not established), so the
    # prologue is staged before the plain prefill
    ("siso", dict(batch=1, seqlen=333, nheads=2), 256, True, True),
    ("siso", dict(batch=2, seqlen=200, nheads=2, rank=2), 128, True, True),
    # the bf16 MIMO shape at N = 128: fused into the streaming kernel (the
    # per-chunk kernel's variant there uses scratch)
    ("mimo", dict(batch=2, seqlen=300, nheads=3), 0, True, True),
    ("mimo", dict(batch=1, seqlen=129, nheads=2), 64, False, False),
    ("mimo", dict(batch=1, seqlen=700, nheads=2, rank=2), 64, True, True),
    ("mimo", dict(batch=1, seqlen=400, nheads=2, dstate=64), 64, True, True),
    ("siso", dict(batch=2, seqlen=200, nheads=2), 128, False, False),
    ("mimo", dict(batch=2, seqlen=130, nheads=2), 64, True, True),
    ("mimo", dict(batch=1, seqlen=97, nheads=2), 32, False, True),
    ("mimo", dict(batch=1, seqlen=70, nheads=2, rank=2, dstate=64), 64, True, True),
    ("mimo", dict(batch=1, seqlen=90, nheads=2, rank=8, dstate=32), 16, True, True),
    ("mimo", dict(batch=1, seqlen=90, nheads=1, rank=8, headdim=128, dstate=128), 16, True, True),
    ("mimo", dict(batch=2, seqlen=130, nheads=2, dstate=64), 32, True, True),
    ("mimo", dict(batch=1, seqlen=150, nheads=2, dstate=64, rank=2), 64, False, True),
    ("tiny", dict(batch=1, seqlen=100, nheads=2, rank=4, headdim=32, dstate=32), 32, True, True),   # fp32
    ("tiny", dict(batch=2, seqlen=77, nheads=1), 16, True, True),                                    # fp32 R=1
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: f"{c[0]}-{c[1]}-q{c[2]}-b{int(c[3])}c{int(c[4])}")
def test_prefill_prologue(case):
    name, kw, chunk, biases, carry = case
    w = inputs.workload(name, **kw)
    seed, eps = 700 + chunk + w.rank, 1e-5
    d = inputs.make_prefill_inputs(w, seed=seed)
    c = inputs.random_carry(w, seed=seed + 1) if carry else {}
    th, bb, bc = _pro_inputs(w, seed + 2, (w.batch, w.seqlen), biases)
    dg, cg = dev_inputs(d), (dev_inputs(c) if c else {})
    if taken_chunk(w, chunk, "prologue") == 0:
        # refused on the host: only where the plain prefill refuses the shape
        # too (the staged form takes every shape the plain prefill takes)
        assert taken_chunk(w, chunk) == 0
        note(f"prefill prologue {name} {kw} chunk={chunk}: refused on the host")
        with pytest.raises(m3.M3Error, match="M3_ERR_SHAPE"):
            m3.scan_prefill_prologue(dg["x"], dg["B"], dg["C"], dg["dt"], dg["A"], dg["lam"], th.cuda(), **cg,
                                     chunk=chunk, eps=eps)
        return
    code = m3.M3_BF16 if w.dtype == "bf16" else m3.M3_FP32
    mode = m3.prefill_prologue_mode(m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank,
                                                  chunk, code))
    note(f"prefill prologue {name} {kw} {w.dtype} chunk={chunk} biases={biases} carry={carry} mode={mode}")
    y, h = m3.scan_prefill_prologue(dg["x"], dg["B"], dg["C"], dg["dt"], dg["A"], dg["lam"], th.cuda(), **cg,
                                    chunk=chunk, eps=eps, bias_B=None if bb is None else bb.cuda(),
                                    bias_C=None if bc is None else bc.cuda())
    torch.cuda.synchronize()
    yr, hr = oracle.scan_prologue(_np(d["x"]), _np(d["B"]), _np(d["C"]), _np(d["dt"]), _np(d["A"]), _np(d["lam"]),
                                  _np(th), h0=_np(c.get("h0")), B_prev=_np(c.get("B_prev")),
                                  x_prev=_np(c.get("x_prev")), eps=eps, bias_B=_np(bb), bias_C=_np(bc))
    tol = TOL[w.dtype]
    check_blocks(to64(y), yr, tol, (1, 3, 4), "prologue y", elem_axes=(3, 4))
    check_blocks(to64(h), hr, tol, (2, 3), "prologue h_out")


def test_prologue_prefill_then_decode():
    """prefill with the prologue over L - 2 tokens, then two decode steps with
    it, equals the prologue's recurrence over the whole sequence."""
    w = inputs.workload("mimo", batch=2, seqlen=70, nheads=2, dstate=64)
    d = inputs.make_prefill_inputs(w, seed=801)
    th, bb, bc = _pro_inputs(w, 802, (w.batch, w.seqlen), True)
    dg = dev_inputs(d)
    thg, bbg, bcg = th.cuda(), bb.cuda(), bc.cuda()
    L0 = w.seqlen - 2
    note("prologue prefill then prologue decode")
    cut = lambda t: t[:, :L0].contiguous()
    y0, h = m3.scan_prefill_prologue(cut(dg["x"]), cut(dg["B"]), cut(dg["C"]), cut(dg["dt"]), dg["A"], cut(dg["lam"]),
                                     cut(thg), chunk=32, eps=1e-5, bias_B=bbg, bias_C=bcg)
    ys = [y0]
    for t in (L0, L0 + 1):
        at = lambda k: dg[k][:, t].contiguous()
        yt = m3.decode_step_prologue(h, at("x"), at("B"), at("C"), at("dt"), dg["A"], at("lam"),
                                     thg[:, t].contiguous(), B_prev=dg["B"][:, t - 1].contiguous(),
                                     x_prev=dg["x"][:, t - 1].contiguous(), eps=1e-5, bias_B=bbg, bias_C=bcg)
        ys.append(yt[:, None])
    torch.cuda.synchronize()
    yr, hr = oracle.scan_prologue(_np(d["x"]), _np(d["B"]), _np(d["C"]), _np(d["dt"]), _np(d["A"]), _np(d["lam"]),
                                  _np(th), eps=1e-5, bias_B=_np(bb), bias_C=_np(bc))
    check_blocks(to64(torch.cat(ys, dim=1)), yr, TOL[w.dtype], (1, 3, 4), "y", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL[w.dtype], (2, 3), "h")


def test_fused_entry_points_edges():
    """L = 0 (h_out receives h0), L = 1 with h_out aliasing h0, for the gated
    and prologue prefill entry points."""
    w = inputs.workload("mimo", batch=2, seqlen=1, nheads=2, dstate=64)
    d = inputs.make_prefill_inputs(w, seed=901)
    c = inputs.random_carry(w, seed=902)
    dg, cg = dev_inputs(d), dev_inputs(c)
    th, bb, bc = _pro_inputs(w, 903, (w.batch, w.seqlen), True)
    note("fused entry points: L=1 in place, L=0")
    h_io = cg["h0"].clone()
    y, h = m3.scan_prefill_prologue(dg["x"], dg["B"], dg["C"], dg["dt"], dg["A"], dg["lam"], th.cuda(),
                                    h0=h_io, B_prev=cg["B_prev"], x_prev=cg["x_prev"], h_out=h_io, chunk=16,
                                    eps=1e-5, bias_B=bb.cuda(), bias_C=bc.cuda())
    torch.cuda.synchronize()
    assert h.data_ptr() == h_io.data_ptr()
    yr, hr = oracle.scan_prologue(_np(d["x"]), _np(d["B"]), _np(d["C"]), _np(d["dt"]), _np(d["A"]), _np(d["lam"]),
                                  _np(th), h0=_np(c["h0"]), B_prev=_np(c["B_prev"]), x_prev=_np(c["x_prev"]),
                                  eps=1e-5, bias_B=_np(bb), bias_C=_np(bc))
    check_blocks(to64(y), yr, TOL[w.dtype], (1, 3, 4), "y L=1", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL[w.dtype], (2, 3), "h L=1")
    d0 = dev_inputs(inputs.make_prefill_inputs(w, seed=901, seqlen=0))
    z0 = torch.empty((w.batch, 0, w.nheads, w.headdim), dtype=w.torch_dtype, device="cuda")
    out0, h0 = m3.scan_prefill_gated(d0["x"], d0["B"], d0["C"], d0["dt"], d0["A"], d0["lam"], d0["theta"],
                                     h0=cg["h0"], z=z0, chunk=16)
    y0, h1 = m3.scan_prefill_prologue(d0["x"], d0["B"], d0["C"], d0["dt"], d0["A"], d0["lam"], d0["theta"],
                                      h0=cg["h0"], chunk=16)
    torch.cuda.synchronize()
    assert out0.numel() == 0 and y0.numel() == 0
    assert torch.equal(h0, cg["h0"]) and torch.equal(h1, cg["h0"])


@pytest.mark.parametrize("kernel", ["stream", "per_chunk"])
def test_prefill_prologue_full_size(kernel):
    """The MIMO workload at full size (4 x 4,096 tokens x 32 heads, N = 128,
    R = 4) through m3_scan_prefill_prologue, every head run: fused into the
    streaming kernel (the library's choice), and with the per-chunk kernel
    forced, whose prologue variant there is not launched, so the prologue is
    staged before it; y and the final state of two heads compared with the
    oracle."""
    w = inputs.workload("mimo")
    shape = m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 0, m3.M3_BF16)
    d = inputs.make_prefill_inputs(w, seed=811)
    c = inputs.random_carry(w, seed=812)
    th, bb, bc = _pro_inputs(w, 813, (w.batch, w.seqlen), True)
    dg, cg = dev_inputs(d), dev_inputs(c)
    m3.debug_set_prefill_kernel(m3.M3_KERNEL_STREAM if kernel == "stream" else m3.M3_KERNEL_PER_CHUNK)
    try:
        mode = m3.prefill_prologue_mode(shape)
        assert mode == (m3.M3_PROLOGUE_FUSED if kernel == "stream" else m3.M3_PROLOGUE_STAGED)
        assert m3.prefill_prologue_kernel_used(shape) == (m3.M3_KERNEL_STREAM if kernel == "stream"
                                                          else m3.M3_KERNEL_PER_CHUNK)
        note(f"prefill prologue full size mimo ({kernel}, mode {mode})")
        y, h = m3.scan_prefill_prologue(dg["x"], dg["B"], dg["C"], dg["dt"], dg["A"], dg["lam"], th.cuda(), **cg,
                                        eps=1e-5, bias_B=bb.cuda(), bias_C=bc.cuda())
        torch.cuda.synchronize()
    finally:
        m3.debug_set_prefill_kernel(0)
    heads = [0, w.nheads - 1]
    tk = lambda t: _np(t[:, :, heads])
    sq = lambda t: _np(t[:, heads])
    yr, hr = oracle.scan_prologue(tk(d["x"]), tk(d["B"]), tk(d["C"]), tk(d["dt"]), _np(d["A"][heads]),
                                  tk(d["lam"]), tk(th), h0=sq(c["h0"]), B_prev=sq(c["B_prev"]),
                                  x_prev=sq(c["x_prev"]), eps=1e-5, bias_B=_np(bb[heads]), bias_C=_np(bc[heads]))
    check_blocks(to64(y[:, :, heads]), yr, TOL["bf16"], (1, 3, 4), "prologue y", elem_axes=(3, 4))
    check_blocks(to64(h[:, heads]), hr, TOL["bf16"], (2, 3), "prologue h_out")


def test_prefill_prologue_stream_long_chain():
    """The streaming kernel's fused prologue with many chunks of a sequence in
    flight (maps in use): 8,192 tokens of two heads at the long shape."""
    w = inputs.workload("long", seqlen=8192, nheads=2)
    d = inputs.make_prefill_inputs(w, seed=821)
    c = inputs.random_carry(w, seed=822)
    th, bb, bc = _pro_inputs(w, 823, (w.batch, w.seqlen), True)
    dg, cg = dev_inputs(d), dev_inputs(c)
    shape = m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 64, m3.M3_BF16)
    assert m3.prefill_prologue_mode(shape) == m3.M3_PROLOGUE_FUSED
    note("prefill prologue long chain (stream, maps)")
    y, h = m3.scan_prefill_prologue(dg["x"], dg["B"], dg["C"], dg["dt"], dg["A"], dg["lam"], th.cuda(), **cg,
                                    chunk=64, eps=1e-5, bias_B=bb.cuda(), bias_C=bc.cuda())
    torch.cuda.synchronize()
    yr, hr = oracle.scan_prologue(_np(d["x"]), _np(d["B"]), _np(d["C"]), _np(d["dt"]), _np(d["A"]), _np(d["lam"]),
                                  _np(th), h0=_np(c["h0"]), B_prev=_np(c["B_prev"]), x_prev=_np(c["x_prev"]),
                                  eps=1e-5, bias_B=_np(bb), bias_C=_np(bc))
    check_blocks(to64(y), yr, TOL["bf16"], (1, 3, 4), "prologue y", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL["bf16"], (2, 3), "prologue h_out")
