"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Small cases span several chunks and MFMA tiles with ragged tails; the workload
cases run at full size in the bench's launch configuration and compare every
head of every sequence (the oracle computes each (batch, head) independently;
the long workload in groups of heads to bound host memory).
"""
import numpy as np
import pytest
import torch

import oracle
import state_space_sequence_02_amd as m3
from state_space_sequence_02_amd import inputs

from _parity import TOL, check_blocks, dev_inputs, note, oracle_inputs, taken_chunk, to64

pytestmark = pytest.mark.gpu

PREFILL_KEYS = ("x", "B", "C", "dt", "A", "lam", "theta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m3.load_library()


def _run_prefill(d, carry=None, chunk=0, h_out=None, want_state=True):
    kw = {k: d[k] for k in PREFILL_KEYS}
    if carry:
        kw.update(carry)
    y, h = m3.scan_prefill(**kw, chunk=chunk, h_out=h_out, want_state=want_state)
    torch.cuda.synchronize()
    return y, h


def _prefill_case(w, seed, carry, chunk, heads=None, seqlen=None):
    d = inputs.make_prefill_inputs(w, seed=seed, seqlen=seqlen)
    c = inputs.random_carry(w, seed=seed + 100) if carry else None
    dg = dev_inputs(d)
    cg = dev_inputs(c) if c else None
    note(f"prefill {w.name} b={w.batch} L={seqlen or w.seqlen} H={w.nheads} P={w.headdim} "
         f"N={w.dstate} R={w.rank} {w.dtype} chunk={chunk} carry={carry} seed={seed}")
    y, h = _run_prefill(dg, cg, chunk)
    o = oracle_inputs({**d, **(c or {})}, heads)
    yr, hr = oracle.scan(**o)
    yg, hg = to64(y), to64(h)
    if heads is not None:
        yg, hg = yg[:, :, heads], hg[:, heads]
    tol = TOL[w.dtype]
    e1 = check_blocks(yg, yr, tol, (1, 3, 4), "y", elem_axes=(3, 4))
    e2 = check_blocks(hg, hr, tol, (2, 3), "h_out")
    return e1, e2


SMALL = [
    dict(name="tiny", kw={}, chunk=64),
    dict(name="tiny", kw={}, chunk=16),
    dict(name="tiny", kw=dict(batch=2, seqlen=150, nheads=3, headdim=32, dstate=64, rank=2), chunk=32),
    dict(name="siso", kw=dict(batch=2, seqlen=200, nheads=3), chunk=64),
    dict(name="siso", kw=dict(batch=1, seqlen=333, nheads=2, headdim=32, dstate=32), chunk=128),
    dict(name="mimo", kw=dict(batch=1, seqlen=130, nheads=2), chunk=32),
    dict(name="mimo", kw=dict(batch=2, seqlen=97, nheads=2), chunk=64),
    dict(name="mimo", kw=dict(batch=1, seqlen=70, nheads=2, headdim=16, dstate=16, rank=8), chunk=16),
    dict(name="mimo", kw=dict(batch=1, seqlen=90, nheads=1, headdim=128, dstate=64, rank=2), chunk=32),
    dict(name="long", kw=dict(seqlen=515, nheads=2), chunk=64),
    # 256 and 512 (token, rank) rows per chunk: two and four 16-row output tiles per wave
    dict(name="siso", kw=dict(batch=1, seqlen=600, nheads=2), chunk=256),
    dict(name="mimo", kw=dict(batch=1, seqlen=300, nheads=2, headdim=64, dstate=32, rank=4), chunk=128),
    dict(name="tiny", kw=dict(batch=1, seqlen=700, nheads=2, headdim=32, dstate=16, rank=2), chunk=256),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c['name']}-{c['kw']}-q{c['chunk']}")
@pytest.mark.parametrize("carry", [False, True])
def test_prefill_small(case, carry):
    w = inputs.workload(case["name"], **case["kw"])
    _prefill_case(w, seed=3, carry=carry, chunk=case["chunk"])


def test_prefill_many_pairs_state_chain():
    """128 (sequence, head) pairs: at most 4 chunks of a sequence are resident at
    once, so chunks hand over states only (no maps)."""
    w = inputs.workload("siso", batch=4, seqlen=300, nheads=32)
    _prefill_case(w, seed=61, carry=True, chunk=64, heads=[0, 13, 31])


def test_prefill_without_rotation():
    w = inputs.workload("mimo", batch=1, seqlen=150, nheads=2, rotation=False)
    _prefill_case(w, seed=4, carry=True, chunk=32)
    w = inputs.workload("tiny", seqlen=100, rotation=False)
    _prefill_case(w, seed=4, carry=True, chunk=32)


@pytest.mark.parametrize("chunk", [64, 128])
def test_large_phases_fp32(chunk):
    """fp32 inputs with angles near 3 rad per step, so the chunk-local phases the
    prefill turns into cos/sin reach hundreds of radians (about 190 at chunk 64,
    380 at 128), held to the fp32 tolerance; the decode step takes the same
    angles one at a time."""
    w = inputs.workload("tiny", batch=1, seqlen=300, nheads=2, headdim=16, dstate=32, rank=2)
    d = inputs.make_prefill_inputs(w, seed=21)
    g = torch.Generator().manual_seed(22)
    d["theta"] = (2.9 + 0.2 * torch.rand(d["theta"].shape, generator=g)).to(torch.float32)
    assert taken_chunk(w, chunk) == chunk
    note(f"prefill fp32 large phases chunk={chunk}")
    y, h = _run_prefill(dev_inputs(d), chunk=chunk)
    yr, hr = oracle.scan(**oracle_inputs(d))
    check_blocks(to64(y), yr, TOL["fp32"], (1, 3, 4), "y", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL["fp32"], (2, 3), "h_out")


def test_zero_angles_match_no_rotation_bitwise():
    w = inputs.workload("mimo", batch=1, seqlen=100, nheads=2)
    d = dev_inputs(inputs.make_prefill_inputs(w, seed=5))
    note("prefill theta=0 vs theta=NULL")
    y0, h0 = _run_prefill(dict(d, theta=torch.zeros_like(d["theta"])), chunk=32)
    yn, hn = _run_prefill(dict(d, theta=None), chunk=32)
    assert torch.equal(y0, yn) and torch.equal(h0, hn)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_chunk_size_invariance(dtype):
    w = inputs.workload("mimo", batch=1, seqlen=300, nheads=2, rank=2, dstate=64, dtype=dtype)
    d = inputs.make_prefill_inputs(w, seed=6)
    c = inputs.random_carry(w, seed=7)
    dg, cg = dev_inputs(d), dev_inputs(c)
    yr, hr = oracle.scan(**oracle_inputs({**d, **c}))
    outs = []
    # (fp32 at 128 tokens x R = 2: the tiles do not fit one compute unit's LDS,
    # so the library refuses that chunk)
    chunks = [q for q in (16, 32, 64, 128) if taken_chunk(w, q) == q]
    assert chunks[:3] == [16, 32, 64]
    for q in chunks:
        note(f"chunk invariance {dtype} q={q}")
        y, h = _run_prefill(dg, cg, chunk=q)
        check_blocks(to64(y), yr, TOL[dtype], (1, 3, 4), f"y q={q}", elem_axes=(3, 4))
        check_blocks(to64(h), hr, TOL[dtype], (2, 3), f"h q={q}")
        outs.append((to64(y), to64(h)))
    for y, h in outs[1:]:
        check_blocks(y, outs[0][0], TOL[dtype], (1, 3, 4), "y vs q=16", elem_axes=(3, 4))


def test_run_twice_bit_exact():
    """64 (sequence, head) pairs at N=128: one workgroup per compute unit fits, so
    at most 4 chunks of a sequence are in flight and chunks hand over states
    only, in a fixed order: two runs give the same bits.  (With fewer pairs a
    chunk may compose its predecessors' maps instead, whose products associate
    differently, so runs agree to rounding only; the parity tests cover that.)"""
    w = inputs.workload("mimo", batch=4, seqlen=257, nheads=16)
    dg = dev_inputs(inputs.make_prefill_inputs(w, seed=8))
    note("prefill run twice")
    y1, h1 = _run_prefill(dg, chunk=32)
    y2, h2 = _run_prefill(dg, chunk=32)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def _shape_of(w, chunk):
    dcode = m3.M3_BF16 if w.dtype == "bf16" else m3.M3_FP32
    return m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, chunk, dcode)


def test_workspace_reused_across_calls_and_shapes():
    """One workspace, zero-filled once, serves successive calls of different
    shapes with nothing done in between; the last call repeats the first shape
    with other inputs, so a flag left by the first call that still counted would
    hand it a stale state."""
    cases = [(inputs.workload("siso", batch=2, seqlen=600, nheads=3), 32),
             (inputs.workload("siso", batch=1, seqlen=70, nheads=2), 16),
             (inputs.workload("mimo", batch=1, seqlen=200, nheads=2), 32),
             (inputs.workload("siso", batch=2, seqlen=600, nheads=3), 32)]
    need = max(m3.prefill_workspace_bytes(_shape_of(w, q)) for w, q in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (w, q) in enumerate(cases):
        d = inputs.make_prefill_inputs(w, seed=70 + i)
        dg = dev_inputs(d)
        note(f"prefill call {i} on a shared workspace: {w.name} b={w.batch} L={w.seqlen} H={w.nheads} chunk={q}")
        y, h = m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS}, chunk=q, workspace=ws)
        torch.cuda.synchronize()
        yr, hr = oracle.scan(**oracle_inputs(d))
        check_blocks(to64(y), yr, TOL[w.dtype], (1, 3, 4), f"y call {i}", elem_axes=(3, 4))
        check_blocks(to64(h), hr, TOL[w.dtype], (2, 3), f"h_out call {i}")


def test_prefill_graph_replay():
    """A prefill captured in a HIP graph is right on every replay, with eager
    calls on the same workspace between the replays."""
    w = inputs.workload("mimo", batch=2, seqlen=300, nheads=2)
    d = inputs.make_prefill_inputs(w, seed=81)
    dg = dev_inputs(d)
    kw = {k: dg[k] for k in PREFILL_KEYS}
    yr, hr = oracle.scan(**oracle_inputs(d))
    ws = torch.zeros(m3.prefill_workspace_bytes(_shape_of(w, 32)), dtype=torch.uint8, device="cuda")
    y, h = torch.empty_like(dg["x"]), torch.empty((w.batch, w.nheads, w.dstate, w.headdim), device="cuda")
    note("prefill graph capture")
    m3.scan_prefill(**kw, y=y, h_out=h, chunk=32, workspace=ws)   # eager, before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            m3.scan_prefill(**kw, y=y, h_out=h, chunk=32, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        h.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_blocks(to64(y), yr, TOL[w.dtype], (1, 3, 4), f"y replay {rep}", elem_axes=(3, 4))
        check_blocks(to64(h), hr, TOL[w.dtype], (2, 3), f"h_out replay {rep}")
        ye, he = m3.scan_prefill(**kw, chunk=32, workspace=ws)   # eager, same workspace
        torch.cuda.synchronize()
        check_blocks(to64(ye), yr, TOL[w.dtype], (1, 3, 4), f"y eager after replay {rep}", elem_axes=(3, 4))
        check_blocks(to64(he), hr, TOL[w.dtype], (2, 3), f"h_out eager after replay {rep}")


def test_state_in_place_and_empty_and_single():
    w = inputs.workload("siso", batch=2, seqlen=1, nheads=3)
    d = inputs.make_prefill_inputs(w, seed=9)
    c = inputs.random_carry(w, seed=10)
    dg, cg = dev_inputs(d), dev_inputs(c)
    yr, hr = oracle.scan(**oracle_inputs({**d, **c}))
    note("prefill L=1, h_out aliases h0")
    h_io = cg["h0"].clone()
    y, h = _run_prefill(dg, dict(cg, h0=h_io), chunk=64, h_out=h_io)
    assert h.data_ptr() == h_io.data_ptr()
    check_blocks(to64(y), yr, TOL["bf16"], (1, 3, 4), "y L=1", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL["bf16"], (2, 3), "h L=1")
    note("prefill L=0")
    d0 = dev_inputs(inputs.make_prefill_inputs(w, seed=9, seqlen=0))
    y0, h0 = _run_prefill(d0, cg, chunk=64)
    assert y0.numel() == 0 and torch.equal(h0, cg["h0"])
    y0, h0 = _run_prefill(d0, None, chunk=64)
    assert not h0.any()


def test_prefill_errors_surface():
    w = inputs.workload("siso", batch=1, seqlen=16, nheads=1)
    dg = dev_inputs(inputs.make_prefill_inputs(w, seed=11))
    note("prefill error paths")
    with pytest.raises(m3.M3Error, match="M3_ERR_WORKSPACE"):
        m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS},
                        workspace=torch.empty(8, dtype=torch.uint8, device="cuda"))
    with pytest.raises(m3.M3Error, match="M3_ERR_ALIAS"):
        m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS}, y=dg["x"])


# ---------------------------------------------------------------------------
# decode

def _decode_case(w, steps, seed, carry_prev=True, h_init=None):
    d = inputs.make_decode_inputs(w, seed=seed, steps=steps)
    dg = dev_inputs(d)
    b, H, N, P = w.batch, w.nheads, w.dstate, w.headdim
    h0 = torch.randn((b, H, N, P), generator=torch.Generator().manual_seed(seed + 1)) * 0.5 \
        if h_init is None else h_init
    h = h0.to("cuda").contiguous().clone()
    ys = []
    note(f"decode b={b} H={H} P={P} N={N} R={w.rank} {w.dtype} steps={steps} seed={seed}")
    for s in range(steps):
        kw = {}
        if s > 0 and carry_prev:
            kw = dict(B_prev=dg["B"][s - 1], x_prev=dg["x"][s - 1])
        ys.append(m3.decode_step(h, dg["x"][s], dg["B"][s], dg["C"][s], dg["dt"][s], dg["A"],
                                 dg["lam"][s], dg["theta"][s] if dg["theta"] is not None else None, **kw))
    torch.cuda.synchronize()
    y = torch.stack(ys)
    return d, h0, y, h


@pytest.mark.parametrize("shape", [
    dict(batch=3, nheads=2, headdim=64, dstate=128, rank=4, dtype="bf16"),
    dict(batch=2, nheads=3, headdim=64, dstate=64, rank=1, dtype="bf16"),
    dict(batch=2, nheads=2, headdim=16, dstate=16, rank=1, dtype="fp32"),
    dict(batch=2, nheads=2, headdim=32, dstate=64, rank=2, dtype="fp32"),
    dict(batch=1, nheads=2, headdim=128, dstate=256, rank=8, dtype="bf16"),
])
def test_decode_small(shape):
    w = inputs.workload("decode", **shape)
    d, h0, y, h = _decode_case(w, steps=12, seed=12)
    yr, hr = oracle.decode_steps(h0, d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"])
    tol = TOL[w.dtype]
    check_blocks(to64(y), yr, tol, (3, 4), "decode y")
    check_blocks(to64(h), hr, tol, (2, 3), "decode h")


def test_decode_several_pairs_per_workgroup():
    """640 (sequence, head) pairs at N=128, P=64, R=4: more workgroups (one
    per pair) than fit on the chip at once, so later ones start on compute
    units that earlier ones free."""
    w = inputs.workload("decode", batch=20, nheads=32, headdim=64, dstate=128, rank=4, dtype="bf16")
    d, h0, y, h = _decode_case(w, steps=3, seed=21)
    yr, hr = oracle.decode_steps(h0, d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"])
    tol = TOL[w.dtype]
    check_blocks(to64(y), yr, tol, (3, 4), "decode y")
    check_blocks(to64(h), hr, tol, (2, 3), "decode h")


@pytest.mark.parametrize("shape", [
    dict(batch=3, nheads=2, headdim=64, dstate=128, rank=4),
    dict(batch=2, nheads=3, headdim=64, dstate=64, rank=1),
    dict(batch=1, nheads=2, headdim=128, dstate=256, rank=8),
    dict(batch=20, nheads=32, headdim=64, dstate=128, rank=4),
])
def test_decode_bf16_state(shape):
    """The state kept in bf16 between steps, against the oracle's bf16-state
    decode (the update in high precision, the stored state rounded to nearest
    even bf16)."""
    w = inputs.workload("decode", dtype="bf16", **shape)
    steps = 12 if w.batch * w.nheads < 100 else 3
    d = inputs.make_decode_inputs(w, seed=51, steps=steps)
    dg = dev_inputs(d)
    h0 = torch.randn((w.batch, w.nheads, w.dstate, w.headdim), generator=torch.Generator().manual_seed(52)) * 0.5
    h = h0.to(torch.bfloat16).to("cuda")
    note(f"decode bf16 state b={w.batch} H={w.nheads} N={w.dstate} P={w.headdim} R={w.rank} steps={steps}")
    ys = []
    for s in range(steps):
        kw = dict(B_prev=dg["B"][s - 1], x_prev=dg["x"][s - 1]) if s else {}
        ys.append(m3.decode_step(h, dg["x"][s], dg["B"][s], dg["C"][s], dg["dt"][s], dg["A"], dg["lam"][s],
                                 dg["theta"][s], **kw))
    torch.cuda.synchronize()
    yr, hr = oracle.decode_steps_bf16_state(h0.to(torch.bfloat16).double().numpy(), d["x"], d["B"], d["C"],
                                            d["dt"], d["A"], d["lam"], d["theta"])
    check_blocks(to64(torch.stack(ys)), yr, TOL["bf16"], (3, 4), "decode bf16-state y")
    check_blocks(to64(h), hr, TOL["bf16"], (2, 3), "decode bf16-state h")
    assert h.dtype == torch.bfloat16


def test_decode_graph_replay_matches_eager():
    """Decode steps captured in a HIP graph give the eager calls' bits on every
    replay, with unrelated eager work and synchronisations between replays."""
    w = inputs.workload("decode", batch=4, nheads=8, headdim=64, dstate=128, rank=4, dtype="bf16")
    steps = 3
    d = inputs.make_decode_inputs(w, seed=31, steps=steps)
    dg = dev_inputs(d)
    h0 = (torch.randn((w.batch, w.nheads, w.dstate, w.headdim), generator=torch.Generator().manual_seed(32))
          * 0.5).to("cuda")

    def run(h, ys):
        for s in range(steps):
            kw = dict(B_prev=dg["B"][s - 1], x_prev=dg["x"][s - 1]) if s else {}
            m3.decode_step(h, dg["x"][s], dg["B"][s], dg["C"][s], dg["dt"][s], dg["A"], dg["lam"][s],
                           dg["theta"][s], y=ys[s], **kw)

    note("decode graph replay vs eager")
    h_ref = h0.clone()
    y_ref = [torch.empty_like(dg["x"][0]) for _ in range(steps)]
    run(h_ref, y_ref)
    torch.cuda.synchronize()
    h = torch.empty_like(h0)
    ys = [torch.empty_like(dg["x"][0]) for _ in range(steps)]
    h.copy_(h0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(h, ys)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        h.copy_(h0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref), f"state differs on replay {rep}"
        for s in range(steps):
            assert torch.equal(ys[s], y_ref[s]), f"y of step {s} differs on replay {rep}"
        float(torch.randn(4096, device="cuda").square().sum())   # unrelated eager work


def test_prefill_then_decode_handoff():
    """prefill(L - k) followed by k decode steps equals prefill(L)."""
    w = inputs.workload("mimo", batch=2, seqlen=133, nheads=2)
    d = inputs.make_prefill_inputs(w, seed=13)
    c = inputs.random_carry(w, seed=14)
    dg, cg = dev_inputs(d), dev_inputs(c)
    k, L = 5, w.seqlen
    note("handoff prefill + decode")
    pre = {kk: (v[:, :L - k].contiguous() if kk in ("x", "B", "C", "dt", "lam", "theta") else v)
           for kk, v in dg.items()}
    y_pre, h = _run_prefill(pre, cg, chunk=32)
    ys = []
    for t in range(L - k, L):
        ys.append(m3.decode_step(h, dg["x"][:, t].contiguous(), dg["B"][:, t].contiguous(),
                                 dg["C"][:, t].contiguous(), dg["dt"][:, t].contiguous(), dg["A"],
                                 dg["lam"][:, t].contiguous(), dg["theta"][:, t].contiguous(),
                                 B_prev=dg["B"][:, t - 1].contiguous(), x_prev=dg["x"][:, t - 1].contiguous()))
    torch.cuda.synchronize()
    yr, hr = oracle.scan(**oracle_inputs({**d, **c}))
    y_all = np.concatenate([to64(y_pre), np.stack([to64(v) for v in ys], axis=1)], axis=1)
    check_blocks(y_all, yr, TOL["bf16"], (1, 3, 4), "handoff y", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL["bf16"], (2, 3), "handoff h")


# ---------------------------------------------------------------------------
# full-size workloads, sampled heads

def test_workload_tiny_exact_config():
    w = inputs.WORKLOADS["tiny"]
    _prefill_case(w, seed=0, carry=False, chunk=w.chunk)


def test_workload_siso_full_size():
    w = inputs.WORKLOADS["siso"]
    _prefill_case(w, seed=0, carry=False, chunk=w.chunk)


def test_workload_mimo_full_size():
    w = inputs.WORKLOADS["mimo"]
    _prefill_case(w, seed=0, carry=False, chunk=w.chunk)


def test_refused_shapes_raise_before_launch():
    """Shapes the host plan refuses (512-row chunks, kernel variants that would
    use scratch memory, N = 256, which is decode-only) raise M3_ERR_SHAPE and
    launch nothing."""
    for name, kw, chunk in (("long", dict(seqlen=300, nheads=2), 128),
                            ("mimo", dict(batch=1, seqlen=90, nheads=1, headdim=128, dstate=128, rank=2), 32),
                            ("mimo", dict(batch=1, seqlen=64, nheads=1, headdim=64, dstate=256, rank=1), 32)):
        w = inputs.workload(name, **kw)
        assert taken_chunk(w, chunk) == 0
        dg = dev_inputs(inputs.make_prefill_inputs(w, seed=2))
        note(f"refused prefill {name} {kw} chunk={chunk}")
        with pytest.raises(m3.M3Error, match="M3_ERR_SHAPE"):
            _run_prefill(dg, chunk=chunk)


def test_workload_siso_default_chunk_all_heads():
    """The SISO workload exactly as the benchmark launches it (the library's
    default chunk, 128 tokens), every head of every sequence."""
    w = inputs.WORKLOADS["siso"]
    assert taken_chunk(w, 0) == 128
    _prefill_case(w, seed=0, carry=False, chunk=0)


def test_workload_long_full_size():
    w = inputs.WORKLOADS["long"]
    note("long: generating inputs on the device")
    d = inputs.make_prefill_inputs(w, seed=0, device="cuda")
    # the configuration's 128-token chunk is 512 (token, rank) rows, which do not
    # fit one compute unit; the largest chunk the library takes for it is used
    q = taken_chunk(w, 0)
    assert taken_chunk(w, w.chunk) == 0 and q == 64
    note(f"prefill long chunk={q}")
    y, h = _run_prefill(d, chunk=q)
    for g0 in range(0, w.nheads, 8):
        heads = list(range(g0, min(g0 + 8, w.nheads)))
        note(f"long: oracle for heads {heads[0]}..{heads[-1]}")
        yr, hr = oracle.scan(**oracle_inputs(d, heads))
        check_blocks(to64(y[:, :, heads]), yr, TOL["bf16"], (1, 3, 4), "long y", elem_axes=(3, 4))
        check_blocks(to64(h[:, heads]), hr, TOL["bf16"], (2, 3), "long h")
        del yr, hr


def test_workload_decode_full_size():
    w = inputs.WORKLOADS["decode"]
    note("decode workload: generating steps on the device")
    d = inputs.make_decode_inputs(w, seed=0, device="cuda")
    h = torch.zeros((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device="cuda")
    ys = []
    note("decode workload: 256 steps")
    for s in range(w.steps):
        kw = dict(B_prev=d["B"][s - 1], x_prev=d["x"][s - 1]) if s else {}
        ys.append(m3.decode_step(h, d["x"][s], d["B"][s], d["C"][s], d["dt"][s], d["A"], d["lam"][s],
                                 d["theta"][s], **kw))
    torch.cuda.synchronize()
    note("decode workload: oracle over every (sequence, head) pair")
    cpu = {k: (v.cpu() if v is not None else v) for k, v in d.items()}
    yr, hr = oracle.decode_steps(np.zeros((w.batch, w.nheads, w.dstate, w.headdim)), cpu["x"], cpu["B"], cpu["C"],
                                 cpu["dt"], cpu["A"], cpu["lam"], cpu["theta"])
    check_blocks(to64(torch.stack(ys)), yr, TOL["bf16"], (3, 4), "decode workload y")
    check_blocks(to64(h), hr, TOL["bf16"], (2, 3), "decode workload h")


def _rotate_pairs(S, ang, scale):
    """scale x R(ang) on row pairs (2k, 2k+1) of S [b, H, N, P]; ang [b, H, N/2], scale [b, H]."""
    c, s = torch.cos(ang)[..., None], torch.sin(ang)[..., None]
    e, o = S[:, :, 0::2], S[:, :, 1::2]
    out = torch.empty_like(S)
    out[:, :, 0::2] = c * e - s * o
    out[:, :, 1::2] = s * e + c * o
    return out * scale[:, :, None, None]


def test_sequence_shards_compose():
    """The sequence-sharding plan for the long prefill, run through the ABI on
    one GPU: the sequence is cut into 4 shards; pass 1 runs every shard from a
    zero state (its first token's delayed write taken from the previous
    shard's last B, x), giving its end state S_g; the shard's map is its total
    decay exp(A sum dt) and total angle sum(phi) per pair; the prefix
    T_g = a_g R(Psi_g) T_{g-1} + S_g gives every shard's entering state; pass 2
    reruns shards 1..3 from T_{g-1}.  The stitched y and the final state match
    the oracle over the whole sequence (with a non-zero incoming carry)."""
    w = inputs.workload("long", seqlen=4096, nheads=4)
    d = inputs.make_prefill_inputs(w, seed=31)
    c = inputs.random_carry(w, seed=32)
    dg, cg = dev_inputs(d), dev_inputs(c)
    G, L = 4, w.seqlen
    Ls = L // G
    sl = [slice(g * Ls, (g + 1) * Ls) for g in range(G)]
    part = lambda g, k: dg[k][:, sl[g]].contiguous()
    halo = lambda g: ((cg["B_prev"], cg["x_prev"]) if g == 0 else
                      (dg["B"][:, g * Ls - 1].contiguous(), dg["x"][:, g * Ls - 1].contiguous()))

    def run(g, h0):
        Bp, xp = halo(g)
        return m3.scan_prefill(part(g, "x"), part(g, "B"), part(g, "C"), part(g, "dt"), dg["A"], part(g, "lam"),
                               part(g, "theta"), h0=h0, B_prev=Bp, x_prev=xp, chunk=64)

    note("sharded prefill: pass 1 (zero entering state)")
    first = [run(g, cg["h0"] if g == 0 else None) for g in range(G)]
    T = first[0][1]
    ys = [first[0][0]]
    for g in range(1, G):
        a = torch.exp(dg["A"][None, :] * dg["dt"][:, sl[g]].double().sum(1).float())   # [b, H]
        psi = dg["theta"][:, sl[g]].double().sum(1).float()                              # [b, H, N/2]
        note(f"sharded prefill: pass 2, shard {g}")
        y, _ = run(g, T)
        ys.append(y)
        T = _rotate_pairs(T, psi, a) + first[g][1]
    torch.cuda.synchronize()
    yr, hr = oracle.scan(**oracle_inputs({**d, **c}))
    check_blocks(to64(torch.cat(ys, dim=1)), yr, TOL["bf16"], (1, 3, 4), "sharded y", elem_axes=(3, 4))
    check_blocks(to64(T), hr, TOL["bf16"], (2, 3), "sharded h_out")


# ---------------------------------------------------------------------------
# error reporting (forced from the host: every kernel still exits normally)

def _ws_for(w, chunk):
    return torch.zeros(m3.prefill_workspace_bytes(_shape_of(w, chunk)), dtype=torch.uint8, device="cuda")


def test_lookback_timeout_is_reported():
    """A look-back wait that gives up (the spin limit lowered to one poll, so
    chunks whose predecessors are still running give up) writes NaN for that
    chunk and sets the workspace's error word: m3_prefill_status reports
    M3_ERR_TIMEOUT once and clears it; the same workspace then serves a normal
    call whose outputs match the oracle."""
    w = inputs.workload("mimo", batch=1, seqlen=2048, nheads=2)
    d = inputs.make_prefill_inputs(w, seed=91)
    dg = dev_inputs(d)
    ws = _ws_for(w, 64)
    note("prefill with a one-poll look-back limit")
    try:
        m3.debug_set_spin_limit(1)
        y, h = m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS}, chunk=64, workspace=ws)
        st = m3.prefill_status(ws)
    finally:
        m3.debug_set_spin_limit(0)
    assert st in (0, 7)
    if st == 7:
        assert torch.isnan(y.float()).any()
    assert m3.prefill_status(ws) == 0          # cleared by the query
    note("prefill on the same workspace, default limit")
    y, h = m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS}, chunk=64, workspace=ws)
    assert m3.prefill_status(ws) == 0
    yr, hr = oracle.scan(**oracle_inputs(d))
    check_blocks(to64(y), yr, TOL["bf16"], (1, 3, 4), "y after timeout", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL["bf16"], (2, 3), "h after timeout")


def test_unzeroed_workspace_is_reported():
    """A workspace that was never zero-filled (all ones here) is reported by
    m3_prefill_status (M3_ERR_WORKSPACE for the out-of-range control word, or
    M3_ERR_TIMEOUT from waits on garbage flags, with the spin limit low so
    they give up at once) instead of silently wrong results; zero-filled, it
    then works."""
    w = inputs.workload("mimo", batch=1, seqlen=300, nheads=2)
    d = inputs.make_prefill_inputs(w, seed=92)
    dg = dev_inputs(d)
    ws = _ws_for(w, 32)
    ws.fill_(255)
    note("prefill on a workspace of all ones")
    try:
        m3.debug_set_spin_limit(4)
        m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS}, chunk=32, workspace=ws)
        st = m3.prefill_status(ws)
    finally:
        m3.debug_set_spin_limit(0)
    assert st in (4, 7), st
    ws.zero_()
    note("prefill on the same workspace, zero-filled")
    y, h = m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS}, chunk=32, workspace=ws)
    assert m3.prefill_status(ws) == 0
    yr, hr = oracle.scan(**oracle_inputs(d))
    check_blocks(to64(y), yr, TOL["bf16"], (1, 3, 4), "y", elem_axes=(3, 4))
