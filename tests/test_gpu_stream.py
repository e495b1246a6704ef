"""GPU parity of the streaming prefill kernel (M3_KERNEL_STREAM) against the
float64 oracle, through the C ABI.

The streaming kernel takes bf16 inputs with P = 64: N = 64 at R = 1, 2 or 4
with 128 or 256 (token, rank) rows per chunk, N = 128 at 128 rows (R = 1, 2,
4) or 256 rows (R = 4).  The cases cover every such (N, R, rows) combination,
both ways chunks hand over their states (maps, when
few sequences x heads leave many chunks of one sequence in flight; states
only, when many do), ragged last chunks, sequences shorter than a chunk, an
incoming carry, no rotation, a long chain of chunks, determinism, and one
workspace shared by calls of both kernels.  The per-chunk kernel runs on the
same inputs for comparison.
"""
import pytest
import torch

import oracle
import state_space_sequence_02_amd as m3
from state_space_sequence_02_amd import inputs

from _parity import TOL, check_blocks, dev_inputs, note, oracle_inputs, to64

pytestmark = pytest.mark.gpu

PREFILL_KEYS = ("x", "B", "C", "dt", "A", "lam", "theta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m3.load_library()


@pytest.fixture(autouse=True)
def _library_choice():
    # (the library takes the streaming kernel by itself at N = 128 only)
    m3.debug_set_prefill_kernel(m3.M3_KERNEL_STREAM)
    yield
    m3.debug_set_prefill_kernel(0)


def _shape(w, chunk):
    return m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, chunk, m3.M3_BF16)


def _check(d, c, y, h, heads, what):
    yr, hr = oracle.scan(**oracle_inputs({**d, **(c or {})}, heads))
    yg, hg = to64(y), to64(h)
    if heads is not None:
        yg, hg = yg[:, :, heads], hg[:, heads]
    check_blocks(yg, yr, TOL["bf16"], (1, 3, 4), f"y {what}", elem_axes=(3, 4))
    check_blocks(hg, hr, TOL["bf16"], (2, 3), f"h_out {what}")


def _run(w, seed, chunk, carry, heads=None, both=True):
    d = inputs.make_prefill_inputs(w, seed=seed)
    c = inputs.random_carry(w, seed=seed + 100) if carry else None
    dg = dev_inputs(d)
    cg = dev_inputs(c) if c else {}
    kw = {k: dg[k] for k in PREFILL_KEYS}
    assert m3.prefill_kernel_used(_shape(w, chunk)) == m3.M3_KERNEL_STREAM
    note(f"stream prefill b={w.batch} L={w.seqlen} H={w.nheads} N={w.dstate} R={w.rank} "
         f"chunk={chunk} carry={carry} seed={seed}")
    y, h = m3.scan_prefill(**kw, **cg, chunk=chunk)
    torch.cuda.synchronize()
    _check(d, c, y, h, heads, "stream")
    if both:
        m3.debug_set_prefill_kernel(m3.M3_KERNEL_PER_CHUNK)
        assert m3.prefill_kernel_used(_shape(w, chunk)) == m3.M3_KERNEL_PER_CHUNK
        note("  the same inputs on the per-chunk kernel")
        y1, h1 = m3.scan_prefill(**kw, **cg, chunk=chunk)
        torch.cuda.synchronize()
        m3.debug_set_prefill_kernel(m3.M3_KERNEL_STREAM)
        _check(d, c, y1, h1, heads, "per-chunk")
    return y, h


# (N, R, tokens per chunk): every (N, R, rows) the kernel takes
SHAPES = [(64, 1, 128), (64, 1, 256), (64, 2, 64), (64, 2, 128), (64, 4, 32), (64, 4, 64),
          (128, 1, 128), (128, 2, 64), (128, 4, 32), (128, 4, 64)]


@pytest.mark.parametrize("N,R,chunk", SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("carry", [False, True])
def test_stream_maps(N, R, chunk, carry):
    """Two sequences x heads: many chunks of one sequence in flight, maps in
    use; a ragged last chunk."""
    w = inputs.workload("mimo", batch=1, seqlen=5 * chunk + 37, nheads=2, dstate=N, rank=R)
    _run(w, seed=200 + N + R + chunk, chunk=chunk, carry=carry)


@pytest.mark.parametrize("N,R,chunk", [(64, 1, 128), (64, 4, 64), (128, 4, 64), (128, 2, 64), (128, 4, 32)],
                         ids=lambda v: str(v))
def test_stream_states_only(N, R, chunk):
    """64 sequences x heads: at most 4 chunks of a sequence in flight, states
    only; compared on a few heads of both sequences."""
    w = inputs.workload("mimo", batch=2, seqlen=3 * chunk + 11, nheads=32, dstate=N, rank=R)
    _run(w, seed=300 + N + R + chunk, chunk=chunk, carry=True, heads=[0, 17, 31])


@pytest.mark.parametrize("seqlen", [1, 2, 31, 63, 64, 65])
def test_stream_short_sequences(seqlen):
    """Sequences of one token up to just past one chunk (64 tokens at R = 4)."""
    w = inputs.workload("mimo", batch=2, seqlen=seqlen, nheads=3)
    _run(w, seed=400 + seqlen, chunk=64, carry=True, both=False)


def test_stream_without_rotation():
    w = inputs.workload("mimo", batch=1, seqlen=300, nheads=2, rotation=False)
    _run(w, seed=501, chunk=64, carry=True)
    w = inputs.workload("siso", batch=1, seqlen=700, nheads=2, rotation=False)
    _run(w, seed=502, chunk=256, carry=True)


def test_stream_long_chain():
    """8,192 tokens of two heads at 64 tokens per chunk: 128 chunks per
    sequence, up to ~128 of them in flight at once, long map chains."""
    w = inputs.workload("long", seqlen=8192, nheads=2)
    _run(w, seed=601, chunk=64, carry=True, both=False)


def test_stream_run_twice_bit_exact():
    """States only (64 sequences x heads at N = 128): a fixed order of hand-off,
    so two runs give the same bits."""
    w = inputs.workload("mimo", batch=4, seqlen=257, nheads=16)
    dg = dev_inputs(inputs.make_prefill_inputs(w, seed=701))
    kw = {k: dg[k] for k in PREFILL_KEYS}
    assert m3.prefill_kernel_used(_shape(w, 64)) == m3.M3_KERNEL_STREAM
    note("stream prefill run twice")
    y1, h1 = m3.scan_prefill(**kw, chunk=64)
    y2, h2 = m3.scan_prefill(**kw, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_workspace_shared_by_both_kernels():
    """One zero-filled workspace serves calls of the per-chunk kernel and the
    streaming kernel in turn (their control words leave it ready for either),
    each call checked against the oracle; the last repeats the first shape
    with other inputs, so a stale flag that still counted would show."""
    w = inputs.workload("mimo", batch=1, seqlen=400, nheads=2)
    ws = torch.zeros(m3.prefill_workspace_bytes(_shape(w, 64)), dtype=torch.uint8, device="cuda")
    for i, kern in enumerate([m3.M3_KERNEL_PER_CHUNK, m3.M3_KERNEL_STREAM, m3.M3_KERNEL_STREAM,
                              m3.M3_KERNEL_PER_CHUNK, m3.M3_KERNEL_STREAM]):
        m3.debug_set_prefill_kernel(kern)
        assert m3.prefill_kernel_used(_shape(w, 64)) == kern
        d = inputs.make_prefill_inputs(w, seed=800 + i)
        dg = dev_inputs(d)
        note(f"shared workspace call {i}, kernel {kern}")
        y, h = m3.scan_prefill(**{k: dg[k] for k in PREFILL_KEYS}, chunk=64, workspace=ws)
        torch.cuda.synchronize()
        assert m3.prefill_status(ws) == 0
        _check(d, None, y, h, None, f"call {i}")


def test_stream_timeout_and_unzeroed_workspace_are_reported():
    """The streaming kernel's error paths, forced from the host so every
    workgroup still exits: a one-poll look-back limit (maps, and states only),
    and a workspace of all ones; then a zero-filled workspace works."""
    for b, H in ((1, 2), (2, 32)):
        w = inputs.workload("mimo", batch=b, seqlen=1024, nheads=H)
        assert m3.prefill_kernel_used(_shape(w, 64)) == m3.M3_KERNEL_STREAM
        dg = dev_inputs(inputs.make_prefill_inputs(w, seed=900 + H))
        kw = {k: dg[k] for k in PREFILL_KEYS}
        ws = torch.zeros(m3.prefill_workspace_bytes(_shape(w, 64)), dtype=torch.uint8, device="cuda")
        note(f"stream prefill, one-poll look-back, b={b} H={H}")
        try:
            m3.debug_set_spin_limit(1)
            y, _ = m3.scan_prefill(**kw, chunk=64, workspace=ws)
            st = m3.prefill_status(ws)
        finally:
            m3.debug_set_spin_limit(0)
        assert st in (0, 7)
        if st == 7:
            assert torch.isnan(y.float()).any()
        assert m3.prefill_status(ws) == 0
        ws.fill_(255)
        note(f"stream prefill on a workspace of all ones, b={b} H={H}")
        try:
            m3.debug_set_spin_limit(4)
            m3.scan_prefill(**kw, chunk=64, workspace=ws)
            st = m3.prefill_status(ws)
        finally:
            m3.debug_set_spin_limit(0)
        assert st in (4, 7), st
        ws.zero_()
        note(f"stream prefill on the zero-filled workspace, b={b} H={H}")
        m3.scan_prefill(**kw, chunk=64, workspace=ws)
        assert m3.prefill_status(ws) == 0
