"""GPU test of m3_scan_prefill_noalloc, called through the C ABI: its outputs
match m3_scan_prefill's (the entry point with a caller workspace) on the same
inputs, within the parity tolerance, on two calls in a row -- the second with
a smaller input, so the buffer holds the first call's contents when it
starts -- and both match the float64 oracle."""
import ctypes

import pytest
import torch

import oracle
import state_space_sequence_02_amd as m3
from state_space_sequence_02_amd import inputs

from _parity import TOL, check_blocks, dev_inputs, note, oracle_inputs, to64

pytestmark = pytest.mark.gpu

KEYS = ("x", "B", "C", "dt", "A", "lam", "theta")


def _noalloc(d, carry, chunk):
    lib = m3.load_library()
    x = d["x"]
    b, L, H, R, P = x.shape
    N = d["B"].shape[-1]
    code = m3.M3_BF16 if x.dtype == torch.bfloat16 else m3.M3_FP32
    shape = m3.make_shape(b, L, H, P, N, R, chunk, code)
    y = torch.empty_like(x)
    h = torch.empty((b, H, N, P), dtype=torch.float32, device=x.device)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.m3_scan_prefill_noalloc(
        ctypes.byref(shape), ptr(x), ptr(d["B"]), ptr(d["C"]), ptr(d["dt"]), ptr(d["A"]), ptr(d["lam"]),
        ptr(d["theta"]), ptr(carry.get("h0")), ptr(carry.get("B_prev")), ptr(carry.get("x_prev")),
        ptr(y), ptr(h), torch.cuda.current_stream().cuda_stream)
    assert st == 0, m3.STATUS.get(st, st)
    return y, h


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m3.load_library()


def test_noalloc_matches_workspace_entry_point():
    cases = [(inputs.workload("mimo", batch=2, seqlen=1000, nheads=4), 64, 201),
             (inputs.workload("mimo", batch=1, seqlen=150, nheads=2), 32, 202)]   # second call: smaller
    for w, chunk, seed in cases:
        shape = m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, chunk, m3.M3_BF16)
        assert m3.prefill_workspace_bytes(shape) <= m3.load_library().m3_prefill_workspace_bytes(
            ctypes.byref(shape)) <= 64 << 20
        d = inputs.make_prefill_inputs(w, seed=seed)
        c = inputs.random_carry(w, seed=seed + 1)
        dg, cg = dev_inputs(d), dev_inputs(c)
        note(f"no-alloc prefill b={w.batch} L={w.seqlen} H={w.nheads} chunk={chunk}")
        y0, h0 = _noalloc(dg, cg, chunk)
        torch.cuda.synchronize()
        note(f"workspace prefill b={w.batch} L={w.seqlen} H={w.nheads} chunk={chunk}")
        y1, h1 = m3.scan_prefill(**{k: dg[k] for k in KEYS}, **cg, chunk=chunk)
        torch.cuda.synchronize()
        check_blocks(to64(y0), to64(y1), TOL["bf16"], (1, 3, 4), "no-alloc y vs workspace y", elem_axes=(3, 4))
        check_blocks(to64(h0), to64(h1), TOL["bf16"], (2, 3), "no-alloc h vs workspace h")
        yr, hr = oracle.scan(**oracle_inputs({**d, **c}))
        check_blocks(to64(y0), yr, TOL["bf16"], (1, 3, 4), "no-alloc y", elem_axes=(3, 4))
        check_blocks(to64(h0), hr, TOL["bf16"], (2, 3), "no-alloc h")


def test_noalloc_graph_replay():
    """The entry point is meant for code under graph capture: a captured call
    is right on every replay, with eager no-alloc calls (sharing the same
    device array) between the replays."""
    w = inputs.workload("mimo", batch=1, seqlen=300, nheads=2)
    d = inputs.make_prefill_inputs(w, seed=203)
    c = inputs.random_carry(w, seed=204)
    dg, cg = dev_inputs(d), dev_inputs(c)
    yr, hr = oracle.scan(**oracle_inputs({**d, **c}))
    note("no-alloc prefill before capture")
    _noalloc(dg, cg, 32)                       # eager: the device array's address is looked up here
    torch.cuda.synchronize()
    out = {}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    note("no-alloc prefill graph capture")
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            out["y"], out["h"] = _noalloc(dg, cg, 32)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out["y"].zero_()
        out["h"].zero_()
        torch.cuda.synchronize()
        note(f"no-alloc graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        check_blocks(to64(out["y"]), yr, TOL["bf16"], (1, 3, 4), f"y replay {rep}", elem_axes=(3, 4))
        check_blocks(to64(out["h"]), hr, TOL["bf16"], (2, 3), f"h replay {rep}")
        ye, he = _noalloc(dg, cg, 32)          # eager, the same device array
        torch.cuda.synchronize()
        check_blocks(to64(ye), yr, TOL["bf16"], (1, 3, 4), f"y eager after replay {rep}", elem_axes=(3, 4))
        check_blocks(to64(he), hr, TOL["bf16"], (2, 3), f"h eager after replay {rep}")
