"""GPU parity over every compiled shape: each (dtype, N, P, R) the library
instantiates, for the chunked prefill (at the library's default chunk and at
the largest chunk the shape allows, which puts two or four 16-row output tiles
on a wave) and for the decode step (fp32 state, and bf16 state with bf16
inputs), against the float64 oracle.  Sizes are small: a prefill spans two
whole chunks and a ragged third, with an incoming state and previous write.
"""
import math

import pytest
import torch

import oracle
import state_space_sequence_02_amd as m3
from state_space_sequence_02_amd import inputs

from _parity import TOL, check_blocks, dev_inputs, gate_scale, note, oracle_inputs, to64

pytestmark = pytest.mark.gpu

DTYPES = ("bf16", "fp32")
STATES = (16, 32, 64, 128, 256)
HEADS = (16, 32, 64, 128)
RANKS = (1, 2, 4, 8)
GRID = [(dt, n, p, r) for dt in DTYPES for n in STATES for p in HEADS for r in RANKS]
KEYS = ("x", "B", "C", "dt", "A", "lam", "theta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m3.load_library()


def _code(dtype):
    return m3.M3_BF16 if dtype == "bf16" else m3.M3_FP32


# shapes whose chunk tiles do not fit a compute unit's LDS even at 16 tokens
# per chunk: the prefill rejects them (the decode takes them)
NO_PREFILL = {("fp32", 128, 128, 8)}
# N = 256 is decode-only: its prefill kernels spilled heavily to scratch and one
# of them (bf16 P=64 R=4) made a GPU memory fault whose cause was not found, so
# the path was taken out of the library
# N256_REFUSED: the N = 256 prefill is not built (heavy scratch spills; one
# unexplained GPU memory fault); every prefill entry point refuses it on the
# host with M3_ERR_SHAPE before anything is launched, which the grid checks
# The library never launches a prefill kernel variant the build's compiler
# report gives scratch memory, nor a fused prologue variant with two or more
# output tiles per wave or with fp32 inputs at N = 128: all the GPU memory
# faults met in this kernel's development (one of them a prologue variant with
# two tiles per wave, bf16 N=64 P=64 R=2, another an fp32 N=128 P=32 R=1
# prologue variant) and the one wrong result came from spilling variants, with
# causes not established.  Where the plain prefill's variant is refused the
# shape is refused (M3_ERR_SHAPE, nothing launched; a refused case checks that
# the call raises); where only the fused prologue's is, the prologue entry
# point stages the prologue before the plain prefill, and the grid runs it.


def _taken(dtype, N, P, R, chunk, variant):
    """The chunk the entry point takes: its default, or the largest it takes."""
    code = _code(dtype)
    if chunk == "default":
        return m3.prefill_chunk_used(m3.make_shape(1, 1, 2, P, N, R, 0, code), variant)
    for c in (256, 128, 64, 32, 16):
        if m3.prefill_chunk_used(m3.make_shape(1, 1, 2, P, N, R, c, code), variant) == c:
            return c
    return 0


def _refused(call, what):
    note(f"{what}: refused on the host")
    with pytest.raises(m3.M3Error, match="M3_ERR_SHAPE"):
        call()


@pytest.mark.parametrize("chunk", ["default", "max"])
@pytest.mark.parametrize("dtype,N,P,R", GRID, ids=lambda v: str(v))
def test_prefill_grid(dtype, N, P, R, chunk):
    q = _taken(dtype, N, P, R, chunk, "plain")
    if q == 0:
        # refused on the host, before any launch (N = 256: N256_REFUSED)
        assert (dtype, N, P, R) in NO_PREFILL or dtype == "fp32" or N >= 128
        w = inputs.workload("mimo", batch=1, seqlen=20, nheads=2, headdim=P, dstate=N, rank=R, dtype=dtype)
        dg = dev_inputs(inputs.make_prefill_inputs(w, seed=1))
        _refused(lambda: m3.scan_prefill(**{k: dg[k] for k in KEYS}, chunk=0),
                 f"prefill grid {dtype} N={N} P={P} R={R}")
        return
    L = 2 * q + q // 2 + 3
    w = inputs.workload("mimo", batch=1, seqlen=L, nheads=2, headdim=P, dstate=N, rank=R,
                        chunk=q, dtype=dtype)
    seed = 1000 + N + P + R
    d = inputs.make_prefill_inputs(w, seed=seed)
    c = inputs.random_carry(w, seed=seed + 1)
    dg, cg = dev_inputs(d), dev_inputs(c)
    note(f"prefill grid {dtype} N={N} P={P} R={R} chunk={q} L={L}")
    y, h = m3.scan_prefill(**{k: dg[k] for k in KEYS}, **cg, chunk=q)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(**oracle_inputs({**d, **c}))
    check_blocks(to64(y), yr, TOL[dtype], (1, 3, 4), "y", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL[dtype], (2, 3), "h_out")


DECODE = [(dt, st, n, p, r) for dt, st in (("bf16", "fp32"), ("fp32", "fp32"), ("bf16", "bf16"))
          for n in STATES for p in HEADS for r in RANKS]


@pytest.mark.parametrize("dtype,state,N,P,R", DECODE, ids=lambda v: str(v))
def test_decode_grid(dtype, state, N, P, R):
    w = inputs.workload("decode", batch=2, nheads=3, headdim=P, dstate=N, rank=R, dtype=dtype)
    steps, seed = 3, 2000 + N + P + R
    d = inputs.make_decode_inputs(w, seed=seed, steps=steps)
    dg = dev_inputs(d)
    h0 = torch.randn((w.batch, w.nheads, N, P), generator=torch.Generator().manual_seed(seed + 1)) * 0.5
    h = (h0.to(torch.bfloat16) if state == "bf16" else h0).to("cuda").contiguous()
    note(f"decode grid {dtype} inputs, {state} state, N={N} P={P} R={R}")
    ys = []
    for s in range(steps):
        kw = dict(B_prev=dg["B"][s - 1], x_prev=dg["x"][s - 1]) if s else {}
        ys.append(m3.decode_step(h, dg["x"][s], dg["B"][s], dg["C"][s], dg["dt"][s], dg["A"],
                                 dg["lam"][s], dg["theta"][s], **kw))
    torch.cuda.synchronize()
    if state == "bf16":
        yr, hr = oracle.decode_steps_bf16_state(h0.to(torch.bfloat16).double().numpy(), d["x"], d["B"],
                                                d["C"], d["dt"], d["A"], d["lam"], d["theta"])
    else:
        yr, hr = oracle.decode_steps(h0, d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"])
    tol = TOL[dtype]
    check_blocks(to64(torch.stack(ys)), yr, tol, (3, 4), "decode y")
    check_blocks(to64(h), hr, tol, (2, 3), "decode h")


def _grid_case(dtype, N, P, R, chunk, seed, variant):
    """The grid's prefill case: (workload, q, inputs, carry), q = 0 when the
    entry point refuses the shape (the inputs are then a short sequence)."""
    q = _taken(dtype, N, P, R, chunk, variant)
    if N == 256:
        assert q == 0   # N256_REFUSED: the call must raise before any launch
    L = 2 * q + q // 2 + 3 if q else 20
    w = inputs.workload("mimo", batch=1, seqlen=L, nheads=2, headdim=P, dstate=N, rank=R, chunk=q, dtype=dtype)
    d = inputs.make_prefill_inputs(w, seed=seed)
    c = inputs.random_carry(w, seed=seed + 1)
    return w, q, d, c


@pytest.mark.parametrize("chunk", ["default", "max"])
@pytest.mark.parametrize("dtype,N,P,R", GRID, ids=lambda v: str(v))
def test_gated_grid(dtype, N, P, R, chunk):
    w, q, d, c = _grid_case(dtype, N, P, R, chunk, 3000 + N + P + R, "gated")
    g = torch.Generator().manual_seed(3100 + N + P + R)
    z = torch.randn((w.batch, w.seqlen, w.nheads, P), generator=g).to(w.torch_dtype)
    wy = torch.randn((w.nheads, R, P), generator=g)
    wz = torch.rand((w.nheads, R, P), generator=g) + 0.5
    dg, cg = dev_inputs(d), dev_inputs(c)
    if q == 0:
        _refused(lambda: m3.scan_prefill_gated(**{k: dg[k] for k in KEYS}, z=z.cuda(), chunk=0),
                 f"gated grid {dtype} N={N} P={P} R={R}")
        return
    note(f"gated grid {dtype} N={N} P={P} R={R} chunk={q}")
    out, h = m3.scan_prefill_gated(**{k: dg[k] for k in KEYS}, **cg, z=z.cuda(), w_y=wy.cuda(), w_z=wz.cuda(),
                                   chunk=q)
    torch.cuda.synchronize()
    zn, wyn, wzn = z.double().numpy(), wy.double().numpy(), wz.double().numpy()
    yref, href = oracle.scan(**oracle_inputs({**d, **c}))
    ref = oracle.gated_readout(yref, zn, wyn, wzn)
    check_blocks(to64(out), ref, TOL[dtype], (1, 3), "gated out", elem_axes=(3,),
                 elem_scale=gate_scale(yref, zn, wyn, wzn, block_axes=(1, 3, 4)))
    check_blocks(to64(h), href, TOL[dtype], (2, 3), "h_out")


@pytest.mark.parametrize("chunk", ["default", "max"])
@pytest.mark.parametrize("dtype,N,P,R", GRID, ids=lambda v: str(v))
def test_prologue_grid(dtype, N, P, R, chunk):
    w, q, d, c = _grid_case(dtype, N, P, R, chunk, 4000 + N + P + R, "prologue")
    g = torch.Generator().manual_seed(4100 + N + P + R)
    th = (torch.rand((w.batch, w.seqlen, w.nheads, N // 2), generator=g) * 2 - 1) * math.pi
    bb = torch.randn((w.nheads, R, N), generator=g) * 0.5
    bc = torch.randn((w.nheads, R, N), generator=g) * 0.5
    dg, cg = dev_inputs(d), dev_inputs(c)
    if q == 0:
        _refused(lambda: m3.scan_prefill_prologue(dg["x"], dg["B"], dg["C"], dg["dt"], dg["A"], dg["lam"],
                                                  th.cuda(), chunk=0), f"prologue grid {dtype} N={N} P={P} R={R}")
        return
    note(f"prologue grid {dtype} N={N} P={P} R={R} chunk={q}")
    y, h = m3.scan_prefill_prologue(dg["x"], dg["B"], dg["C"], dg["dt"], dg["A"], dg["lam"], th.cuda(), **cg,
                                    chunk=q, eps=1e-5, bias_B=bb.cuda(), bias_C=bc.cuda())
    torch.cuda.synchronize()
    n = lambda t: t.double().numpy()
    yr, hr = oracle.scan_prologue(n(d["x"]), n(d["B"]), n(d["C"]), n(d["dt"]), n(d["A"]), n(d["lam"]), n(th),
                                  h0=n(c["h0"]), B_prev=n(c["B_prev"]), x_prev=n(c["x_prev"]),
                                  eps=1e-5, bias_B=n(bb), bias_C=n(bc))
    check_blocks(to64(y), yr, TOL[dtype], (1, 3, 4), "prologue y", elem_axes=(3, 4))
    check_blocks(to64(h), hr, TOL[dtype], (2, 3), "prologue h_out")
