"""Host replay of the per-chunk prefill kernel's index arithmetic (CPU only).

The kernel (csrc/m3_fused_kernel.h) divides one chunk's work among its waves
and lanes with integer formulas that are restated here, once per variant and
chunk size, and checked for coverage and bounds:
  - output row tiles: every 16-row tile of the chunk's Q x R rows is taken by
    exactly one (wave, slot), and no wave holds more than its RT register
    tiles;
  - state tiles: every (16-row N tile, 16-column P tile) pair of the state is
    owned by exactly one (wave, slot);
  - angles: the token segments of the phase scan cover the chunk exactly, fit
    the thread's register array, and land inside the cos/sin table's rows;
  - LDS: the layout's regions are ordered, disjoint, as large as the tiles
    stored in them, and fit the 160 KiB of a compute unit.
The grid is a superset of the built variants: N in 16..128, P in 16..128,
R in 1..8, RT in 1, 2, 4, both element sizes, with and without the prologue,
and every power-of-two chunk from 16 to 256 whose rows fit RT tiles per wave
and whose angles fit the angle cap.

The look-back between chunks is replayed as a protocol: every chunk of a
(sequence, head) runs concurrently under a random schedule, publishes its map
(flag 1) when its early poll did not find the predecessor's state, walks back
over windows of at most 64 predecessors exactly as the kernel's wave 0 does,
and publishes its state (flag 2) when done.  Every flag read must lie in
[0, c - 1], every composed map must be published when read, the state read
must be published, the composed chunks must be exactly those after it, and
every chunk must finish.
"""
import itertools
import random

import pytest

LDS_BUDGET = 160 * 1024
ANGLE_CAP = 8192


def fused_threads(N):
    return 1024 if N >= 128 else 512


def round_up(a, b):
    return (a + b - 1) // b * b


def x_stride(P, esz):
    return (16 if P == 16 else P + 16) if esz == 2 else P + 8


def lds_layout(Q, R, N, P, esz, pro):
    """The per-chunk kernel's LDS regions (byte offsets) and what each holds."""
    QRp = round_up(Q * R, 32)
    waves = fused_threads(N) // 64
    scan = 4 * waves + 16 * waves * (N // 8)
    o = {"row": 0}
    o["rw"] = o["row"] + 16 * QRp
    o["W"] = o["rw"] + 4 * QRp
    o["csH"] = o["W"] + 4 * QRp
    o["B"] = o["csH"] + round_up(max(8 * Q * (N // 2 + 1), esz * P * (N + 8)), 16)
    o["X"] = o["B"] + round_up(max(esz * QRp * (N + 8), scan), 16)
    o["misc"] = o["X"] + esz * QRp * x_stride(P, esz)
    o["pb"] = o["misc"] + 64
    o["total"] = o["pb"] + (4 * R * (2 * N + 4) if pro else 0)
    return o


def variants():
    for N, P, R, RT in itertools.product((16, 32, 64, 128), (16, 32, 64, 128), (1, 2, 4, 8), (1, 2, 4)):
        waves = fused_threads(N) // 64
        for Q in (16, 32, 64, 128, 256):
            if Q * R > RT * 16 * waves or Q * (N // 2) > ANGLE_CAP:
                continue
            yield N, P, R, RT, Q


def tile_of(wave, k, MT, waves, RT):
    rev = RT == 1 and MT == waves and wave >= waves // 2
    if rev:
        return MT - 1 - (wave - waves // 2)
    pair = k >> 1
    return MT - 1 - (wave + 2 * waves * pair) if k & 1 else wave + 2 * waves * pair


def test_output_row_tiles_cover_the_chunk_once():
    n = 0
    for N, P, R, RT, Q in variants():
        waves = fused_threads(N) // 64
        MT = round_up(Q * R, 32) // 16
        taken = []
        for w in range(waves):
            nt = (MT + waves - 1 - w) // waves
            assert nt <= RT, (N, P, R, RT, Q, w)
            taken += [tile_of(w, k, MT, waves, RT) for k in range(nt)]
        assert sorted(taken) == list(range(MT)), (N, P, R, RT, Q)
        n += 1
    assert n > 300


def test_state_tiles_cover_the_state_once():
    for N, P in itertools.product((16, 32, 64, 128), (16, 32, 64, 128)):
        waves = fused_threads(N) // 64
        TPt, TNt = P // 16, N // 16
        NGRP = min(TNt, waves)
        NPW, WPN = TNt // NGRP, waves // NGRP
        PTW = (TPt + WPN - 1) // WPN
        owned = []
        for w in range(waves):
            nslot, pslot = w % NGRP, w // NGRP
            for i in range(NPW):
                for j in range(PTW):
                    if pslot + WPN * j < TPt:
                        owned.append((nslot + NGRP * i, pslot + WPN * j))
        assert sorted(owned) == sorted(itertools.product(range(TNt), range(TPt))), (N, P)


def test_angle_segments_cover_the_chunk_and_fit_their_arrays():
    for N, P, R, RT, Q in variants():
        threads = fused_threads(N)
        waves = threads // 64
        NG = (N // 2) // 4
        CSS = N // 2 + 1
        qmax_t = RT * 16 * waves // R
        al0 = max(qmax_t // (threads // NG), 1)
        kAL = min(al0, 4)
        NSEG = min(threads // NG, Q)
        ALEN = Q // NSEG
        assert NSEG * ALEN == Q and ALEN <= kAL, (N, P, R, RT, Q)
        toks = sorted(sg * ALEN + j for sg in range(NSEG) for j in range(ALEN))
        assert toks == list(range(Q))
        # table entries written: row = token, column = group slot; inside Q rows of CSS
        last = ((NSEG - 1) * ALEN + ALEN - 1) * CSS + (NG - 1) + 3 * NG
        assert last < Q * CSS


@pytest.mark.parametrize("esz", [2, 4])
@pytest.mark.parametrize("pro", [0, 1])
def test_lds_regions_are_disjoint_and_hold_their_tiles(esz, pro):
    fits = 0
    for N, P, R, RT, Q in variants():
        o = lds_layout(Q, R, N, P, esz, pro)
        QRp = round_up(Q * R, 32)
        order = ["row", "rw", "W", "csH", "B", "X", "misc", "pb", "total"]
        assert all(o[a] <= o[b] for a, b in zip(order, order[1:]))
        assert o["rw"] - o["row"] >= 16 * QRp and o["W"] - o["rw"] >= 4 * QRp and o["csH"] - o["W"] >= 4 * QRp
        # cos/sin of Phi for Q tokens, then S_in^T [P][N + 8] in the same bytes
        assert o["B"] - o["csH"] >= max(8 * Q * (N // 2 + 1), esz * P * (N + 8))
        assert o["X"] - o["B"] >= esz * QRp * (N + 8)
        assert o["misc"] - o["X"] >= esz * QRp * x_stride(P, esz)
        assert o["pb"] - o["misc"] >= 4 * 16   # 8 scalars, then up to 8 B_prev norm factors
        if pro:
            assert o["total"] - o["pb"] >= 4 * (R * N + R * (N + 4))
        # every 16-byte-aligned region start (the kernel reads them as float4 / 16-byte rows)
        assert all(o[k] % 16 == 0 for k in ("rw", "csH", "B", "X", "misc", "pb"))
        fits += o["total"] <= LDS_BUDGET
    assert fits > 100


def _chunk(c, nc, flags, log, use_maps):
    """One chunk of the look-back protocol as a generator; yields when it waits.
    With maps, the first poll is issued with the chunk's loads and decides
    whether to publish a map; without, it is issued once the chunk's own work
    is done and no chunk publishes a map."""
    W0 = min(c, 64)
    if use_maps:
        fpoll = [flags[c - 1 - lane] for lane in range(W0)]
    yield
    if not use_maps:
        fpoll = [flags[c - 1 - lane] for lane in range(W0)]
    elif c > 0 and fpoll[0] != 2:
        flags[c] = 1                                   # map published
    yield
    composed = []
    if c > 0:
        hi, first = c - 1, True
        while True:
            W = min(hi + 1, 64)
            while True:
                f = fpoll if first else [flags[hi - lane] for lane in range(W)]
                for lane in range(W):
                    assert 0 <= hi - lane <= c - 1
                first = False
                k2 = next((k for k in range(W) if f[k] == 2), W)
                k0 = next((k for k in range(W) if f[k] == 0), 64)
                if k0 > k2 or (k2 == W and k0 >= W):
                    nmap, state = k2, int(k2 < W)
                    break
                if k0 > 0:
                    nmap, state = k0, 0
                    break
                yield
            for m in range(nmap):
                j = hi - m
                assert 0 <= j <= c - 1 and f[m] == 1, (c, hi, m)   # a published map
                composed.append(j)
            if state:
                s = hi - nmap
                assert 0 <= s <= c - 1 and f[nmap] == 2
                assert sorted(composed) == list(range(s + 1, c)), (c, s, composed)
                break
            hi -= nmap
            assert hi >= 0, (c, composed)
    if c + 1 < nc:
        flags[c] = 2                                   # state published
    log.append(("done", c))


@pytest.mark.parametrize("nc", [1, 2, 3, 17, 64, 65, 66, 150, 300])
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("use_maps", [True, False])
def test_look_back_reads_in_range_and_composes_each_chunk_once(nc, seed, use_maps):
    rng = random.Random(seed * 1000 + nc + 7 * use_maps)
    flags = [0] * nc
    log = []
    # chunks start in ticket order, each after a random number of scheduler steps
    pending = list(range(nc))
    live = {}
    steps = 0
    while pending or live:
        if pending and (not live or rng.random() < 0.3):
            c = pending.pop(0)
            live[c] = _chunk(c, nc, flags, log, use_maps)
        c = rng.choice(list(live))
        try:
            next(live[c])
        except StopIteration:
            del live[c]
        steps += 1
        assert steps < 200 * nc + 1000, "the look-back did not finish"
    assert sorted(e[1] for e in log if e[0] == "done") == list(range(nc))
