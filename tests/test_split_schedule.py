"""The split-KV kernel's integer work split, modelled on the CPU.

The persistent split kernel gives every workgroup a contiguous range of the
global tile order (sequence, block of rows, tile) and derives everything
else from integers: the tile a range starts at (found by a lane-parallel
prefix scan over the sequences' tile counts), the tile iterator that walks
the range, the partial-output slot each range writes for each block of rows,
and the slots marked empty. This test restates that logic in Python and
checks, over the decode/verify shapes of the GPU tests and random ones:

* every tile of every (sequence, KV head, block of rows) is visited by
  exactly one workgroup, and the tiles of a block of rows cover its visible
  keys with no gap and stay inside the sequence;
* every partial slot the combine kernel reads (ceil(len / kv_chunk) + 1 per
  row, none for an empty sequence) is written exactly once, as a partial or
  as empty;
* the values the kernel takes from a lane-parallel scan (the starting
  sequence and its tile offset) are the same whichever lane computes them
  (they are read with readlane from one lane, so they are wave-uniform by
  construction; the model checks that every lane would agree).

It is a check of the host-visible scheduling arithmetic (no attention math),
written from the kernel's description: a range holds at least one chunk,
tiles never straddle a chunk, a range merges its chunks and writes one
partial per block of rows, in slot r - r0.
"""

import math
import random

import pytest

BN = 32


def row_span(len_, rb, *, Sq, G, BM, causal, window, chunk):
    """(c_lo, k0, c_hi, k1, nt) of one block of rows, as the kernel computes it."""
    tpc = (chunk + BN - 1) // BN
    rows = Sq * G
    r_lo, r_hi = rb * BM, min(rb * BM + BM, rows)
    shift = len_ - Sq
    lo, hi = 0, len_
    if causal:
        hi = min(hi, (r_hi - 1) // G + shift + 1)
        if window > 0:
            lo = max(lo, r_lo // G + shift - window + 1)
    if hi <= lo:
        return (0, 0, 0, 0, 0), (lo, hi)
    c_lo, c_hi = lo // chunk, (hi - 1) // chunk
    k0 = (lo - c_lo * chunk) // BN
    k1 = (hi - 1 - c_hi * chunk) // BN
    nt = k1 - k0 + 1 if c_lo == c_hi else (tpc - k0) + (c_hi - c_lo - 1) * tpc + k1 + 1
    return (c_lo, k0, c_hi, k1, nt), (lo, hi)


def simulate(B, Sq, Hq, Hkv, lens, chunk, W, *, causal=True, window=0, BM=32):
    G = Hq // Hkv
    n_rb = (Sq * G + BM - 1) // BM
    tpc = (chunk + BN - 1) // BN
    span = lambda L, rb: row_span(L, rb, Sq=Sq, G=G, BM=BM, causal=causal, window=window, chunk=chunk)
    seq_tiles = [sum(span(L, rb)[0][4] for rb in range(n_rb)) for L in lens]
    T = sum(seq_tiles)
    sets = W // Hkv
    per = max(-(-T // sets), tpc)
    visits = {}        # (b, g, rb, i) -> count
    slots = {}         # (b, g, rb, slot) -> count

    def write(b, g, rb, s):
        slots[(b, g, rb, s)] = slots.get((b, g, rb, s), 0) + 1

    # blocks of rows with no visible key: every slot of their rows is empty
    for w in range(W):
        for bb in range(w, B, W):
            L = lens[bb]
            nch = -(-L // chunk)
            if nch == 0:
                continue
            for rb in range(n_rb):
                if span(L, rb)[0][4] > 0:
                    continue
                for gg in range(Hkv):
                    for s in range(nch + 1):
                        write(bb, gg, rb, s)

    for w in range(W):
        g = w % Hkv
        x0 = (w // Hkv) * per
        if x0 >= T:
            continue
        x1 = min(x0 + per, T)
        # locate tile x0: a lane-parallel inclusive scan over 64 sequences at
        # a time; the first lane whose running total passes x0 names the
        # sequence (every lane computes the same ballot, so the same answer)
        found = None
        base = 0
        for b0 in range(0, B, 64):
            incl, run = [], base
            for lane in range(64):
                bb = b0 + lane
                run += seq_tiles[bb] if bb < B else 0
                incl.append(run)
            hits = [lane for lane in range(64) if b0 + lane < B and incl[lane] > x0]
            if hits and found is None:
                L = hits[0]
                bx = b0 + L
                sx = incl[L] - seq_tiles[bx]
                # what each lane would read back with readlane(L)
                assert all(incl[L] - seq_tiles[bx] == sx for _ in range(64))
                found = (bx, sx)
            base = incl[63]
        assert found is not None
        b, sx = found
        o = x0 - sx
        rb = 0
        while True:
            sp = span(lens[b], rb)[0]
            if o < sp[4]:
                break
            o -= sp[4]
            rb += 1
        c_lo, k0, c_hi, k1, nt = sp
        i = o
        if i < tpc - k0:
            c, k = c_lo, k0 + i
        else:
            i2 = i - (tpc - k0)
            c, k = c_lo + 1 + i2 // tpc, i2 % tpc
        slot = x0 // per - (x0 - i) // per
        for it in range(x1 - x0):
            L = lens[b]
            tb = c * chunk + k * BN
            ke = min((c + 1) * chunk, L)
            assert tb < ke, (b, rb, c, k)
            visits[(b, g, rb, i)] = visits.get((b, g, rb, i), 0) + 1
            visits.setdefault(("keys", b, g, rb), []).append((tb, min(tb + BN, ke)))
            range_end = it + 1 == x1 - x0
            rows_end = i == nt - 1
            if range_end or rows_end:
                write(b, g, rb, slot)
                if rows_end:
                    for s in range(slot + 1, -(-L // chunk) + 1):
                        write(b, g, rb, s)
            if not range_end:
                i += 1
                if i < nt:
                    k += 1
                    if k == tpc:
                        k, c = 0, c + 1
                else:
                    while True:
                        rb += 1
                        if rb == n_rb:
                            rb = 0
                            b += 1
                            assert b < B
                        sp = span(lens[b], rb)[0]
                        if sp[4] > 0:
                            c_lo, k0, c_hi, k1, nt = sp
                            i, c, k = 0, c_lo, k0
                            break
                    slot = 0
    # coverage: tiles and keys
    for b in range(B):
        L = lens[b]
        nch = -(-L // chunk)
        for g in range(Hkv):
            for rb in range(n_rb):
                (c_lo, k0, c_hi, k1, nt), (lo, hi) = span(L, rb)
                for i in range(nt):
                    assert visits.get((b, g, rb, i)) == 1, ("tile", b, g, rb, i)
                if nt:
                    segs = sorted(visits[("keys", b, g, rb)])
                    assert segs[0][0] <= lo and segs[-1][1] >= hi and segs[-1][1] <= L
                    for (a0, a1), (b0_, _) in zip(segs, segs[1:]):
                        assert a1 == b0_, ("gap", b, g, rb)
                want = set(range(nch + 1)) if nch else set()
                got = {s for (bb, gg, r, s) in slots if (bb, gg, r) == (b, g, rb)}
                assert got == want, ("slots", b, g, rb, sorted(got), nch)
                assert all(slots[(b, g, rb, s)] == 1 for s in got)
    return T, per


GRID_SHAPES = [
    # B, Sq, Hq, Hkv, max_len, chunk, BM (rows per block), W (grid)
    (3, 1, 8, 8, 1024, 128, 32, 1024),
    (2, 8, 64, 8, 1024, 256, 64, 1024),
    (2, 8, 16, 8, 768, 96, 32, 512),
    (2, 2, 4, 1, 256, 64, 32, 1024),
    (64, 1, 16, 4, 4096, 32, 32, 1024),
    (40, 2, 8, 4, 4096, 32, 32, 1024),
    (4, 8, 64, 8, 32768, 1024, 64, 1024),     # the verify workload's shape
]


@pytest.mark.parametrize("shape", GRID_SHAPES)
def test_split_schedule_covers_every_tile_and_slot(shape):
    B, Sq, Hq, Hkv, max_len, chunk, BM, W = shape
    rng = random.Random(hash(shape) % 1000)
    lens = [rng.randint(0, max_len) for _ in range(B)]
    lens[0] = max_len
    simulate(B, Sq, Hq, Hkv, lens, chunk, W, BM=BM)


def test_split_schedule_windows_and_random_shapes():
    rng = random.Random(7)
    for _ in range(150):
        Hkv = rng.choice([1, 2, 4, 8])
        G = rng.choice([1, 2, 4, 8])
        B = rng.randint(1, 70)
        Sq = rng.randint(1, 9)
        chunk = 32 * rng.randint(1, 8)
        BM = rng.choice([32, 64, 128])
        max_len = rng.randint(1, 3000)
        lens = [rng.randint(0, max_len) for _ in range(B)]
        window = rng.choice([0, 0, rng.randint(1, 300)])
        W = Hkv * rng.randint(1, 300)
        simulate(B, Sq, Hkv * G, Hkv, lens, chunk, W, window=window, BM=BM)
