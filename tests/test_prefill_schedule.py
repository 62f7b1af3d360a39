"""The persistent prefill's block schedule, modelled on the CPU.

At head dim 256 the prefill runs a persistent grid of G workgroups (as many
as the GPU holds at once). Workgroup w runs on XCD w % 8 and takes, in
zig-zag rounds, the blocks of rows that a one-block-per-workgroup grid
would give that XCD: the XCD's contiguous chunk of the logical block order
(bg-major, heaviest causal block first within each (sequence, KV head) bg),
round r taking local block r * P + k for even r and r * P + P - 1 - k for
odd r (P workgroups on the XCD, k = w // 8); a grid of fewer than eight
workgroups (some XCD would have none) deals the blocks round-robin
instead. This test restates that
integer logic and checks, over the GPU tests' shapes, the full-size
workloads and random sizes, that every block is taken by exactly one
workgroup in exactly one round, that every workgroup's rounds stop at the
first empty one (the kernel's loop ends there), and that the workgroups of
an XCD take only blocks of that XCD's chunk. (Scheduling arithmetic only,
written from the kernel's description; no attention math.)
"""

import random

import pytest

X = 8


def chunk(n, x):
    """(first block, count) of XCD x's chunk of n blocks (the one-block grid's remap)."""
    per, rem = n // X, n % X
    cnt = per + (1 if x < rem else 0)
    base = x * (per + 1) if x < rem else rem * (per + 1) + (x - rem) * per
    return base, cnt


def item(n, G, w, r):
    """The block workgroup w of a grid of G takes in round r, or -1."""
    if G < X:
        # fewer workgroups than XCDs: round-robin over all blocks
        L = r * G + w
        return L if L < n else -1
    x, k = w % X, w // X
    P = G // X + (1 if x < G % X else 0)
    base, cnt = chunk(n, x)
    jl = r * P + ((P - 1 - k) if r & 1 else k)
    return base + jl if jl < cnt else -1


def schedule(n, G):
    taken = {}
    for w in range(G):
        r = 0
        while True:
            L = item(n, G, w, r)
            if L < 0:
                break
            assert L not in taken, f"block {L} taken twice"
            taken[L] = (w, r)
            r += 1
        # the loop ends at the first empty round: no later round has a block
        assert all(item(n, G, w, rr) < 0 for rr in range(r, r + 3))
    return taken


def test_every_xcd_needs_a_workgroup_without_the_fallback():
    """The reason for the round-robin fallback: with the XCD chunks alone, a
    grid of fewer than eight workgroups leaves the chunks of the XCDs
    without a workgroup unprocessed."""
    def item_xcd_only(n, G, w, r):
        x, k = w % X, w // X
        P = G // X + (1 if x < G % X else 0)
        base, cnt = chunk(n, x)
        jl = r * P + ((P - 1 - k) if r & 1 else k)
        return base + jl if jl < cnt else -1
    n, G = 100, 3
    seen = set()
    for w in range(G):
        r = 0
        while item_xcd_only(n, G, w, r) >= 0:
            seen.add(item_xcd_only(n, G, w, r))
            r += 1
    assert len(seen) < n


def blocks(B, Hkv, Sq, G_heads, BM=128):
    return B * Hkv * ((Sq * G_heads + BM - 1) // BM)


SHAPES = [
    # B, Hkv, Sq, heads per KV head: the GPU tests' head-dim-256 shapes and the C4A workload
    (1, 1, 257, 4), (1, 8, 64, 2), (1, 1, 70, 8), (1, 2, 520, 1),
    (4, 8, 2048, 2), (8, 8, 2048, 1), (2, 4, 1536, 3), (1, 8, 8192, 2),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("grid", [256, 255, 97, 8, 1])
def test_every_block_taken_once(shape, grid):
    n = blocks(*shape)
    G = min(n, grid)
    taken = schedule(n, G)
    assert sorted(taken) == list(range(n))
    if G >= X:
        for L, (w, _) in taken.items():
            base, cnt = chunk(n, w % X)
            assert base <= L < base + cnt, "a block left its XCD's chunk"


def test_random_sizes():
    rnd = random.Random(3)
    for _ in range(400):
        n = rnd.randint(1, 6000)
        G = min(n, rnd.choice([1, 3, 8, 64, 200, 255, 256, 512]))
        assert sorted(schedule(n, G)) == list(range(n))


def test_c4a_rounds_are_balanced():
    """C4A (1024 blocks of 128 rows, 34 tiles each except the 16 shortest of
    each KV head) on 256 workgroups: four rounds each, and no workgroup
    takes more than 136 tiles (127.5 on average)."""
    B, Hkv, S, Gh, W = 1, 8, 8192, 2, 1024
    n_rb = S * Gh // 128
    n = B * Hkv * n_rb

    def tiles(L):
        rb = n_rb - 1 - (L % n_rb)
        lo, hi = max(0, 64 * rb - W + 1), 64 * rb + 64
        ts = (lo // 32) * 32
        return (hi - ts + 31) // 32

    taken = schedule(n, 256)
    load = {}
    for L, (w, r) in taken.items():
        load[w] = load.get(w, 0) + tiles(L)
    assert max(r for _, r in taken.values()) == 3
    assert max(load.values()) == 136 and abs(sum(load.values()) / 256 - 127.5) < 1e-9
