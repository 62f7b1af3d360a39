"""Prefill parity: the HIP kernel (through the C ABI) against the fp64 oracle,
element by element on small shapes that span several tiles with ragged tails,
and on sampled rows of the full-size workloads."""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
import workloads
from tests.gpu_util import DEV, assert_parity, to_np

pytestmark = pytest.mark.gpu

GRID = [
    # B, Sq, Skv, Hq, Hkv, D, causal, window
    (1, 128, 128, 2, 1, 64, 1, 0),
    (1, 1, 1, 4, 4, 64, 1, 0),
    (2, 6, 6, 8, 2, 128, 1, 0),
    (1, 16, 16, 4, 1, 128, 0, 0),
    (1, 48, 48, 8, 8, 64, 1, 0),
    (2, 130, 130, 8, 2, 128, 1, 0),
    (1, 257, 257, 4, 1, 256, 1, 0),
    (1, 257, 257, 4, 2, 512, 1, 0),
    (1, 100, 300, 8, 1, 128, 1, 0),
    (1, 300, 100, 4, 2, 64, 1, 0),
    (1, 200, 200, 4, 2, 128, 1, 1),
    (1, 200, 200, 4, 2, 128, 1, 63),
    (1, 200, 200, 4, 2, 128, 1, 64),
    (1, 200, 200, 4, 2, 128, 1, 65),
    (1, 333, 333, 6, 3, 64, 1, 100),
    (1, 77, 77, 24, 8, 128, 1, 0),
    (1, 64, 64, 16, 2, 256, 1, 31),
    (1, 300, 300, 4, 1, 512, 1, 0),
    (1, 70, 200, 8, 1, 256, 0, 0),
    (1, 129, 129, 8, 1, 64, 1, 0),
    (1, 520, 520, 2, 2, 256, 1, 200),
    (1, 96, 160, 4, 2, 512, 1, 33),
    # head dim 128 without modifiers runs two wave groups in ping-pong over a
    # ring of three tile buffers: tile counts of every residue mod 3, long
    # windows, non-causal ragged keys, many query heads per KV head
    (1, 700, 700, 8, 2, 128, 1, 300),
    (1, 300, 333, 2, 2, 128, 0, 0),
    (1, 65, 65, 16, 1, 128, 1, 0),
]


def _run(q, k, v, causal, window, scale):
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=bool(causal), window=window, scale=scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", GRID, ids=lambda c: "B{}_Sq{}_Skv{}_H{}x{}_D{}_c{}_w{}".format(*c))
def test_prefill_grid(case):
    B, Sq, Skv, Hq, Hkv, D, causal, window = case
    print(f"case {case}", flush=True)
    q, k, v = workloads.random_inputs(B, Sq, Skv, Hq, Hkv, D, seed=hash(case) % 10007)
    scale = 1.0 / np.sqrt(D)
    o, lse = _run(q, k, v, causal, window, scale)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=bool(causal), window=window, scale=scale)
    assert_parity(o, lse, o_ref, lse_ref, f"prefill {case}")


def test_prefill_c1_exact_config():
    s = workloads.C1
    q, k, v = workloads.prefill_inputs(s)
    o, lse = _run(q, k, v, True, 0, s.scale)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=True, scale=s.scale)
    assert_parity(o, lse, o_ref, lse_ref, "prefill C1")
    # causal row 0 sees only key 0: O equals V[0] (to bf16 rounding)
    np.testing.assert_array_equal(to_np(o)[0, 0, 0], to_np(v)[0, 0, 0])


def test_prefill_empty_kv_and_rows():
    q, k, v = workloads.random_inputs(1, 5, 1, 4, 2, 128, seed=3)
    k0 = k[:, :0].contiguous()
    o, lse = fa.prefill(q.to(DEV), k0.to(DEV), k0.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # Sq = 0 and B = 0 are no-ops
    qe = q[:, :0].contiguous().to(DEV)
    o, lse = fa.prefill(qe, k.to(DEV), v.to(DEV), causal=True)
    assert o.numel() == 0


# Scores that grow along the keys: a component shared by every query and by
# the keys past `start`, growing with the key index, moves the row max by
# many powers of two from tile to tile (every lazy-rescale path: the
# reference max moves on most tiles after `start`, and a tile whose weights
# pass the bound after being exponentiated against the old reference is
# exponentiated again), and with `spike` a single late key dominates.
GROW = [
    # B, S, Hq, Hkv, D, causal, start, slope, spike
    (1, 600, 8, 2, 128, 1, 200, 0.02, 0),
    (1, 600, 8, 2, 128, 0, 300, 0.05, 0),
    (1, 600, 8, 2, 128, 1, 0, 0.0, 451),
    (1, 400, 4, 2, 64, 1, 100, 0.03, 0),
    (1, 400, 4, 2, 256, 1, 100, 0.03, 333),
    (1, 300, 4, 2, 512, 1, 50, 0.03, 0),
]


@pytest.mark.parametrize("case", GROW, ids=lambda c: "S{1}_H{2}x{3}_D{4}_c{5}_start{6}_sl{7}_spike{8}".format(*c))
def test_prefill_growing_scores(case):
    B, S, Hq, Hkv, D, causal, start, slope, spike = case
    print(f"case {case}", flush=True)
    q, k, v = workloads.random_inputs(B, S, S, Hq, Hkv, D, seed=17 + D + S)
    gen = torch.Generator("cpu").manual_seed(99)
    u = torch.randn(D, generator=gen) / np.sqrt(D)
    qf, kf = q.float(), k.float()
    qf = qf + 2.0 * u
    ramp = torch.clamp(torch.arange(S, dtype=torch.float32) - start, min=0) * slope
    kf = kf + (ramp[None, :, None, None] * np.sqrt(D)) * u
    if spike:
        kf[:, spike] = kf[:, spike] + 6.0 * np.sqrt(D) * u
    q, k = qf.to(torch.bfloat16), kf.to(torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    o, lse = _run(q, k, v, causal, 0, scale)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=bool(causal), scale=scale)
    # the shared component spans many powers of two of the softmax weights
    assert float(np.nanmax(lse_ref) - np.nanmin(lse_ref)) > 10.0
    assert_parity(o, lse, o_ref, lse_ref, f"prefill growing scores {case}")


def test_prefill_deterministic():
    q, k, v = workloads.random_inputs(2, 300, 300, 8, 2, 128, seed=5)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fa.prefill(q, k, v, causal=True)
    o2, l2 = fa.prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _sampled(shape, q, k, v, rows, heads):
    o, lse = _run(q, k, v, shape.causal, shape.window, shape.scale)
    o = to_np(o)
    lse = to_np(lse)
    for b in range(shape.B):
        o_ref, lse_ref = oracle.attention_ref(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=shape.causal,
                                              window=shape.window, scale=shape.scale,
                                              rows=rows, heads=heads)
        og = o[b:b + 1][:, rows][:, :, heads]
        orf = o_ref[:, rows][:, :, heads]
        lg = lse[b:b + 1][:, heads][:, :, rows]
        lrf = lse_ref[:, heads][:, :, rows]
        assert_parity(og, lg, orf, lrf, f"{shape.name} b{b} sampled")


def _rows(S):
    base = [0, 1, 31, 32, 63, 64, 65, 127, 128, 1000, S // 2 - 1, S // 2, S - 129, S - 2, S - 1]
    gen = np.random.default_rng(0)
    return np.unique(np.array(base + list(gen.integers(0, S, 17)))).astype(np.int64)


# Head dim 256 runs a persistent grid (one workgroup per CU, each taking
# several blocks of 128 rows in zig-zag rounds and loading the next block's
# Q and first tiles before writing the current block's O). Shapes with more
# blocks than workgroups exercise the rounds: rows sampled in every block,
# blocks without any visible key (Sq > Skv) between ones with keys, and a
# score transform.
PERSISTENT = [
    # B, Sq, Skv, Hq, Hkv, causal, window, softcap, additive mask
    (4, 2048, 2048, 16, 8, 1, 300, 0.0, False),
    (8, 2048, 512, 8, 8, 1, 0, 0.0, False),
    (2, 1536, 1536, 12, 4, 0, 0, 0.0, False),
    (4, 2048, 2048, 16, 8, 1, 0, 20.0, False),
    (4, 2048, 2048, 16, 8, 1, 0, 0.0, True),
]


@pytest.mark.parametrize("case", PERSISTENT, ids=lambda c: "B{}_Sq{}_Skv{}_H{}x{}_c{}_w{}_cap{}_mask{}".format(*c))
def test_prefill_persistent_rounds(case):
    B, Sq, Skv, Hq, Hkv, causal, window, softcap, with_mask = case
    print(f"case {case}", flush=True)
    D = 256
    q, k, v = workloads.random_inputs(B, Sq, Skv, Hq, Hkv, D, seed=B * Sq + Skv + Hq)
    scale = 1.0 / np.sqrt(D)
    mask = None
    if with_mask:
        # N(0, 2) per (sequence, row, key), a hidden band of keys per sequence
        g = torch.Generator().manual_seed(11)
        m = 2.0 * torch.randn(B, Sq, Skv, generator=g)
        for b in range(B):
            m[b, :, 300 * b + 100:300 * b + 140] = -float("inf")
        mask = m.to(torch.bfloat16)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=bool(causal), window=window, scale=scale,
                        softcap=softcap, mask=None if mask is None else mask.to(DEV))
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    G = Hq // Hkv
    pos_per_block = 128 // G
    gen = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(0, Sq, pos_per_block),
                                     np.arange(pos_per_block - 1, Sq, pos_per_block),
                                     gen.integers(0, Sq, 64)])).astype(np.int64)
    heads = sorted({0, 1, Hq // 2, Hq - 1})
    for b in sorted({0, B - 1}):
        o_ref, lse_ref = oracle.attention_ref(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=bool(causal),
                                              window=window, scale=scale, rows=rows, heads=heads,
                                              softcap=softcap, mask=None if mask is None else mask[b:b + 1])
        assert_parity(o[b:b + 1][:, rows][:, :, heads], lse[b:b + 1][:, heads][:, :, rows],
                      o_ref[:, rows][:, :, heads], lse_ref[:, heads][:, :, rows], f"persistent {case} b{b}")


def test_prefill_c2_full_size_sampled():
    s = workloads.C2
    q, k, v = workloads.prefill_inputs(s)
    _sampled(s, q, k, v, _rows(s.Sq), [0, 3, 4, 17, 31])


def test_prefill_c4a_full_size_sampled():
    s = workloads.C4A
    q, k, v = workloads.c4_inputs()[0]
    _sampled(s, q, k, v, _rows(s.Sq), [0, 1, 9, 15])


def test_prefill_c4b_full_size_sampled():
    s = workloads.C4B
    q, k, v = workloads.c4_inputs()[1]
    _sampled(s, q, k, v, _rows(s.Sq), [0, 1, 14, 15])
