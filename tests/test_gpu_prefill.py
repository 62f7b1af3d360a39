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
