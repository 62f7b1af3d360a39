"""Split-KV decode / verify parity through the C ABI: against the fp64
oracle on ragged lengths with NaN-poisoned cache slots past each sequence's
end, paged (random page permutation) vs contiguous bit identity, the paged
gather against a CPU gather byte for byte, the LSE combine against the
oracle merge, and sampled outputs of the full-size decode and verify
workloads."""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
import workloads
from tests.gpu_util import DEV, assert_parity, to_np

pytestmark = pytest.mark.gpu


def _decode(di, shape, **kw):
    table = None if di.block_table is None else di.block_table.to(DEV)
    ps = shape.page_size or 16
    o, lse = fa.decode_paged(di.q.to(DEV), di.kcache.to(DEV), di.vcache.to(DEV), table,
                             di.seq_lens.to(DEV), page_size=ps, kv_chunk=shape.kv_chunk,
                             causal=shape.causal, window=shape.window, scale=shape.scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def _ref(di, shape, **kw):
    ps = shape.page_size or 16
    return oracle.decode_paged_ref(di.q, di.kcache, di.vcache, di.block_table, di.seq_lens,
                                   page_size=ps, causal=shape.causal, window=shape.window,
                                   scale=shape.scale, **kw)


DECODE_GRID = [
    # B, Sq, Hq, Hkv, D, page_size (0 = contiguous), max_len, len range, chunk, window
    (4, 1, 32, 8, 128, 0, 2048, (1, 2048), 256, 0),
    (3, 1, 8, 8, 64, 16, 1024, (1, 1024), 128, 0),
    (2, 8, 64, 8, 128, 16, 1024, (8, 1024), 256, 0),
    (2, 8, 16, 8, 128, 16, 768, (300, 768), 96, 0),
    (2, 4, 8, 2, 256, 32, 512, (4, 512), 128, 0),
    (2, 3, 8, 4, 512, 16, 512, (3, 512), 160, 0),
    (2, 1, 16, 2, 256, 0, 640, (17, 640), 64, 0),
    (2, 16, 32, 4, 128, 16, 512, (16, 512), 128, 0),    # 128 rows per KV head
    (2, 8, 64, 8, 128, 16, 1024, (8, 1024), 256, 100),  # sliding window
    (2, 2, 4, 1, 64, 64, 256, (0, 256), 64, 0),         # zero-length sequences possible
    # over 16384 (sequence, KV head, chunk) slots: several chunks per workgroup
    (64, 1, 16, 4, 64, 0, 4096, (1, 4096), 32, 0),
    (40, 2, 8, 4, 128, 16, 4096, (1, 4096), 32, 0),
]


@pytest.mark.parametrize("case", DECODE_GRID, ids=lambda c: "B{}_Sq{}_H{}x{}_D{}_ps{}_L{}_{}_c{}_w{}".format(*c))
def test_decode_grid(case):
    B, Sq, Hq, Hkv, D, ps, max_len, (lo, hi), chunk, window = case
    print(f"case {case}", flush=True)
    shape = workloads.DecodeShape("grid", B=B, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, page_size=ps,
                                  max_len=max_len, len_lo=lo, len_hi=hi, kv_chunk=chunk,
                                  window=window, seed=abs(hash(case)) % 10007)
    di = workloads.decode_inputs(shape, poison_tail=True)
    o, lse = _decode(di, shape)
    o_ref, lse_ref = _ref(di, shape)
    assert_parity(o, lse, o_ref, lse_ref, f"decode {case}")


def test_paged_equals_contiguous_bitwise():
    shape = workloads.DecodeShape("pc", B=3, Sq=8, Hq=32, Hkv=4, D=128, page_size=16, max_len=1024,
                                  len_lo=200, len_hi=1024, kv_chunk=256, seed=21)
    di = workloads.decode_inputs(shape)
    # lay the same tokens out contiguously
    kc = oracle.paged_gather_ref(di.kcache, di.block_table, di.seq_lens, 16, shape.max_len)
    vc = oracle.paged_gather_ref(di.vcache, di.block_table, di.seq_lens, 16, shape.max_len)
    o1, l1 = _decode(di, shape)
    cont = workloads.DecodeInputs(di.q, kc.contiguous(), vc.contiguous(), None, di.seq_lens)
    o2, l2 = _decode(cont, shape)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_gather_bitexact():
    gen = torch.Generator().manual_seed(4)
    P, ps, Hkv, D, B, mp = 97, 16, 3, 64, 4, 20
    cache = torch.randn(P, ps, Hkv, D, generator=gen).to(torch.bfloat16)
    table = torch.randint(0, P, (B, mp), generator=gen, dtype=torch.int32)
    table[1, 3] = P + 5          # out-of-range entries read the page they clamp to
    table[2, 0] = -1
    lens = torch.tensor([320, 60, 1, 0], dtype=torch.int32)
    out = fa.paged_gather(cache.to(DEV), table.to(DEV), lens.to(DEV))
    torch.cuda.synchronize()
    ref = torch.zeros(B, mp * ps, Hkv, D, dtype=torch.bfloat16)
    for b in range(B):
        for t in range(int(lens[b])):
            pg = min(max(int(table[b, t // ps]), 0), P - 1)
            ref[b, t] = cache[pg, t % ps]
    assert torch.equal(out.cpu().view(torch.int16), ref.view(torch.int16))
    # the oracle's gather agrees where every table entry is valid
    valid = table.clone()
    valid[1, 3] = 0
    valid[2, 0] = 0
    g2 = fa.paged_gather(cache.to(DEV), valid.to(DEV), lens.to(DEV)).cpu()
    r2 = oracle.paged_gather_ref(cache, valid, lens, ps, mp * ps)
    assert torch.equal(g2.view(torch.int16), r2.view(torch.int16))


def test_out_of_range_table_entry_is_clamped():
    """A block-table entry outside [0, num_pages) is clamped into range by the
    decode kernel (the rule the gather hook shares): the call equals the
    same call over the clamped table, bit for bit, and reads nothing out of
    bounds."""
    shape = workloads.DecodeShape("clamp", B=3, Sq=8, Hq=16, Hkv=2, D=128, page_size=16, max_len=1024,
                                  len_lo=600, len_hi=1024, kv_chunk=256, seed=23)
    di = workloads.decode_inputs(shape)
    P = di.kcache.shape[0]
    bad = di.block_table.clone()
    bad[0, 2] = P + 7
    bad[1, 0] = -3
    bad[2, 5] = 1 << 30
    clamped = bad.clamp(0, P - 1)
    o1, l1 = _decode(workloads.DecodeInputs(di.q, di.kcache, di.vcache, bad, di.seq_lens), shape)
    o2, l2 = _decode(workloads.DecodeInputs(di.q, di.kcache, di.vcache, clamped, di.seq_lens), shape)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_combine_caps_lengths_at_the_cache():
    """seq_lens beyond the cache's capacity are clamped to it, also when the
    capacity is zero: rows of an empty cache get O = 0 and LSE = -inf."""
    B, Sq, Hq, Hkv, D = 2, 1, 8, 2, 64
    q = torch.randn(B, Sq, Hq, D).to(torch.bfloat16).to(DEV)
    kc = torch.zeros(B, 0, Hkv, D, dtype=torch.bfloat16, device=DEV)
    lens = torch.tensor([5, 300], dtype=torch.int32, device=DEV)
    o, lse = fa.decode_paged(q, kc, kc, None, lens, page_size=16, kv_chunk=64)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


COMBINE_CASES = [(D, 7, (7, 5, 0)) for D in (64, 128, 256, 512)] + [
    (128, 70, (70, 65, 1)),        # chunks past the first 64 (second LSE register)
    (64, 300, (300, 257, 64)),     # more than 256 chunks (LSEs re-read from memory)
    (512, 300, (299, 130, 256)),
]


@pytest.mark.parametrize("case", COMBINE_CASES, ids=lambda c: "D{}_C{}".format(c[0], c[1]))
def test_combine_against_oracle(case):
    D, C, counts = case
    gen = torch.Generator().manual_seed(D + C)
    B, Hq, Sq = 3, 4, 2
    o_part = torch.randn(B, Hq, Sq, C, D, generator=gen)
    lse_part = 3 * torch.randn(B, Hq, Sq, C, generator=gen)
    empty = [(0, 1, 0, 2), (0, 3, 1, C - 2)]
    for e in empty:
        lse_part[e] = float("-inf")                 # an empty chunk
        o_part[e] = float("nan")                    # whose contents must be ignored
    lse_part[1, 2, 1, :] = float("-inf")            # a row with no key at all
    n_chunks = torch.tensor(counts, dtype=torch.int32)
    o, lse = fa.combine_lse(o_part.to(DEV), lse_part.to(DEV), n_chunks.to(DEV))
    torch.cuda.synchronize()
    op = o_part.clone()
    for e in empty:
        op[e] = 0.0
    o_ref, lse_ref = oracle.combine_ref(op, lse_part, n_chunks.tolist())
    assert_parity(o, lse, o_ref, lse_ref, f"combine D{D} C{C}")


def test_decode_c3_full_size_sampled():
    s = workloads.C3
    di = workloads.decode_inputs(s)
    o, lse = _decode(di, s)
    heads = [0, 5, 31]
    o, lse = to_np(o), to_np(lse)
    for b in (0, 7, 15):
        sub = workloads.DecodeInputs(di.q[b:b + 1], di.kcache[b:b + 1], di.vcache[b:b + 1], None,
                                     di.seq_lens[b:b + 1])
        o_ref, lse_ref = _ref(sub, s, heads=heads)
        assert_parity(o[b:b + 1][:, :, heads], lse[b:b + 1][:, heads], o_ref[:, :, heads],
                      lse_ref[:, heads], f"C3 b{b} len {int(di.seq_lens[b])}")


def test_verify_c5_full_size_sampled():
    s = workloads.C5
    di = workloads.decode_inputs(s)
    o, lse = _decode(di, s)
    heads = [0, 7, 8, 63]
    o_ref, lse_ref = _ref(di, s, heads=heads)
    assert_parity(to_np(o)[:, :, heads], to_np(lse)[:, heads], o_ref[:, :, heads], lse_ref[:, heads],
                  "C5 sampled heads")


def _ws_for(shape, fill=None):
    ps = shape.page_size or 16
    n = fa.decode_workspace_bytes(shape.B, shape.Sq, shape.Hq, shape.D, shape.max_len, shape.kv_chunk)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    if fill is not None:
        ws.view(torch.float32)[: n // 4].fill_(fill)
    return ws


@pytest.mark.parametrize("mods", [False, True])
def test_decode_deterministic(mods):
    """Repeated calls give the same bits (the split depends only on shapes,
    lengths and the GPU)."""
    shape = workloads.DecodeShape("det", B=6, Sq=4, Hq=32, Hkv=8, D=128, page_size=16, max_len=2048,
                                  len_lo=1, len_hi=2048, kv_chunk=256, seed=31)
    di = workloads.decode_inputs(shape)
    kw = dict(softcap=25.0, max_bias=6.0, sinks=torch.randn(32).to(DEV)) if mods else {}
    o1, l1 = _decode(di, shape, **kw)
    o2, l2 = _decode(di, shape, **kw)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_poisoned_workspace():
    """A workspace full of NaN before the call changes nothing: the combine
    reads only slots written by this call."""
    shape = workloads.DecodeShape("poison", B=5, Sq=8, Hq=64, Hkv=8, D=128, page_size=16, max_len=1536,
                                  len_lo=0, len_hi=1536, kv_chunk=128, seed=33)
    di = workloads.decode_inputs(shape)
    o1, l1 = _decode(di, shape, workspace=_ws_for(shape, fill=0.0))
    o2, l2 = _decode(di, shape, workspace=_ws_for(shape, fill=float("nan")))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    o_ref, lse_ref = _ref(di, shape)
    assert_parity(o2, l2, o_ref, lse_ref, "decode with a NaN-filled workspace")


def test_decode_workspace_reused_across_shapes():
    """One workspace serves a large call and then smaller ones: no stale
    partial of the earlier call leaks into a later one."""
    big = workloads.DecodeShape("big", B=8, Sq=8, Hq=32, Hkv=4, D=128, page_size=16, max_len=4096,
                                len_lo=2000, len_hi=4096, kv_chunk=128, seed=35)
    ws = _ws_for(big)
    _decode(workloads.decode_inputs(big), big, workspace=ws)
    for i, (B, Sq, Hq, Hkv, D, L, chunk) in enumerate([(3, 2, 16, 4, 128, 1024, 256), (2, 8, 32, 4, 64, 512, 64),
                                                        (4, 1, 32, 8, 128, 3000 // 16 * 16, 128)]):
        small = workloads.DecodeShape("small", B=B, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, page_size=16, max_len=L,
                                      len_lo=0, len_hi=L, kv_chunk=chunk, seed=36 + i)
        di = workloads.decode_inputs(small)
        assert fa.decode_workspace_bytes(B, Sq, Hq, D, L, chunk) <= ws.numel()
        o1, l1 = _decode(di, small, workspace=ws)
        o2, l2 = _decode(di, small, workspace=_ws_for(small, fill=0.0))
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), i
