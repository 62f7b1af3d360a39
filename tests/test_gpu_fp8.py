"""fp8 (OCP e4m3) KV caches through the C ABI: the quantising append must
produce the oracle's codes byte for byte (values from subnormal to
saturating, per-head scales, paged and contiguous caches), and decode /
verify over fp8 caches must match the fp64 oracle on the dequantised cache
at the usual tolerances (NaN codes past each sequence's end, score
modifiers, the full-size decode workload on sampled rows)."""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
import workloads
from tests.gpu_util import DEV, assert_parity, to_np

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


def _quantized_cache(gen, shape, scale):
    """uint8 codes of N(0,1) bf16 values quantised by the oracle with the
    per-head scales (shape [..., Hkv, D])."""
    x = torch.randn(shape, generator=gen).to(torch.bfloat16).float().numpy()
    q = x.astype(np.float32) / scale.numpy().astype(np.float32)[:, None]
    return torch.from_numpy(oracle.quantize_e4m3(q))


def _scales(gen, Hkv, base):
    return (base * torch.exp(0.5 * torch.randn(Hkv, generator=gen))).float()


def _deq(codes, scale):
    return oracle.dequantize_e4m3(codes.numpy(), scale.numpy())


@pytest.mark.parametrize("D", [128, 256, 512])
def test_fp8_every_code_widens_exactly(D):
    """Every finite e4m3 code through the kernels' widening, both paths: one
    key per sequence, so O is that key's V row (each code once per 128
    columns) and LSE is its single score; with one-hot queries the score is
    one K element times the softmax scale (unit dequantisation scales)."""
    print(f"fp8 codes D={D}", flush=True)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)   # 254 finite codes
    B, Hq, Hkv = 2 * (D // 32), 32, 1
    # sequence b holds 128 codes (half b % 2 of the code list) in V at columns
    # (c + 37 b) % D, and in K; query head h of sequence b is one-hot at
    # column d = 32 (b // 2) + h
    half = [codes[:128], np.concatenate([codes[128:], codes[:2]])]
    kc = np.zeros((B, 1, Hkv, D), np.uint8)
    vc = np.zeros((B, 1, Hkv, D), np.uint8)
    for b in range(B):
        row = np.resize(half[b % 2], D)
        kc[b, 0, 0] = row
        vc[b, 0, 0] = np.roll(row, 37 * b)
    q = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16)
    for b in range(B):
        for h in range(Hq):
            q[b, 0, h, 32 * (b // 2) + h] = 1.0
    one = torch.ones(Hkv, dtype=torch.float32)
    lens = torch.ones(B, dtype=torch.int32)
    scale = 0.125
    o, lse = fa.decode_paged_fp8(q.to(DEV), torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                                 one.to(DEV), one.to(DEV), None, lens.to(DEV), page_size=1, kv_chunk=32,
                                 scale=scale)
    torch.cuda.synchronize()
    vref = oracle.dequantize_e4m3(vc, one.numpy())            # fp64 [B, 1, 1, D]
    kref = oracle.dequantize_e4m3(kc, one.numpy())
    o = to_np(o)
    lse = to_np(lse)
    for b in range(B):
        np.testing.assert_array_equal(o[b, 0], np.broadcast_to(vref[b, 0, 0], (Hq, D)))
        d = 32 * (b // 2) + np.arange(Hq)
        np.testing.assert_allclose(lse[b, :, 0], kref[b, 0, 0, d] * scale, rtol=1e-6, atol=1e-30)
    # the one-hot queries read every finite code out of K, and every V row holds its half of them
    seen_k = {int(x) for b in range(B) for x in kc[b, 0, 0][32 * (b // 2):32 * (b // 2) + 32]}
    seen_v = {int(x) for b in range(B) for x in vc[b, 0, 0]}
    assert seen_k == set(codes.tolist()) and seen_v == set(codes.tolist())


@pytest.mark.parametrize("paged", [True, False])
def test_fp8_append_bitexact(paged):
    print(f"fp8 append paged={paged}", flush=True)
    g = torch.Generator().manual_seed(71 + int(paged))
    B, Snew, Hkv, D, ps, mp = 4, 8, 4, 128, 16, 10
    P = B * mp + 3
    if paged:
        table = torch.randperm(P, generator=g)[: B * mp].reshape(B, mp).to(torch.int32)
        table[3, 0] = -1                                   # out of range: sequence 3's first page skipped
        kc = torch.randint(0, 256, (P, ps, Hkv, D), generator=g, dtype=torch.int32).to(torch.uint8)
    else:
        table = None
        kc = torch.randint(0, 256, (B, mp * ps, Hkv, D), generator=g, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, kc.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    lens = torch.tensor([mp * ps, 37, 5, 12], dtype=torch.int32)
    # magnitudes from 1e-6 (subnormal codes and zero) to 1e4 (saturating)
    mag = torch.pow(10.0, torch.empty(B, Snew, Hkv, D).uniform_(-6, 4, generator=g))
    kn = (torch.randn(B, Snew, Hkv, D, generator=g) * mag).to(torch.bfloat16)
    vn = (torch.randn(B, Snew, Hkv, D, generator=g) * mag).to(torch.bfloat16)
    kn[0, 0, 0, :4] = torch.tensor([0.0, -0.0, float("inf"), float("-inf")], dtype=torch.bfloat16)
    ks = torch.tensor([0.5, 0.01, 3.0, 1.0], dtype=torch.float32)
    vs = torch.tensor([0.25, 2.0, 0.003, 1.0], dtype=torch.float32)
    kd, vd = kc.to(DEV), vc.to(DEV)
    fa.kv_append_fp8(kd, vd, ks.to(DEV), vs.to(DEV), None if table is None else table.to(DEV), lens.to(DEV),
                     kn.to(DEV), vn.to(DEV), page_size=ps)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.kv_append_fp8_ref(kc.numpy(), vc.numpy(), None if table is None else table.numpy(),
                                            lens.numpy(), kn, vn, ks.numpy(), vs.numpy(), page_size=ps)
    kg, vg = kd.cpu().numpy(), vd.cpu().numpy()
    bad = np.argwhere(kg != k_ref)
    assert bad.size == 0, f"{len(bad)} K codes differ, first at {bad[:3].tolist()}"
    assert np.array_equal(vg, v_ref)


DECODE = [
    # B, Sq, Hq, Hkv, page_size (0 = contiguous), max_len, len range, chunk
    (4, 1, 32, 8, 0, 2048, (1, 2048), 256),
    (3, 1, 16, 4, 16, 1024, (1, 1024), 128),
    (2, 8, 64, 8, 16, 1024, (8, 1024), 256),           # verify: 64 rows per KV head
    (2, 4, 32, 4, 32, 768, (4, 768), 96),
    (2, 2, 8, 1, 64, 256, (0, 256), 64),                # zero-length sequences possible
    (40, 2, 8, 4, 16, 4096, (1, 4096), 32),             # several ranges per workgroup set
]


def _fp8_case(case, seed, D=128):
    B, Sq, Hq, Hkv, ps, max_len, (lo, hi), chunk = case
    shape = workloads.DecodeShape("fp8", B=B, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, max_len=max_len,
                                  len_lo=lo, len_hi=hi, kv_chunk=chunk, seed=seed)
    di = workloads.decode_inputs(shape)
    g = torch.Generator().manual_seed(seed + 1)
    ks, vs = _scales(g, Hkv, 4.0 / 448), _scales(g, Hkv, 4.0 / 448)
    kc = _quantized_cache(g, di.kcache.shape, ks)
    vc = _quantized_cache(g, di.vcache.shape, vs)
    # NaN codes in every slot past each sequence's end
    lens = di.seq_lens.tolist()
    for b, n in enumerate(lens):
        if di.block_table is None:
            kc[b, n:] = NAN_CODE
            vc[b, n:] = NAN_CODE
        else:
            for t in range(n, di.block_table.shape[1] * ps):
                page = int(di.block_table[b, t // ps])
                kc[page, t % ps] = NAN_CODE
                vc[page, t % ps] = NAN_CODE
    return shape, di, kc, vc, ks, vs


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B{}_Sq{}_H{}x{}_ps{}_L{}_{}_c{}".format(*c))
def test_fp8_decode(case):
    print(f"fp8 decode {case}", flush=True)
    shape, di, kc, vc, ks, vs = _fp8_case(case, seed=case[0] * 13 + case[1])
    ps = shape.page_size or 16
    table = None if di.block_table is None else di.block_table.to(DEV)
    o, lse = fa.decode_paged_fp8(di.q.to(DEV), kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV), table,
                                 di.seq_lens.to(DEV), page_size=ps, kv_chunk=shape.kv_chunk, causal=True,
                                 scale=shape.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, _deq(kc, ks), _deq(vc, vs), di.block_table, di.seq_lens,
                                             page_size=ps, causal=True, scale=shape.scale)
    assert_parity(o, lse, o_ref, lse_ref, f"fp8 decode {case}")


def test_fp8_verify_all_modifiers():
    case = (2, 8, 32, 4, 16, 768, (300, 768), 256)
    shape, di, kc, vc, ks, vs = _fp8_case(case, seed=501)
    g = torch.Generator().manual_seed(502)
    sinks = torch.randn(shape.Hq, generator=g).float()
    mask = (2.0 * torch.randn(shape.B, shape.Sq, shape.max_len, generator=g)).to(torch.bfloat16)
    mask[:, :, 3:9] = -float("inf")
    kw = dict(softcap=20.0, max_bias=4.0)
    o, lse = fa.decode_paged_fp8(di.q.to(DEV), kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV),
                                 di.block_table.to(DEV), di.seq_lens.to(DEV), page_size=16, kv_chunk=256,
                                 causal=True, scale=shape.scale, sinks=sinks.to(DEV), mask=mask.to(DEV), **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, _deq(kc, ks), _deq(vc, vs), di.block_table, di.seq_lens,
                                             page_size=16, causal=True, scale=shape.scale,
                                             sinks=sinks.double().numpy(), mask=mask, **kw)
    assert_parity(o, lse, o_ref, lse_ref, "fp8 verify all modifiers")


def test_fp8_append_then_decode():
    g = torch.Generator().manual_seed(601)
    B, Sq, Hq, Hkv, D, ps, mp = 2, 4, 16, 2, 128, 16, 20
    P = B * mp
    table = torch.randperm(P, generator=g).reshape(B, mp).to(torch.int32)
    ks, vs = _scales(g, Hkv, 3.0 / 448), _scales(g, Hkv, 3.0 / 448)
    kc = _quantized_cache(g, (P, ps, Hkv, D), ks)
    vc = _quantized_cache(g, (P, ps, Hkv, D), vs)
    lens = torch.tensor([mp * ps - 7, 150], dtype=torch.int32)
    kn = torch.randn(B, Sq, Hkv, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, Sq, Hkv, D, generator=g).to(torch.bfloat16)
    q = torch.randn(B, Sq, Hq, D, generator=g).to(torch.bfloat16)
    kd, vd = kc.to(DEV), vc.to(DEV)
    fa.kv_append_fp8(kd, vd, ks.to(DEV), vs.to(DEV), table.to(DEV), lens.to(DEV), kn.to(DEV), vn.to(DEV),
                     page_size=ps)
    o, lse = fa.decode_paged_fp8(q.to(DEV), kd, vd, ks.to(DEV), vs.to(DEV), table.to(DEV), lens.to(DEV),
                                 page_size=ps, kv_chunk=128)
    torch.cuda.synchronize()
    k2, v2 = oracle.kv_append_fp8_ref(kc.numpy(), vc.numpy(), table.numpy(), lens.numpy(), kn, vn,
                                      ks.numpy(), vs.numpy(), page_size=ps)
    assert np.array_equal(kd.cpu().numpy(), k2) and np.array_equal(vd.cpu().numpy(), v2)
    o_ref, lse_ref = oracle.decode_paged_ref(q, oracle.dequantize_e4m3(k2, ks.numpy()),
                                             oracle.dequantize_e4m3(v2, vs.numpy()), table, lens, page_size=ps,
                                             causal=True, scale=1.0 / np.sqrt(D))
    assert_parity(o, lse, o_ref, lse_ref, "fp8 append + decode")


def test_fp8_decode_c3_shape_sampled():
    """The 1-row decode workload at full size over an fp8 cache: sampled
    sequences and heads against the oracle."""
    s = workloads.C3
    di = workloads.decode_inputs(s)
    g = torch.Generator().manual_seed(701)
    ks, vs = _scales(g, s.Hkv, 4.0 / 448), _scales(g, s.Hkv, 4.0 / 448)
    # each sequence's valid tokens quantised by the oracle; NaN codes past its end
    kq = torch.full(di.kcache.shape, NAN_CODE, dtype=torch.uint8)
    vq = torch.full(di.vcache.shape, NAN_CODE, dtype=torch.uint8)
    ksn, vsn = ks.numpy().astype(np.float32)[:, None], vs.numpy().astype(np.float32)[:, None]
    for b in range(s.B):
        n = int(di.seq_lens[b])
        kq[b, :n] = torch.from_numpy(oracle.quantize_e4m3(di.kcache[b, :n].float().numpy() / ksn))
        vq[b, :n] = torch.from_numpy(oracle.quantize_e4m3(di.vcache[b, :n].float().numpy() / vsn))
    o, lse = fa.decode_paged_fp8(di.q.to(DEV), kq.to(DEV), vq.to(DEV), ks.to(DEV), vs.to(DEV), None,
                                 di.seq_lens.to(DEV), page_size=16, kv_chunk=s.kv_chunk, causal=True,
                                 scale=s.scale)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    heads = sorted({0, 5, s.Hq // 2, s.Hq - 1})
    for b in sorted({0, s.B // 2, s.B - 1}):
        n = int(di.seq_lens[b])
        kd = oracle.dequantize_e4m3(kq[b:b + 1, :n].numpy(), ks.numpy())
        vd = oracle.dequantize_e4m3(vq[b:b + 1, :n].numpy(), vs.numpy())
        o_ref, lse_ref = oracle.decode_paged_ref(di.q[b:b + 1], kd, vd, None, di.seq_lens[b:b + 1],
                                                 page_size=16, causal=True, scale=s.scale, heads=heads)
        assert_parity(o[b:b + 1][:, :, heads], lse[b:b + 1][:, heads], o_ref[:, :, heads], lse_ref[:, heads],
                      f"fp8 C3 b{b}")


def test_fp8_interleaved_cache_bitwise():
    """K and V interleaved per slot in one uint8 allocation (strided views)
    give the same bits as separate contiguous caches."""
    case = (3, 4, 32, 4, 16, 512, (4, 512), 128)
    shape, di, kc, vc, ks, vs = _fp8_case(case, seed=901)
    both = torch.stack([kc, vc], dim=2).to(DEV)          # [pages, slot, 2, Hkv, D]
    args = (ks.to(DEV), vs.to(DEV), di.block_table.to(DEV), di.seq_lens.to(DEV))
    o1, l1 = fa.decode_paged_fp8(di.q.to(DEV), both[:, :, 0], both[:, :, 1], *args, page_size=16,
                                 kv_chunk=128, scale=shape.scale)
    o2, l2 = fa.decode_paged_fp8(di.q.to(DEV), kc.to(DEV), vc.to(DEV), *args, page_size=16, kv_chunk=128,
                                 scale=shape.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_fp8_decode_window():
    case = (2, 8, 64, 8, 16, 1024, (8, 1024), 256)
    shape, di, kc, vc, ks, vs = _fp8_case(case, seed=911)
    o, lse = fa.decode_paged_fp8(di.q.to(DEV), kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV),
                                 di.block_table.to(DEV), di.seq_lens.to(DEV), page_size=16, kv_chunk=256,
                                 causal=True, window=100, scale=shape.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, _deq(kc, ks), _deq(vc, vs), di.block_table, di.seq_lens,
                                             page_size=16, causal=True, window=100, scale=shape.scale)
    assert_parity(o, lse, o_ref, lse_ref, "fp8 verify window 100")


# head dims 256 and 512 (the pages' quantised-cache layers: head 256 on SWA
# layers, 512 on global layers): the D-split fp8 kernels
LARGE = [
    # D, B, Sq, Hq, Hkv, page_size (0 = contiguous), max_len, len range, chunk
    (256, 3, 1, 16, 8, 16, 1024, (1, 1024), 128),
    (256, 2, 8, 32, 4, 0, 768, (8, 768), 256),          # 64 rows per KV head: two row groups
    (256, 2, 2, 8, 1, 64, 256, (0, 256), 64),            # zero-length sequences possible
    (512, 3, 1, 16, 8, 16, 1024, (1, 1024), 128),
    (512, 2, 4, 32, 4, 0, 512, (4, 512), 96),            # 32 rows per KV head, several row blocks
    (512, 20, 2, 8, 4, 16, 2048, (1, 2048), 32),         # several ranges per workgroup set
]


@pytest.mark.parametrize("case", LARGE, ids=lambda c: "D{}_B{}_Sq{}_H{}x{}_ps{}_L{}_{}_c{}".format(*c))
def test_fp8_decode_large_head_dims(case):
    print(f"fp8 decode large head dim {case}", flush=True)
    D = case[0]
    shape, di, kc, vc, ks, vs = _fp8_case(case[1:], seed=case[1] * 17 + D + case[2], D=D)
    ps = shape.page_size or 16
    table = None if di.block_table is None else di.block_table.to(DEV)
    o, lse = fa.decode_paged_fp8(di.q.to(DEV), kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV), table,
                                 di.seq_lens.to(DEV), page_size=ps, kv_chunk=shape.kv_chunk, causal=True,
                                 scale=shape.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, _deq(kc, ks), _deq(vc, vs), di.block_table, di.seq_lens,
                                             page_size=ps, causal=True, scale=shape.scale)
    assert_parity(o, lse, o_ref, lse_ref, f"fp8 decode D{D} {case}")


@pytest.mark.parametrize("D", [256, 512])
def test_fp8_large_head_dims_modifiers_and_append(D):
    """Every score modifier and a window over an fp8 cache at head dim 256 /
    512, then an fp8 append of 4 new rows and the verify over the result."""
    case = (2, 4, 16, 2, 16, 640, (300, 640), 128)
    shape, di, kc, vc, ks, vs = _fp8_case(case, seed=1200 + D, D=D)
    g = torch.Generator().manual_seed(1300 + D)
    sinks = torch.randn(shape.Hq, generator=g).float()
    mask = (2.0 * torch.randn(shape.B, shape.Sq, shape.max_len, generator=g)).to(torch.bfloat16)
    mask[:, :, 5:11] = -float("inf")
    kw = dict(softcap=20.0, max_bias=4.0)
    o, lse = fa.decode_paged_fp8(di.q.to(DEV), kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV),
                                 di.block_table.to(DEV), di.seq_lens.to(DEV), page_size=16, kv_chunk=128,
                                 causal=True, window=200, scale=shape.scale, sinks=sinks.to(DEV),
                                 mask=mask.to(DEV), **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, _deq(kc, ks), _deq(vc, vs), di.block_table, di.seq_lens,
                                             page_size=16, causal=True, window=200, scale=shape.scale,
                                             sinks=sinks.double().numpy(), mask=mask, **kw)
    assert_parity(o, lse, o_ref, lse_ref, f"fp8 D{D} all modifiers")
    # append 4 new rows (placed at the end of each sequence), then verify
    Hkv = shape.Hkv
    kn = torch.randn(shape.B, 4, Hkv, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(shape.B, 4, Hkv, D, generator=g).to(torch.bfloat16)
    kd, vd = kc.to(DEV), vc.to(DEV)
    fa.kv_append_fp8(kd, vd, ks.to(DEV), vs.to(DEV), di.block_table.to(DEV), di.seq_lens.to(DEV), kn.to(DEV),
                     vn.to(DEV), page_size=16)
    o, lse = fa.decode_paged_fp8(di.q.to(DEV), kd, vd, ks.to(DEV), vs.to(DEV), di.block_table.to(DEV),
                                 di.seq_lens.to(DEV), page_size=16, kv_chunk=128, causal=True, scale=shape.scale)
    torch.cuda.synchronize()
    k2, v2 = oracle.kv_append_fp8_ref(kc.numpy(), vc.numpy(), di.block_table.numpy(), di.seq_lens.numpy(), kn,
                                      vn, ks.numpy(), vs.numpy(), page_size=16)
    assert np.array_equal(kd.cpu().numpy(), k2) and np.array_equal(vd.cpu().numpy(), v2)
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, oracle.dequantize_e4m3(k2, ks.numpy()),
                                             oracle.dequantize_e4m3(v2, vs.numpy()), di.block_table, di.seq_lens,
                                             page_size=16, causal=True, scale=shape.scale)
    assert_parity(o, lse, o_ref, lse_ref, f"fp8 D{D} append + verify")
