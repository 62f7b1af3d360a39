"""Score modifiers (logit softcap, ALiBi from max_bias, attention sinks)
through the C ABI against the fp64 oracle: prefill at every head dimension,
decode and verify over paged and contiguous caches (where the sinks enter
in the LSE combine), rows with no visible key (O = 0, LSE = the sink), and
sampled outputs of a full-size decode workload with all three on."""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
import workloads
from tests.gpu_util import DEV, assert_parity, to_np

pytestmark = pytest.mark.gpu


def _sinks(Hq, seed):
    g = torch.Generator().manual_seed(seed)
    return (2.0 * torch.randn(Hq, generator=g)).float()


MODS = {
    "softcap": dict(softcap=30.0),
    "tight_cap": dict(softcap=2.5),
    "alibi": dict(max_bias=8.0),
    "sinks": dict(sinks=True),
    "all": dict(softcap=20.0, max_bias=4.0, sinks=True),
}


def _kw(name, Hq, seed, dev):
    kw = dict(MODS[name])
    sk = None
    if kw.pop("sinks", False):
        sk = _sinks(Hq, seed)
        kw["sinks"] = sk.to(dev) if dev is not None else sk
    return kw, sk


PREFILL = [
    # B, Sq, Skv, Hq, Hkv, D, causal, window, modifiers
    (2, 200, 200, 8, 2, 64, True, 0, "all"),
    (1, 130, 300, 12, 4, 128, True, 0, "alibi"),       # 12 heads: two slope sequences
    (2, 257, 257, 8, 2, 128, True, 64, "softcap"),
    (1, 96, 96, 4, 4, 128, False, 0, "tight_cap"),
    (1, 150, 150, 8, 2, 256, True, 0, "all"),
    (1, 70, 70, 4, 2, 512, True, 0, "sinks"),
    (1, 80, 48, 8, 2, 128, True, 0, "sinks"),          # Sq > Skv: the first rows see no key
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}_S{}x{}_H{}x{}_D{}_c{}_w{}_{}".format(*c))
def test_prefill_mods(case):
    B, Sq, Skv, Hq, Hkv, D, causal, window, mods = case
    print(f"prefill mods {case}", flush=True)
    q, k, v = workloads.random_inputs(B, Sq, Skv, Hq, Hkv, D, seed=Sq + 7 * D)
    scale = 1.0 / np.sqrt(D)
    kw, sk = _kw(mods, Hq, D + Sq, DEV)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, scale=scale, **kw)
    torch.cuda.synchronize()
    rkw = dict(kw)
    if sk is not None:
        rkw["sinks"] = sk.double().numpy()
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=causal, window=window, scale=scale, **rkw)
    assert_parity(o, lse, o_ref, lse_ref, f"prefill mods {case}")
    if Sq > Skv and causal:
        # rows before the first key: O = 0 exactly, LSE = the head's sink
        ln = to_np(lse)[:, :, : Sq - Skv]
        assert np.all(to_np(o)[:, : Sq - Skv] == 0.0)
        assert np.allclose(ln, sk.double().numpy()[None, :, None], rtol=0, atol=1e-6)


DECODE = [
    # B, Sq, Hq, Hkv, D, page_size, max_len, len range, chunk, window, modifiers
    (4, 1, 32, 8, 128, 16, 2048, (1, 2048), 256, 0, "all"),
    (3, 1, 8, 2, 64, 0, 1024, (1, 1024), 128, 0, "sinks"),
    (2, 8, 64, 8, 128, 16, 1024, (8, 1024), 256, 0, "alibi"),
    (2, 8, 16, 8, 128, 16, 768, (300, 768), 96, 100, "softcap"),
    (2, 4, 8, 2, 256, 32, 512, (4, 512), 128, 0, "all"),
    (2, 3, 8, 4, 512, 16, 512, (3, 512), 160, 0, "all"),
    (2, 2, 4, 1, 64, 64, 256, (0, 256), 64, 0, "sinks"),        # zero-length sequences possible
    (40, 2, 8, 4, 128, 16, 4096, (1, 4096), 32, 0, "all"),      # several ranges per workgroup set
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B{}_Sq{}_H{}x{}_D{}_ps{}_L{}_{}_c{}_w{}_{}".format(*c))
def test_decode_mods(case):
    B, Sq, Hq, Hkv, D, ps, max_len, (lo, hi), chunk, window, mods = case
    print(f"decode mods {case}", flush=True)
    shape = workloads.DecodeShape("mods", B=B, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, max_len=max_len,
                                  len_lo=lo, len_hi=hi, kv_chunk=chunk, window=window,
                                  seed=B * 31 + D + Sq)
    di = workloads.decode_inputs(shape, poison_tail=True)
    kw, sk = _kw(mods, Hq, 5 + D, DEV)
    table = None if di.block_table is None else di.block_table.to(DEV)
    o, lse = fa.decode_paged(di.q.to(DEV), di.kcache.to(DEV), di.vcache.to(DEV), table, di.seq_lens.to(DEV),
                             page_size=ps or 16, kv_chunk=chunk, causal=True, window=window,
                             scale=shape.scale, **kw)
    torch.cuda.synchronize()
    rkw = dict(kw)
    if sk is not None:
        rkw["sinks"] = sk.double().numpy()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, di.kcache, di.vcache, di.block_table, di.seq_lens,
                                             page_size=ps or 16, causal=True, window=window,
                                             scale=shape.scale, **rkw)
    assert_parity(o, lse, o_ref, lse_ref, f"decode mods {case}")
    if sk is not None:
        lens = di.seq_lens.numpy()
        for b in np.nonzero(lens == 0)[0]:
            assert np.all(to_np(o)[b] == 0.0)
            assert np.allclose(to_np(lse)[b], sk.double().numpy()[:, None], rtol=0, atol=1e-6)


def test_mods_off_is_plain_kernel():
    """All modifiers at their off values take the plain path bit for bit."""
    q, k, v = workloads.random_inputs(1, 100, 100, 8, 2, 128, seed=12)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fa.prefill(q, k, v, causal=True)
    o2, l2 = fa.prefill(q, k, v, causal=True, softcap=0.0, max_bias=0.0, sinks=None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_c3_shape_all_mods_sampled():
    """The 1-row decode workload at full size with all three modifiers on:
    sampled rows and heads against the oracle."""
    s = workloads.C3
    di = workloads.decode_inputs(s)
    sk = _sinks(s.Hq, 77)
    kw = dict(softcap=30.0, max_bias=8.0)
    table = None if di.block_table is None else di.block_table.to(DEV)
    o, lse = fa.decode_paged(di.q.to(DEV), di.kcache.to(DEV), di.vcache.to(DEV), table, di.seq_lens.to(DEV),
                             page_size=s.page_size or 16, kv_chunk=s.kv_chunk, causal=s.causal,
                             window=s.window, scale=s.scale, sinks=sk.to(DEV), **kw)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    bs = sorted({0, 1, s.B // 2, s.B - 1})
    heads = sorted({0, 1, s.Hq // 2, s.Hq - 1})
    for b in bs:
        sl = slice(b, b + 1)
        tb = None if di.block_table is None else di.block_table[sl]
        o_ref, lse_ref = oracle.decode_paged_ref(di.q[sl], di.kcache if tb is not None else di.kcache[sl],
                                                 di.vcache if tb is not None else di.vcache[sl], tb,
                                                 di.seq_lens[sl], page_size=s.page_size or 16,
                                                 causal=s.causal, window=s.window, scale=s.scale,
                                                 heads=heads, sinks=sk.double().numpy(), **kw)
        assert_parity(o[sl][:, :, heads], lse[sl][:, heads], o_ref[:, :, heads], lse_ref[:, heads],
                      f"C3 all mods b{b}")


def _mask(B, Sq, n_keys, seed, width=None, hide=True):
    """bf16 additive mask [B, Sq, width] (width a multiple of 4, >= n_keys):
    N(0, 2) values, a band of hidden keys per sequence and one fully hidden
    row in sequence 0."""
    g = torch.Generator().manual_seed(seed)
    w = width or (n_keys + 3) // 4 * 4
    m = (2.0 * torch.randn(B, Sq, w, generator=g))
    if hide:
        for b in range(B):
            lo = int(torch.randint(0, max(n_keys - 8, 1), (1,), generator=g))
            m[b, :, lo:lo + 8] = -float("inf")
        m[0, Sq // 2, :] = -float("inf")
    return m.to(torch.bfloat16)


MASK_PREFILL = [
    # B, Sq, Skv, Hq, Hkv, D, causal, window, other modifiers, broadcast
    (2, 130, 130, 8, 2, 128, True, 0, None, False),
    (2, 64, 200, 8, 4, 64, False, 0, None, True),
    (1, 100, 100, 4, 2, 256, True, 40, "all", False),
    (1, 77, 77, 4, 2, 512, True, 0, "softcap", False),
]


@pytest.mark.parametrize("case", MASK_PREFILL, ids=lambda c: "B{}_S{}x{}_H{}x{}_D{}_c{}_w{}_{}_bc{}".format(*c))
def test_prefill_mask(case):
    B, Sq, Skv, Hq, Hkv, D, causal, window, other, bcast = case
    print(f"prefill mask {case}", flush=True)
    q, k, v = workloads.random_inputs(B, Sq, Skv, Hq, Hkv, D, seed=Skv + D)
    scale = 1.0 / np.sqrt(D)
    kw, sk = _kw(other, Hq, 3, DEV) if other else ({}, None)
    m = _mask(1 if bcast else B, Sq, Skv, seed=Sq + D, width=(Skv + 3) // 4 * 4 + 8)
    mdev = m.to(DEV)[:, :, 4:Skv + 4]            # a strided view: row stride = width
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, scale=scale,
                        mask=mdev, **kw)
    torch.cuda.synchronize()
    rkw = dict(kw)
    if sk is not None:
        rkw["sinks"] = sk.double().numpy()
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=causal, window=window, scale=scale,
                                          mask=m[:, :, 4:Skv + 4], **rkw)
    assert_parity(o, lse, o_ref, lse_ref, f"prefill mask {case}")
    if sk is None:
        # the row the mask hides entirely
        assert torch.all(o[0, Sq // 2] == 0) and torch.all(torch.isneginf(lse[0, :, Sq // 2]))


MASK_DECODE = [
    # B, Sq, Hq, Hkv, D, page_size, max_len, len range, chunk, other modifiers
    (4, 1, 32, 8, 128, 16, 1024, (1, 1024), 256, None),
    (2, 8, 64, 8, 128, 16, 1024, (8, 1024), 256, "all"),
    (3, 4, 8, 2, 64, 0, 512, (4, 512), 64, None),
    (2, 4, 8, 2, 256, 32, 512, (4, 512), 128, "alibi"),
    (2, 3, 8, 4, 512, 16, 256, (3, 256), 96, None),
]


@pytest.mark.parametrize("case", MASK_DECODE, ids=lambda c: "B{}_Sq{}_H{}x{}_D{}_ps{}_L{}_{}_c{}_{}".format(*c))
def test_decode_mask(case):
    B, Sq, Hq, Hkv, D, ps, max_len, (lo, hi), chunk, other = case
    print(f"decode mask {case}", flush=True)
    shape = workloads.DecodeShape("mask", B=B, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, max_len=max_len,
                                  len_lo=lo, len_hi=hi, kv_chunk=chunk, seed=B * 17 + D + Sq)
    di = workloads.decode_inputs(shape, poison_tail=True)
    kw, sk = _kw(other, Hq, 9, DEV) if other else ({}, None)
    m = _mask(B, Sq, max_len, seed=D + Sq, hide=False)
    m[:, :, 5:9] = -float("inf")                 # a band of hidden tokens in every row
    table = None if di.block_table is None else di.block_table.to(DEV)
    o, lse = fa.decode_paged(di.q.to(DEV), di.kcache.to(DEV), di.vcache.to(DEV), table, di.seq_lens.to(DEV),
                             page_size=ps or 16, kv_chunk=chunk, causal=True, scale=shape.scale,
                             mask=m.to(DEV), **kw)
    torch.cuda.synchronize()
    rkw = dict(kw)
    if sk is not None:
        rkw["sinks"] = sk.double().numpy()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, di.kcache, di.vcache, di.block_table, di.seq_lens,
                                             page_size=ps or 16, causal=True, scale=shape.scale, mask=m,
                                             **rkw)
    assert_parity(o, lse, o_ref, lse_ref, f"decode mask {case}")


def test_verify_mask_as_causal():
    """The causal rule written as a mask (in token positions) with causal
    off matches causal on, both against the oracle."""
    shape = workloads.DecodeShape("maskc", B=3, Sq=8, Hq=32, Hkv=4, D=128, page_size=16, max_len=768,
                                  len_lo=8, len_hi=768, kv_chunk=256, seed=123)
    di = workloads.decode_inputs(shape)
    lens = di.seq_lens
    m = torch.zeros(shape.B, shape.Sq, shape.max_len)
    for b in range(shape.B):
        for i in range(shape.Sq):
            m[b, i, int(lens[b]) - shape.Sq + i + 1:] = -float("inf")
    m = m.to(torch.bfloat16)
    args = (di.q.to(DEV), di.kcache.to(DEV), di.vcache.to(DEV), di.block_table.to(DEV), lens.to(DEV))
    o1, l1 = fa.decode_paged(*args, page_size=16, kv_chunk=256, causal=False, mask=m.to(DEV))
    o2, l2 = fa.decode_paged(*args, page_size=16, kv_chunk=256, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, di.kcache, di.vcache, di.block_table, lens, page_size=16,
                                             causal=True, scale=shape.scale)
    assert_parity(o1, l1, o_ref, lse_ref, "verify causal-as-mask")
    assert_parity(o2, l2, o_ref, lse_ref, "verify causal")
