"""Strided views and the KV-cache append through the C ABI.

Strided calls must be bitwise equal to the same calls on contiguous copies
(the kernels do the same arithmetic in the same order; only addresses
differ): q, k and v cut from one fused QKV tensor, outputs written into a
slice of a larger buffer, K and V interleaved in one paged allocation. The
append must match the oracle's index map byte for byte, and an append
followed by a verify call must match the oracle on the appended cache."""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
import workloads
from tests.gpu_util import DEV, assert_parity

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("D,Hq,Hkv,S,causal,window", [
    (64, 8, 2, 77, True, 0), (128, 8, 2, 130, True, 33), (256, 4, 2, 70, True, 0),
    (512, 4, 2, 40, False, 0), (128, 4, 4, 96, True, 0),
])
def test_prefill_strided_views_bitwise(D, Hq, Hkv, S, causal, window):
    print(f"prefill views D{D} Hq{Hq} Hkv{Hkv} S{S}", flush=True)
    gen = torch.Generator().manual_seed(D + S)
    B = 2
    qkv = torch.randn(B, S, Hq + 2 * Hkv, D, generator=gen).to(torch.bfloat16).to(DEV)
    q, k, v = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:]
    big = torch.zeros(B, S, Hq + 3, D, dtype=torch.bfloat16, device=DEV)
    o_view = big[:, :, 1:Hq + 1]
    o1, l1 = fa.prefill(q, k, v, causal=causal, window=window, out=o_view)
    o2, l2 = fa.prefill(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal, window=window)
    torch.cuda.synchronize()
    assert o1.data_ptr() == o_view.data_ptr()
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(l1), _bits(l2))
    # the rest of the output buffer is untouched
    assert torch.count_nonzero(big[:, :, 0]) == 0 and torch.count_nonzero(big[:, :, Hq + 1:]) == 0


@pytest.mark.parametrize("D,Sq,paged", [(128, 1, True), (128, 8, True), (64, 4, False), (256, 2, True)])
def test_decode_strided_views_bitwise(D, Sq, paged):
    print(f"decode views D{D} Sq{Sq} paged{paged}", flush=True)
    shape = workloads.DecodeShape("views", B=3, Sq=Sq, Hq=16, Hkv=4, D=D, page_size=16 if paged else 0,
                                  max_len=512, len_lo=Sq, len_hi=512, kv_chunk=128, seed=40 + D + Sq)
    di = workloads.decode_inputs(shape)
    kc, vc = di.kcache, di.vcache
    # K and V interleaved in one allocation: [.., 2, Hkv, D] per token slot
    kv = torch.stack([kc, vc], dim=2).to(DEV)
    k_view, v_view = kv[:, :, 0], kv[:, :, 1]
    qbig = torch.zeros(shape.B, Sq, shape.Hq + 2, D, dtype=torch.bfloat16)
    qbig[:, :, 2:] = di.q
    q_view = qbig.to(DEV)[:, :, 2:]
    table = None if di.block_table is None else di.block_table.to(DEV)
    lens = di.seq_lens.to(DEV)
    obig = torch.zeros(shape.B, Sq, 2 * shape.Hq, D, dtype=torch.bfloat16, device=DEV)
    o_view = obig[:, :, ::2]     # head stride 2 D
    o1, l1 = fa.decode_paged(q_view, k_view, v_view, table, lens, page_size=16, kv_chunk=shape.kv_chunk,
                             out=o_view)
    o2, l2 = fa.decode_paged(di.q.to(DEV), kc.to(DEV), vc.to(DEV), table, lens, page_size=16,
                             kv_chunk=shape.kv_chunk)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1.contiguous()), _bits(o2)) and torch.equal(_bits(l1), _bits(l2))
    assert torch.count_nonzero(obig[:, :, 1::2]) == 0


def _append_case(paged, seed):
    gen = torch.Generator().manual_seed(seed)
    B, Snew, Hkv, D, ps, mp = 4, 8, 2, 128, 16, 12
    if paged:
        P = B * mp + 5
        table = torch.randperm(P, generator=gen)[: B * mp].reshape(B, mp).to(torch.int32)
        table[1, 3] = P + 7                  # out of range: rows on sequence 1's page 3 are skipped
        kc = torch.randn(P, ps, Hkv, D, generator=gen).to(torch.bfloat16)
    else:
        table = None
        kc = torch.randn(B, mp * ps, Hkv, D, generator=gen).to(torch.bfloat16)
    vc = torch.randn(kc.shape, generator=gen).to(torch.bfloat16)
    # full cache; new rows of sequence 1 at tokens 58..65 (pages 3 and 4);
    # a sequence shorter than Snew; an interior length
    lens = torch.tensor([mp * ps, 4 * ps + 2, 3, 100], dtype=torch.int32)
    kn = torch.randn(B, Snew, Hkv, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, Snew, Hkv, D, generator=gen).to(torch.bfloat16)
    return table, kc, vc, lens, kn, vn, ps


@pytest.mark.parametrize("paged", [True, False])
def test_kv_append_bitexact(paged):
    print(f"kv append paged={paged}", flush=True)
    table, kc, vc, lens, kn, vn, ps = _append_case(paged, 11 + int(paged))
    kc_ref, vc_ref = oracle.kv_append_ref(kc, vc, table, lens, kn, vn, page_size=ps)
    # new rows as views of one fused [B, Snew, 2, Hkv, D] tensor
    fused = torch.stack([kn, vn], dim=2).to(DEV)
    kd, vd = kc.to(DEV), vc.to(DEV)
    fa.kv_append(kd, vd, None if table is None else table.to(DEV), lens.to(DEV), fused[:, :, 0],
                 fused[:, :, 1], page_size=ps)
    torch.cuda.synchronize()
    assert torch.equal(_bits(kd.cpu()), _bits(kc_ref)) and torch.equal(_bits(vd.cpu()), _bits(vc_ref))


def test_append_then_verify():
    """The step before a verify call: append 8 draft rows, then attend."""
    print("append then verify", flush=True)
    gen = torch.Generator().manual_seed(99)
    B, Sq, Hq, Hkv, D, ps, mp = 2, 8, 32, 4, 128, 16, 40
    P = B * mp
    table = torch.randperm(P, generator=gen).reshape(B, mp).to(torch.int32)
    kc = torch.randn(P, ps, Hkv, D, generator=gen).to(torch.bfloat16)
    vc = torch.randn(P, ps, Hkv, D, generator=gen).to(torch.bfloat16)
    lens = torch.tensor([mp * ps - 5, 301], dtype=torch.int32)
    kn = torch.randn(B, Sq, Hkv, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, Sq, Hkv, D, generator=gen).to(torch.bfloat16)
    q = torch.randn(B, Sq, Hq, D, generator=gen).to(torch.bfloat16)
    kd, vd = kc.to(DEV), vc.to(DEV)
    fa.kv_append(kd, vd, table.to(DEV), lens.to(DEV), kn.to(DEV), vn.to(DEV), page_size=ps)
    o, lse = fa.decode_paged(q.to(DEV), kd, vd, table.to(DEV), lens.to(DEV), page_size=ps, kv_chunk=256)
    torch.cuda.synchronize()
    kc2, vc2 = oracle.kv_append_ref(kc, vc, table, lens, kn, vn, page_size=ps)
    o_ref, lse_ref = oracle.decode_paged_ref(q, kc2, vc2, table, lens, page_size=ps, causal=True,
                                             scale=1.0 / np.sqrt(D))
    assert_parity(o, lse, o_ref, lse_ref, "append + verify")
