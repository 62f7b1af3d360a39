"""Long contexts through the C ABI, against the fp64 oracle on sampled rows
and heads: decode over a 131,072-token sequence (beside a 70,001-token one,
contiguous and paged caches), and a chunked-prefill shape (256 new query rows
over 65,536 keys, causal, bottom-right aligned) that loops over two thousand
key tiles per block of rows."""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
from tests.gpu_util import DEV, assert_parity, to_np

pytestmark = pytest.mark.gpu


def _randn(gen, shape):
    return torch.randn(shape, generator=gen).to(torch.bfloat16)


@pytest.mark.parametrize("paged", [False, True])
def test_decode_131072_tokens(paged):
    print(f"decode 131072 tokens paged={paged}", flush=True)
    B, Sq, Hq, Hkv, D, ps = 2, 2, 32, 8, 128, 64
    L = 131072
    lens = [L, 70001]
    g = torch.Generator().manual_seed(1311 + int(paged))
    q = _randn(g, (B, Sq, Hq, D))
    kc = _randn(g, (B, L, Hkv, D))
    vc = _randn(g, (B, L, Hkv, D))
    lens_t = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    if paged:
        mp = L // ps
        table = torch.randperm(B * mp, generator=g).reshape(B, mp).to(torch.int32)
        inv = torch.empty(B * mp, dtype=torch.long)
        inv[table.reshape(-1).long()] = torch.arange(B * mp)
        kp = kc.reshape(B * mp, ps, Hkv, D)[inv]        # page table[b, p] holds tokens p*ps .. of sequence b
        vp = vc.reshape(B * mp, ps, Hkv, D)[inv]
        o, lse = fa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens_t.to(DEV),
                                 page_size=ps, kv_chunk=256, causal=True, scale=scale)
        del kp, vp
    else:
        o, lse = fa.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), None, lens_t.to(DEV), page_size=ps,
                                 kv_chunk=256, causal=True, scale=scale)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    heads = [0, 7, 16, 31]
    for b in range(B):
        n = lens[b]
        o_ref, lse_ref = oracle.attention_ref(q[b:b + 1], kc[b:b + 1, :n], vc[b:b + 1, :n], causal=True,
                                              scale=scale, heads=heads)
        assert_parity(o[b:b + 1][:, :, heads], lse[b:b + 1][:, heads], o_ref[:, :, heads], lse_ref[:, heads],
                      f"decode {n} tokens paged={paged}")


def test_prefill_256_rows_over_65536_keys():
    print("prefill 256 x 65536", flush=True)
    B, Sq, Skv, Hq, Hkv, D = 1, 256, 65536, 8, 2, 128
    g = torch.Generator().manual_seed(1701)
    q, k, v = _randn(g, (B, Sq, Hq, D)), _randn(g, (B, Skv, Hkv, D)), _randn(g, (B, Skv, Hkv, D))
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 254, 255]
    heads = [0, 3, 4, 7]
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=True, scale=scale, rows=rows, heads=heads)
    og, lg = to_np(o)[:, rows][:, :, heads], to_np(lse)[:, heads][:, :, rows]
    assert_parity(og, lg, o_ref[:, rows][:, :, heads], lse_ref[:, heads][:, :, rows], "prefill 256 x 65536")
