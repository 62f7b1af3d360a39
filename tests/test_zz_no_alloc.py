"""fa_decode_paged_noalloc (the decode / verify entry point for callers that
cannot allocate: its split partials live in the library's static device
buffer) against fa_decode_paged_strided with a caller workspace, through the
C ABI: two calls in a row, the second smaller, each bitwise equal to the
workspace call and within the parity bar of the fp64 oracle; a call too
large for the buffer is refused before anything runs."""

import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
import workloads
from gqa_flash_attention_amd._lib import NOALLOC_SCRATCH_BYTES
from tests.gpu_util import DEV, assert_parity

pytestmark = pytest.mark.gpu


def _run(shape):
    di = workloads.decode_inputs(shape, poison_tail=True)
    table = None if di.block_table is None else di.block_table.to(DEV)
    args = (di.q.to(DEV), di.kcache.to(DEV), di.vcache.to(DEV), table, di.seq_lens.to(DEV))
    kw = dict(page_size=shape.page_size or 16, kv_chunk=shape.kv_chunk, causal=True, window=shape.window,
              scale=shape.scale)
    o1, l1 = fa.decode_paged_noalloc(*args, **kw)
    o2, l2 = fa.decode_paged(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), shape.name
    o_ref, lse_ref = oracle.decode_paged_ref(di.q, di.kcache, di.vcache, di.block_table, di.seq_lens,
                                             page_size=shape.page_size or 16, causal=True, window=shape.window,
                                             scale=shape.scale)
    assert_parity(o1, l1, o_ref, lse_ref, f"noalloc {shape.name}")


def test_noalloc_matches_workspace_call_twice_then_smaller():
    big = workloads.DecodeShape("noalloc_big", B=4, Sq=8, Hq=64, Hkv=8, D=128, page_size=16, max_len=4096,
                                len_lo=3000, len_hi=4096, kv_chunk=1024, seed=901)
    small = workloads.DecodeShape("noalloc_small", B=3, Sq=1, Hq=16, Hkv=4, D=64, page_size=0, max_len=1024,
                                  len_lo=1, len_hi=1024, kv_chunk=256, seed=902)
    _run(big)
    _run(small)


def test_noalloc_refuses_calls_beyond_its_buffer():
    B, Sq, Hq, Hkv, D = 64, 16, 64, 8, 512
    max_len = 4096
    need = fa.decode_workspace_bytes(B, Sq, Hq, D, max_len, 256)
    assert need > NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, Sq, Hq, D, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(D, dtype=torch.bfloat16, device=DEV).as_strided((B, max_len, Hkv, D), (0, 0, 0, 1))
    lens = torch.full((B,), max_len, dtype=torch.int32, device=DEV)
    with pytest.raises(fa.FAError) as e:
        fa.decode_paged_noalloc(q, kc, kc, None, lens, page_size=16, kv_chunk=256)
    assert e.value.status == -5
