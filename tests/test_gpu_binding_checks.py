"""The Python binding checks every tensor's shape, dtype and device against
the call before anything is launched (the C ABI sees only pointers, so a
short buffer would otherwise be read or written out of bounds). Each case
here must raise ValueError or TypeError; no kernel runs."""

import pytest
import torch

import gqa_flash_attention_amd as fa
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

B, Sq, Hq, Hkv, D, PS = 2, 4, 8, 2, 64, 16


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device=DEV)


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device=DEV)


def _decode_args():
    q = _bf(B, Sq, Hq, D)
    kc = _bf(6, PS, Hkv, D)
    vc = _bf(6, PS, Hkv, D)
    table = _i32(B, 3)
    lens = torch.full((B,), 20, dtype=torch.int32, device=DEV)
    return q, kc, vc, table, lens


def test_decode_rejects_wrong_seq_lens_and_table():
    q, kc, vc, table, lens = _decode_args()
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, table, lens[:1], page_size=PS)
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, table[:1], lens, page_size=PS)
    with pytest.raises(TypeError):
        fa.decode_paged(q, kc, vc, table, lens.to(torch.int64), page_size=PS)


def test_decode_rejects_short_contiguous_cache():
    q, _, _, _, lens = _decode_args()
    kc = _bf(B - 1, 64, Hkv, D)
    vc = _bf(B - 1, 64, Hkv, D)
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, None, lens, page_size=PS)


def test_decode_rejects_bad_out_lse_workspace():
    q, kc, vc, table, lens = _decode_args()
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, table, lens, page_size=PS, lse=torch.zeros(B, Hq, Sq + 1, device=DEV))
    with pytest.raises(TypeError):
        fa.decode_paged(q, kc, vc, table, lens, page_size=PS,
                        lse=torch.zeros(B, Hq, Sq, dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, table, lens, page_size=PS, out=_bf(B, Sq, Hq, D + 8))
    need = fa.decode_workspace_bytes(B, Sq, Hq, D, 3 * PS, 256)
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, table, lens, page_size=PS,
                        workspace=torch.empty(need - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, table, lens, page_size=PS,
                        workspace=torch.empty(need, dtype=torch.uint8))


def test_prefill_rejects_bad_lse():
    q, k, v = _bf(1, 16, Hq, D), _bf(1, 16, Hkv, D), _bf(1, 16, Hkv, D)
    with pytest.raises(ValueError):
        fa.prefill(q, k, v, lse=torch.zeros(1, Hq, 15, device=DEV))


def test_append_rejects_short_cache_and_lengths():
    knew, vnew = _bf(B, 2, Hkv, D), _bf(B, 2, Hkv, D)
    lens = _i32(B)
    with pytest.raises(ValueError):
        fa.kv_append(_bf(B - 1, 32, Hkv, D), _bf(B - 1, 32, Hkv, D), None, lens, knew, vnew, page_size=PS)
    with pytest.raises(ValueError):
        fa.kv_append(_bf(B, 32, Hkv, D), _bf(B, 32, Hkv, D), None, lens[:1], knew, vnew, page_size=PS)
    with pytest.raises(ValueError):
        fa.kv_append(_bf(6, PS, Hkv, D), _bf(6, PS, Hkv, D), _i32(B + 1, 3), lens, knew, vnew, page_size=PS)


def test_combine_rejects_mismatched_partials():
    o_part = torch.zeros(B, Hq, Sq, 5, D, device=DEV)
    with pytest.raises(ValueError):
        fa.combine_lse(o_part, torch.zeros(B, Hq, Sq, 4, device=DEV))
    with pytest.raises(ValueError):
        fa.combine_lse(o_part, torch.zeros(B, Hq, Sq, 5, device=DEV), _i32(B + 1))
    with pytest.raises(ValueError):
        fa.combine_lse(o_part, torch.zeros(B, Hq, Sq, 5, device=DEV), out=_bf(B, Sq, Hq, D // 2))


def test_gather_rejects_bad_out():
    cache = _bf(6, PS, Hkv, D)
    table, lens = _i32(B, 3), _i32(B)
    with pytest.raises(ValueError):
        fa.paged_gather(cache, table, lens, out=_bf(B, 3 * PS - 1, Hkv, D))
    with pytest.raises(ValueError):
        fa.paged_gather(cache, table, lens[:1])
