"""The oracle against torch's fp64 CPU scaled_dot_product_attention with an
explicit boolean mask and repeated KV heads (a library special case), and
against invariants of the definition."""

import numpy as np
import pytest
import torch

import oracle

CASES = [
    # B, Sq, Skv, Hq, Hkv, D, causal, window
    (2, 33, 33, 8, 2, 16, True, 0),
    (1, 17, 50, 4, 4, 32, True, 0),
    (1, 40, 40, 6, 3, 8, True, 7),
    (2, 9, 21, 4, 1, 16, False, 0),
    (1, 64, 64, 2, 1, 64, True, 1),
]


def _mask(Sq, Skv, causal, window):
    # written independently of the oracle: bottom-right causal band
    m = torch.ones(Sq, Skv, dtype=torch.bool)
    for i in range(Sq):
        pos = i + Skv - Sq
        for j in range(Skv):
            if causal and j > pos:
                m[i, j] = False
            if causal and window > 0 and pos - j >= window:
                m[i, j] = False
    return m


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_torch_sdpa_fp64(case):
    B, Sq, Skv, Hq, Hkv, D, causal, window = case
    g = torch.Generator().manual_seed(11)
    q = torch.randn(B, Sq, Hq, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, Skv, Hkv, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, Skv, Hkv, D, generator=g, dtype=torch.float64)
    scale = 1.0 / np.sqrt(D)
    o, lse = oracle.attention_ref(q, k, v, causal=causal, window=window, scale=scale)
    G = Hq // Hkv
    qt = q.permute(0, 2, 1, 3)                                   # B, Hq, Sq, D
    kt = k.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = v.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    m = _mask(Sq, Skv, causal, window)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    rows_ok = m.any(dim=1).numpy()
    np.testing.assert_allclose(o[:, rows_ok], ref[:, rows_ok], rtol=0, atol=1e-12)
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~m, float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    np.testing.assert_allclose(lse[:, :, rows_ok], ref_lse[:, :, rows_ok], rtol=0, atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv():
    r = np.random.default_rng(12)
    q = r.standard_normal((2, 11, 8, 16))
    k = r.standard_normal((2, 19, 2, 16))
    v = r.standard_normal((2, 19, 2, 16))
    o1, l1 = oracle.attention_ref(q, k, v, causal=True, scale=0.25)
    o2, l2 = oracle.attention_ref(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), causal=True, scale=0.25)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_key_permutation_invariance_without_mask():
    r = np.random.default_rng(13)
    q = r.standard_normal((1, 5, 2, 8))
    k = r.standard_normal((1, 23, 1, 8))
    v = r.standard_normal((1, 23, 1, 8))
    p = r.permutation(23)
    o1, l1 = oracle.attention_ref(q, k, v, causal=False, scale=0.5)
    o2, l2 = oracle.attention_ref(q, k[:, p], v[:, p], causal=False, scale=0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_window_at_least_skv_is_no_window():
    r = np.random.default_rng(14)
    q = r.standard_normal((1, 12, 2, 8))
    k = r.standard_normal((1, 12, 1, 8))
    v = r.standard_normal((1, 12, 1, 8))
    o1, l1 = oracle.attention_ref(q, k, v, causal=True, window=12, scale=0.5)
    o2, l2 = oracle.attention_ref(q, k, v, causal=True, window=0, scale=0.5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    o3, _ = oracle.attention_ref(q, k, v, causal=True, window=11, scale=0.5)
    assert not np.allclose(o3[0, -1], o2[0, -1])      # window 11 drops key 0 from the last row


def test_decode_and_verify_equal_last_prefill_rows():
    r = np.random.default_rng(15)
    q = r.standard_normal((2, 30, 4, 8))
    k = r.standard_normal((2, 30, 2, 8))
    v = r.standard_normal((2, 30, 2, 8))
    o, l = oracle.attention_ref(q, k, v, causal=True, scale=0.5)
    for R in (1, 8):
        od, ld = oracle.decode_paged_ref(q[:, -R:], k, v, None, [30, 30], page_size=0, causal=True, scale=0.5)
        np.testing.assert_allclose(od, o[:, -R:], atol=1e-13)
        np.testing.assert_allclose(ld, l[:, :, -R:], atol=1e-13)
