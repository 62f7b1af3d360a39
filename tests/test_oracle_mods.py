"""Pins of the oracle's score modifiers (CPU): logit softcap, ALiBi slopes
from max_bias, attention sinks and the additive mask tensor; and of key and
value head dims that differ (any multiple of 8 up to 512). Each pin is independent of the oracle's
own formula: published slope values, hand-derived closed forms, limits,
torch's fp64 scaled_dot_product_attention with an explicit additive bias,
and a pure-Python brute force."""

import math
import random

import numpy as np
import torch

import oracle


def check_alibi_slopes_published_values(orc):
    # 8 heads, max_bias 8: the geometric sequence 1/2, 1/4, ..., 1/256
    assert np.allclose(orc.alibi_slopes(8, 8.0), [2.0 ** -(h + 1) for h in range(8)], rtol=0, atol=0)
    # 12 heads: the first 8 as above, then odd powers of 2^-1/2
    want = [2.0 ** -(h + 1) for h in range(8)] + [2.0 ** -0.5, 2.0 ** -1.5, 2.0 ** -2.5, 2.0 ** -3.5]
    assert np.allclose(orc.alibi_slopes(12, 8.0), want, rtol=1e-15, atol=0)
    assert not np.any(orc.alibi_slopes(4, 0.0))


def _one_head(q, k, v):
    """[S, D] arrays -> [1, S, 1, D] float64 tensors."""
    f = lambda a: np.asarray(a, dtype=np.float64)[None, :, None, :]
    return f(q), f(k), f(v)


def check_sink_single_key_closed_form(orc):
    # q . k = 2, scale 0.5 -> s = 1; sink 0.3
    q, k, v = _one_head([[1.0, 1.0]], [[1.0, 1.0]], [[3.0, -4.0]])
    o, lse = orc.attention_ref(q, k, v, causal=True, scale=0.5, sinks=[0.3])
    w = math.exp(1.0) / (math.exp(1.0) + math.exp(0.3))
    assert np.allclose(o[0, 0, 0], [3.0 * w, -4.0 * w], rtol=1e-14, atol=0)
    assert abs(lse[0, 0, 0] - math.log(math.exp(1.0) + math.exp(0.3))) < 1e-14


def check_sink_limits_and_empty_row(orc):
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((1, 5, 2, 8)), rng.standard_normal((1, 7, 1, 8)), rng.standard_normal((1, 7, 1, 8))
    o0, l0 = orc.attention_ref(q, k, v, causal=True, scale=0.3)
    o1, l1 = orc.attention_ref(q, k, v, causal=True, scale=0.3, sinks=[-np.inf, -np.inf])
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # Sq > Skv: the first rows see no key; with a sink, O = 0 and LSE = sink
    q2 = rng.standard_normal((1, 9, 1, 8))
    o2, l2 = orc.attention_ref(q2, k, v, causal=True, scale=0.3, sinks=[0.7])
    assert np.all(o2[0, :2, 0] == 0.0) and np.all(l2[0, 0, :2] == 0.7)


def check_softcap_closed_forms(orc):
    # one visible key: O = V, LSE = c tanh(s / c)
    q, k, v = _one_head([[2.0, 0.0]], [[3.0, 0.0]], [[1.5, 2.5]])
    o, lse = orc.attention_ref(q, k, v, causal=True, scale=1.0, softcap=4.0)
    assert np.allclose(o[0, 0, 0], [1.5, 2.5], rtol=0, atol=0)
    assert abs(lse[0, 0, 0] - 4.0 * math.tanh(6.0 / 4.0)) < 1e-14
    # two keys: logistic weights of the capped score difference
    q, k, v = _one_head([[1.0, 0.0], [1.0, 0.0]], [[5.0, 0.0], [-2.0, 0.0]], [[1.0, 0.0], [0.0, 1.0]])
    o, _ = orc.attention_ref(q, k, v, causal=True, scale=1.0, softcap=3.0)
    a, b = 3.0 * math.tanh(5.0 / 3.0), 3.0 * math.tanh(-2.0 / 3.0)
    w0 = 1.0 / (1.0 + math.exp(b - a))
    assert np.allclose(o[0, 1, 0], [w0, 1.0 - w0], rtol=1e-14, atol=1e-15)


def check_softcap_large_cap_is_plain(orc):
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((2, 6, 4, 16)), rng.standard_normal((2, 6, 2, 16)), rng.standard_normal((2, 6, 2, 16))
    o0, l0 = orc.attention_ref(q, k, v, causal=True, scale=0.25)
    o1, l1 = orc.attention_ref(q, k, v, causal=True, scale=0.25, softcap=1e7)
    assert np.allclose(o0, o1, rtol=0, atol=1e-10) and np.allclose(l0, l1, rtol=0, atol=1e-10)


def check_alibi_against_torch_sdpa(orc):
    torch.manual_seed(2)
    B, Sq, Skv, Hq, Hkv, D, scale, mb = 2, 5, 11, 6, 3, 8, 0.35, 8.0
    q, k, v = torch.randn(B, Sq, Hq, D, dtype=torch.float64), torch.randn(B, Skv, Hkv, D, dtype=torch.float64), \
        torch.randn(B, Skv, Hkv, D, dtype=torch.float64)
    o, lse = orc.attention_ref(q, k, v, causal=True, window=6, scale=scale, max_bias=mb)
    # library path: explicit additive mask (bias and -inf), repeated KV heads
    n = 1 << int(math.floor(math.log2(Hq)))
    slopes = [2.0 ** (-mb / n * (h + 1)) if h < n else 2.0 ** (-mb / (2 * n) * (2 * (h - n) + 1)) for h in range(Hq)]
    pos = torch.arange(Sq)[:, None] + (Skv - Sq)
    j = torch.arange(Skv)[None, :]
    vis = (j <= pos) & (pos - j < 6)
    kk = k.repeat_interleave(Hq // Hkv, dim=2).permute(0, 2, 1, 3)
    vv = v.repeat_interleave(Hq // Hkv, dim=2).permute(0, 2, 1, 3)
    qq = q.permute(0, 2, 1, 3)
    bias = torch.stack([s * (j - pos).double() for s in slopes])[None]            # [1, Hq, Sq, Skv]
    mask = torch.where(vis, bias, torch.tensor(-math.inf, dtype=torch.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    logits = scale * (qq @ kk.transpose(-1, -2)) + mask
    assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
    assert np.allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


def _brute(q, k, v, causal, window, scale, softcap, mb, sinks, mask=None):
    """Pure-Python loops, no max subtraction: the definition written out."""
    B, Sq, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Skv, Hkv = len(k[0]), len(k[0][0])
    if mb > 0:
        n = 1 << int(math.floor(math.log2(Hq)))
        slopes = [2.0 ** (-mb / n * (h + 1)) if h < n else 2.0 ** (-mb / (2 * n) * (2 * (h - n) + 1))
                  for h in range(Hq)]
    else:
        slopes = [0.0] * Hq
    out, lses = [], []
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                g, p = h // (Hq // Hkv), i + Skv - Sq
                num, den = [0.0] * D, 0.0
                for jj in range(Skv):
                    if causal and (jj > p or (window > 0 and p - jj >= window)):
                        continue
                    s = scale * sum(q[b][i][h][d] * k[b][jj][g][d] for d in range(D))
                    if softcap > 0:
                        s = softcap * math.tanh(s / softcap)
                    s += slopes[h] * (jj - p)
                    if mask is not None:
                        s += mask[b if len(mask) > 1 else 0][i][jj]
                    if s == -math.inf:
                        continue
                    e = math.exp(s)
                    den += e
                    for d in range(D):
                        num[d] += e * v[b][jj][g][d]
                if sinks is not None:
                    den += math.exp(sinks[h])
                out.append(([x / den for x in num] if den > 0 else [0.0] * D, (b, i, h)))
                lses.append((math.log(den) if den > 0 else -math.inf, (b, h, i)))
    return out, lses


def check_brute_force_all_modifiers(orc):
    rng = random.Random(4)
    for trial in range(16):
        B, Sq, Skv, Hkv, G, D = 1, rng.randint(1, 4), rng.randint(1, 6), rng.randint(1, 2), rng.randint(1, 3), 3
        Hq = Hkv * G
        mk = lambda *sh: np.array([rng.gauss(0, 1) for _ in range(int(np.prod(sh)))]).reshape(sh)
        q, k, v = mk(B, Sq, Hq, D), mk(B, Skv, Hkv, D), mk(B, Skv, Hkv, D)
        causal = rng.random() < 0.7
        window = rng.choice([0, 2]) if causal else 0
        softcap = rng.choice([0.0, 1.5])
        mb = rng.choice([0.0, 4.0])
        sinks = [rng.gauss(0, 1) for _ in range(Hq)] if rng.random() < 0.5 else None
        mask = None
        if trial % 2 == 1:
            mask = mk(B, Sq, Skv)
            for _ in range(2):
                mask[0, rng.randrange(Sq), rng.randrange(Skv)] = -math.inf
        o, lse = orc.attention_ref(q, k, v, causal=causal, window=window, scale=0.6, softcap=softcap,
                                      max_bias=mb, sinks=sinks, mask=mask)
        bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), causal, window, 0.6, softcap, mb, sinks,
                        None if mask is None else mask.tolist())
        for vec, (b, i, h) in bo:
            assert np.allclose(o[b, i, h], vec, rtol=1e-12, atol=1e-12), trial
        for val, (b, h, i) in bl:
            assert (val == -math.inf and lse[b, h, i] == -np.inf) or abs(lse[b, h, i] - val) < 1e-12, trial


def check_split_combine_with_sinks_equals_whole(orc):
    rng = np.random.default_rng(6)
    B, Sq, Skv, Hq, Hkv, D = 2, 3, 40, 4, 2, 8
    q, k, v = rng.standard_normal((B, Sq, Hq, D)), rng.standard_normal((B, Skv, Hkv, D)), rng.standard_normal((B, Skv, Hkv, D))
    sinks = rng.standard_normal(Hq)
    lens = [40, 17]
    o, lse = orc.attention_ref(q, k, v, causal=True, scale=0.4, seq_lens=lens, sinks=sinks)
    op, lp = orc.partial_attention_ref(q, k, v, causal=True, scale=0.4, seq_lens=lens, chunk=8)
    n = [-(-x // 8) for x in lens]
    oc, lc = orc.combine_ref(op, lp, n, sinks=sinks)
    assert np.allclose(o, oc, rtol=0, atol=1e-12) and np.allclose(lse, lc, rtol=0, atol=1e-12)


def check_mask_hiding_keys_equals_deleting_them(orc):
    rng = np.random.default_rng(8)
    B, Sq, Skv, Hq, Hkv, D = 2, 4, 12, 4, 2, 8
    q, k, v = rng.standard_normal((B, Sq, Hq, D)), rng.standard_normal((B, Skv, Hkv, D)), \
        rng.standard_normal((B, Skv, Hkv, D))
    mask = np.zeros((B, Sq, Skv))
    keep = [np.r_[0:3, 7:12], np.r_[2:12]]
    mask[0, :, 3:7] = -np.inf
    mask[1, :, 0:2] = -np.inf
    o, lse = orc.attention_ref(q, k, v, causal=False, scale=0.4, mask=mask)
    for b in range(B):
        ob, lb = orc.attention_ref(q[b:b + 1], k[b:b + 1, keep[b]], v[b:b + 1, keep[b]], causal=False, scale=0.4)
        assert np.allclose(o[b], ob[0], rtol=0, atol=1e-13) and np.allclose(lse[b], lb[0], rtol=0, atol=1e-13)


def check_mask_against_torch_sdpa(orc):
    torch.manual_seed(9)
    B, Sq, Skv, Hq, Hkv, D, scale = 2, 6, 13, 6, 2, 8, 0.3
    q, k, v = torch.randn(B, Sq, Hq, D, dtype=torch.float64), torch.randn(B, Skv, Hkv, D, dtype=torch.float64), \
        torch.randn(B, Skv, Hkv, D, dtype=torch.float64)
    m = 3.0 * torch.randn(B, Sq, Skv, dtype=torch.float64)
    m[0, 2, 4] = -math.inf
    m[1, 5, 0:5] = -math.inf
    o, lse = orc.attention_ref(q, k, v, causal=True, window=9, scale=scale, mask=m.numpy())
    pos = torch.arange(Sq)[:, None] + (Skv - Sq)
    j = torch.arange(Skv)[None, :]
    vis = (j <= pos) & (pos - j < 9)
    full = torch.where(vis[None], m, torch.tensor(-math.inf, dtype=torch.float64))[:, None]   # [B, 1, Sq, Skv]
    kk = k.repeat_interleave(Hq // Hkv, dim=2).permute(0, 2, 1, 3)
    vv = v.repeat_interleave(Hq // Hkv, dim=2).permute(0, 2, 1, 3)
    qq = q.permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=full, scale=scale)
    logits = scale * (qq @ kk.transpose(-1, -2)) + full
    assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
    assert np.allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


def check_mask_as_causal_and_broadcast(orc):
    rng = np.random.default_rng(10)
    B, Sq, Hq, Hkv, D, ps = 3, 4, 4, 2, 8, 4
    lens = [13, 4, 9]
    P = 12
    table = rng.permutation(P).reshape(B, 4)
    kc, vc = rng.standard_normal((P, ps, Hkv, D)), rng.standard_normal((P, ps, Hkv, D))
    q = rng.standard_normal((B, Sq, Hq, D))
    # -inf wherever the key lies after the row's position: the causal rule
    # written as a mask, in token coordinates
    M = 16
    mask = np.zeros((B, Sq, M))
    for b in range(B):
        for i in range(Sq):
            mask[b, i, lens[b] - Sq + i + 1:] = -np.inf
    o1, l1 = orc.decode_paged_ref(q, kc, vc, table, lens, page_size=ps, causal=False, scale=0.5, mask=mask)
    o2, l2 = orc.decode_paged_ref(q, kc, vc, table, lens, page_size=ps, causal=True, scale=0.5)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)
    # one [1, Sq, M] mask shared by every sequence equals it repeated
    shared = rng.standard_normal((1, Sq, M))
    o3, l3 = orc.decode_paged_ref(q, kc, vc, table, lens, page_size=ps, causal=True, scale=0.5, mask=shared)
    o4, l4 = orc.decode_paged_ref(q, kc, vc, table, lens, page_size=ps, causal=True, scale=0.5,
                                  mask=np.repeat(shared, B, axis=0))
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
    assert not np.allclose(o3, o2)


def check_dk_dv_against_torch_sdpa(orc):
    torch.manual_seed(11)
    for Dk, Dv in ((72, 72), (80, 96), (192, 128), (320, 256), (40, 8)):
        B, Sq, Skv, Hq, Hkv, scale = 2, 5, 9, 4, 2, 1.0 / math.sqrt(Dk)
        q = torch.randn(B, Sq, Hq, Dk, dtype=torch.float64)
        k = torch.randn(B, Skv, Hkv, Dk, dtype=torch.float64)
        v = torch.randn(B, Skv, Hkv, Dv, dtype=torch.float64)
        o, lse = orc.attention_ref(q, k, v, causal=True, window=7, scale=scale)
        assert o.shape == (B, Sq, Hq, Dv)
        pos = torch.arange(Sq)[:, None] + (Skv - Sq)
        j = torch.arange(Skv)[None, :]
        vis = (j <= pos) & (pos - j < 7)
        add = torch.where(vis, torch.tensor(0.0, dtype=torch.float64), torch.tensor(-math.inf, dtype=torch.float64))
        kk = k.repeat_interleave(Hq // Hkv, dim=2).permute(0, 2, 1, 3)
        vv = v.repeat_interleave(Hq // Hkv, dim=2).permute(0, 2, 1, 3)
        qq = q.permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=add, scale=scale)
        assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12), (Dk, Dv)
        lref = torch.logsumexp(scale * (qq @ kk.transpose(-1, -2)) + add, dim=-1)
        assert np.allclose(lse, lref.numpy(), rtol=0, atol=1e-12), (Dk, Dv)


def check_dk_dv_padding_and_column_split(orc):
    rng = np.random.default_rng(12)
    B, Sq, Skv, Hq, Hkv, Dk, Dv = 1, 6, 10, 4, 2, 72, 80
    q, k = rng.standard_normal((B, Sq, Hq, Dk)), rng.standard_normal((B, Skv, Hkv, Dk))
    v = rng.standard_normal((B, Skv, Hkv, Dv))
    o, lse = orc.attention_ref(q, k, v, causal=True, scale=0.2)
    # zero columns appended to Q and K change no score
    zq = np.concatenate([q, np.zeros((B, Sq, Hq, 56))], axis=3)
    zk = np.concatenate([k, np.zeros((B, Skv, Hkv, 56))], axis=3)
    o2, l2 = orc.attention_ref(zq, zk, v, causal=True, scale=0.2)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # the output's columns are those of V: splitting V splits O
    oa, la = orc.attention_ref(q, k, v[..., :24], causal=True, scale=0.2)
    ob, lb = orc.attention_ref(q, k, v[..., 24:], causal=True, scale=0.2)
    assert np.allclose(o, np.concatenate([oa, ob], axis=3), rtol=0, atol=1e-14)
    assert np.array_equal(la, lse) and np.array_equal(lb, lse)


def check_dk_dv_brute_force(orc):
    rng = random.Random(13)
    for trial in range(6):
        Sq, Skv, Hkv, G = rng.randint(1, 3), rng.randint(1, 5), rng.randint(1, 2), rng.randint(1, 2)
        Dk, Dv = rng.choice([(3, 5), (8, 2), (4, 4), (2, 7)])
        Hq = Hkv * G
        mk = lambda *sh: np.array([rng.gauss(0, 1) for _ in range(int(np.prod(sh)))]).reshape(sh)
        q, k, v = mk(1, Sq, Hq, Dk), mk(1, Skv, Hkv, Dk), mk(1, Skv, Hkv, Dv)
        o, lse = orc.attention_ref(q, k, v, causal=True, scale=0.7)
        for i in range(Sq):
            for h in range(Hq):
                g, p = h // G, i + Skv - Sq
                w = [math.exp(0.7 * sum(q[0, i, h, d] * k[0, j, g, d] for d in range(Dk)))
                     for j in range(Skv) if j <= p]
                den = sum(w)
                if den == 0:
                    assert lse[0, h, i] == -np.inf and np.all(o[0, i, h] == 0)
                    continue
                want = [sum(w[j] * v[0, j, g, e] for j in range(len(w))) / den for e in range(Dv)]
                assert np.allclose(o[0, i, h], want, rtol=1e-12, atol=1e-13), trial
                assert abs(lse[0, h, i] - math.log(den)) < 1e-12, trial


MOD_CHECKS = [check_alibi_slopes_published_values, check_sink_single_key_closed_form, check_sink_limits_and_empty_row, check_softcap_closed_forms, check_softcap_large_cap_is_plain, check_alibi_against_torch_sdpa, check_brute_force_all_modifiers, check_split_combine_with_sinks_equals_whole, check_mask_hiding_keys_equals_deleting_them, check_mask_against_torch_sdpa, check_mask_as_causal_and_broadcast, check_dk_dv_against_torch_sdpa, check_dk_dv_padding_and_column_split, check_dk_dv_brute_force]


def test_alibi_slopes_published_values():
    check_alibi_slopes_published_values(oracle)


def test_sink_single_key_closed_form():
    check_sink_single_key_closed_form(oracle)


def test_sink_limits_and_empty_row():
    check_sink_limits_and_empty_row(oracle)


def test_softcap_closed_forms():
    check_softcap_closed_forms(oracle)


def test_softcap_large_cap_is_plain():
    check_softcap_large_cap_is_plain(oracle)


def test_alibi_against_torch_sdpa():
    check_alibi_against_torch_sdpa(oracle)


def test_brute_force_all_modifiers():
    check_brute_force_all_modifiers(oracle)


def test_split_combine_with_sinks_equals_whole():
    check_split_combine_with_sinks_equals_whole(oracle)


def test_mask_hiding_keys_equals_deleting_them():
    check_mask_hiding_keys_equals_deleting_them(oracle)


def test_mask_against_torch_sdpa():
    check_mask_against_torch_sdpa(oracle)


def test_mask_as_causal_and_broadcast():
    check_mask_as_causal_and_broadcast(oracle)


def test_dk_dv_against_torch_sdpa():
    check_dk_dv_against_torch_sdpa(oracle)


def test_dk_dv_padding_and_column_split():
    check_dk_dv_padding_and_column_split(oracle)


def test_dk_dv_brute_force():
    check_dk_dv_brute_force(oracle)
