"""Pins for the fp64 oracle that do not go through the oracle's own formula.

Each check takes the oracle module as an argument so the mutation test can
run the same battery against deliberately broken copies of the oracle.
Every check raises AssertionError on a mismatch.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def check_golden(orc):
    """Hand-derived cases with integer-ratio softmax weights."""
    with open(GOLDEN) as f:
        g = json.load(f)
    K = np.array(g["K"])
    V = np.array(g["V"])
    for case in g["cases"]:
        q = np.array(case["q"])[None]                       # [1, Sq, Hq, D]
        Sq = q.shape[1]
        k = np.broadcast_to(K[None, :, None, :], (1, K.shape[0], case["Hkv"], K.shape[1]))
        v = np.broadcast_to(V[None, :, None, :], (1, V.shape[0], case["Hkv"], V.shape[1]))
        o, lse = orc.attention_ref(q, k, v, causal=case["causal"], window=case["window"],
                                   scale=case["scale"])
        assert o.shape == (1, Sq, q.shape[2], 2), case["name"]
        np.testing.assert_allclose(o[0], np.array(case["O"]), rtol=0, atol=TOL, err_msg=case["name"])
        np.testing.assert_allclose(lse[0], np.array(case["LSE"]), rtol=0, atol=TOL, err_msg=case["name"])
    c = g["combine"]
    o_part = np.array(c["O_part"])[None, None, None]          # [1,1,1,C,D]
    lse_part = np.array(c["LSE_part"])[None, None, None]
    o, lse = orc.combine_ref(o_part, lse_part)
    np.testing.assert_allclose(o[0, 0, 0], c["O"], rtol=0, atol=TOL)
    np.testing.assert_allclose(lse[0, 0, 0], c["LSE"], rtol=0, atol=TOL)


def check_single_key(orc):
    """One visible key: O is that key's V row and LSE its score."""
    r = _rng(1)
    q = r.standard_normal((2, 5, 4, 16))
    k = r.standard_normal((2, 1, 2, 16))
    v = r.standard_normal((2, 1, 2, 16))
    o, lse = orc.attention_ref(q, k, v, causal=False, scale=0.3)
    for b in range(2):
        for h in range(4):
            g = h // 2
            np.testing.assert_allclose(o[b, :, h], np.broadcast_to(v[b, 0, g], (5, 16)), atol=TOL)
            np.testing.assert_allclose(lse[b, h], 0.3 * q[b, :, h] @ k[b, 0, g], atol=TOL)
    # causal row 0 (Sq == Skv) sees only key 0; window 1 sees only the diagonal
    q = r.standard_normal((1, 7, 2, 8))
    k = r.standard_normal((1, 7, 1, 8))
    v = r.standard_normal((1, 7, 1, 8))
    o, lse = orc.attention_ref(q, k, v, causal=True, scale=0.5)
    np.testing.assert_allclose(o[0, 0, :, :], np.broadcast_to(v[0, 0, 0], (2, 8)), atol=TOL)
    o, lse = orc.attention_ref(q, k, v, causal=True, window=1, scale=0.5)
    for i in range(7):
        for h in range(2):
            np.testing.assert_allclose(o[0, i, h], v[0, i, 0], atol=TOL)
            np.testing.assert_allclose(lse[0, h, i], 0.5 * q[0, i, h] @ k[0, i, 0], atol=TOL)


def check_constant_v(orc):
    """Constant V rows: every non-empty output row equals that constant."""
    r = _rng(2)
    q = 3.0 * r.standard_normal((1, 9, 4, 8))
    k = 3.0 * r.standard_normal((1, 13, 2, 8))
    c = r.standard_normal(8)
    v = np.broadcast_to(c, (1, 13, 2, 8)).copy()
    for causal, window in ((False, 0), (True, 0), (True, 3)):
        o, _ = orc.attention_ref(q, k, v, causal=causal, window=window, scale=0.7)
        np.testing.assert_allclose(o[0], np.broadcast_to(c, (9, 4, 8)), atol=1e-12)


def check_equal_scores(orc):
    """q = 0 gives equal scores: O is the mean of the visible V rows and
    LSE = ln(number of visible keys). Causal rows give running means; a
    window gives a moving average."""
    r = _rng(3)
    Sq, Skv, w = 6, 10, 4
    q = np.zeros((1, Sq, 2, 8))
    k = r.standard_normal((1, Skv, 1, 8))
    v = r.standard_normal((1, Skv, 1, 8))
    o, lse = orc.attention_ref(q, k, v, causal=False, scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (Sq, 8)), atol=TOL)
    np.testing.assert_allclose(lse[0], math.log(Skv), atol=TOL)
    o, lse = orc.attention_ref(q, k, v, causal=True, scale=1.0)
    for i in range(Sq):
        p = i + Skv - Sq
        np.testing.assert_allclose(o[0, i, 1], v[0, :p + 1, 0].mean(0), atol=TOL)
        np.testing.assert_allclose(lse[0, 1, i], math.log(p + 1), atol=TOL)
    o, lse = orc.attention_ref(q, k, v, causal=True, window=w, scale=1.0)
    for i in range(Sq):
        p = i + Skv - Sq
        lo = max(0, p - w + 1)
        np.testing.assert_allclose(o[0, i, 0], v[0, lo:p + 1, 0].mean(0), atol=TOL)
        np.testing.assert_allclose(lse[0, 0, i], math.log(p + 1 - lo), atol=TOL)


def _sigmoid(x):
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def check_two_keys(orc):
    """Two keys: O = sigma(s0 - s1) v0 + sigma(s1 - s0) v1, LSE = log(e^s0 + e^s1),
    including scores large enough that exp(s) alone would overflow."""
    r = _rng(4)
    for big in (1.0, 400.0):
        q = r.standard_normal((1, 1, 1, 4))
        k = big * r.standard_normal((1, 2, 1, 4))
        v = r.standard_normal((1, 2, 1, 4))
        s = q[0, 0, 0] @ k[0, :, 0].T
        d = s[0] - s[1]
        sig0, sig1 = _sigmoid(d), _sigmoid(-d)
        o, lse = orc.attention_ref(q, k, v, causal=False, scale=1.0)
        np.testing.assert_allclose(o[0, 0, 0], sig0 * v[0, 0, 0] + sig1 * v[0, 1, 0], rtol=1e-12, atol=1e-12)
        hi = max(s[0], s[1])
        want = hi + math.log1p(math.exp(-abs(d)))
        np.testing.assert_allclose(lse[0, 0, 0], want, rtol=1e-13, atol=1e-12)


def check_empty_rows(orc):
    """Rows with no visible key (Sq > Skv under bottom-right causal, or a
    zero-length sequence) give O = 0 and LSE = -inf."""
    r = _rng(5)
    q = r.standard_normal((1, 5, 1, 4))
    k = r.standard_normal((1, 3, 1, 4))
    v = r.standard_normal((1, 3, 1, 4))
    o, lse = orc.attention_ref(q, k, v, causal=True, scale=1.0)
    # rows 0 and 1 are at positions -2 and -1
    assert np.all(o[0, :2] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(np.isfinite(lse[0, 0, 2:]))
    np.testing.assert_allclose(o[0, 2, 0], v[0, 0, 0], atol=TOL)
    o, lse = orc.attention_ref(q, k, v, causal=False, scale=1.0, seq_lens=[0])
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def brute_force(q, k, v, causal, window, scale, seq_lens=None):
    """One-pass attention with explicit Python loops and no max subtraction
    (valid for small scores): O = sum exp(s_j) v_j / sum exp(s_j)."""
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        n = Skv if seq_lens is None else int(seq_lens[b])
        for h in range(Hq):
            kh = h // G
            for i in range(Sq):
                pos = n - Sq + i
                num = [0.0] * D
                den = 0.0
                for j in range(n):
                    if causal and j > pos:
                        continue
                    if causal and window > 0 and j <= pos - window:
                        continue
                    s = scale * sum(float(q[b, i, h, d]) * float(k[b, j, kh, d]) for d in range(D))
                    w = math.exp(s)
                    den += w
                    for d in range(D):
                        num[d] += w * float(v[b, j, kh, d])
                if den > 0:
                    o[b, i, h] = [x / den for x in num]
                    lse[b, h, i] = math.log(den)
    return o, lse


BRUTE_CASES = [
    # B, Sq, Skv, Hq, Hkv, D, causal, window, seq_lens
    (1, 4, 4, 2, 1, 8, True, 0, None),
    (2, 3, 7, 4, 2, 4, True, 0, None),
    (1, 5, 9, 3, 3, 4, True, 3, None),
    (1, 6, 6, 4, 1, 4, False, 0, None),
    (2, 2, 6, 2, 2, 4, True, 2, [6, 4]),
    (1, 7, 3, 2, 1, 4, True, 0, None),        # Sq > Skv: leading rows empty
]


def check_brute_force(orc):
    r = _rng(6)
    for (B, Sq, Skv, Hq, Hkv, D, causal, window, lens) in BRUTE_CASES:
        q = r.standard_normal((B, Sq, Hq, D))
        k = r.standard_normal((B, Skv, Hkv, D))
        v = r.standard_normal((B, Skv, Hkv, D))
        o, lse = orc.attention_ref(q, k, v, causal=causal, window=window, scale=0.4, seq_lens=lens)
        ob, lb = brute_force(q, k, v, causal, window, 0.4, lens)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
        fin = np.isfinite(lb)
        np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


def check_combine_partition(orc):
    """Merging the partials of any chunking gives the unsplit result."""
    r = _rng(7)
    q = r.standard_normal((2, 3, 4, 8))
    k = r.standard_normal((2, 37, 2, 8))
    v = r.standard_normal((2, 37, 2, 8))
    lens = [37, 20]
    whole_o, whole_l = orc.attention_ref(q, k, v, causal=True, window=0, scale=0.5, seq_lens=lens)
    for chunk in (1, 5, 16, 37, 64):
        op, lp = orc.partial_attention_ref(q, k, v, causal=True, scale=0.5, seq_lens=lens, chunk=chunk)
        o, l = orc.combine_ref(op, lp)
        np.testing.assert_allclose(o, whole_o, atol=1e-12)
        np.testing.assert_allclose(l, whole_l, atol=1e-12)


def check_paged_equals_contiguous(orc):
    """Decode over a randomly permuted paged cache equals decode over the
    same tokens stored contiguously; the gather is a pure index map."""
    r = _rng(8)
    B, Hkv, D, ps, ppseq = 3, 2, 8, 4, 5
    Smax = ps * ppseq
    kc = r.standard_normal((B, Smax, Hkv, D))
    vc = r.standard_normal((B, Smax, Hkv, D))
    perm = r.permutation(B * ppseq)
    table = perm.reshape(B, ppseq)
    kp = np.zeros((B * ppseq, ps, Hkv, D))
    vp = np.zeros((B * ppseq, ps, Hkv, D))
    for b in range(B):
        for t in range(Smax):
            kp[table[b, t // ps], t % ps] = kc[b, t]
            vp[table[b, t // ps], t % ps] = vc[b, t]
    lens = [20, 7, 13]
    g = orc.paged_gather_ref(kp, table, lens, ps, Smax)
    for b in range(B):
        np.testing.assert_array_equal(g[b, :lens[b]], kc[b, :lens[b]])
        assert np.all(g[b, lens[b]:] == 0)
    q = r.standard_normal((B, 3, 4, D))
    o1, l1 = orc.decode_paged_ref(q, kp, vp, table, lens, page_size=ps, causal=True, scale=0.3)
    o2, l2 = orc.decode_paged_ref(q, kc, vc, None, lens, page_size=ps, causal=True, scale=0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


ALL_CHECKS = [
    check_golden,
    check_single_key,
    check_constant_v,
    check_equal_scores,
    check_two_keys,
    check_empty_rows,
    check_brute_force,
    check_combine_partition,
    check_paged_equals_contiguous,
]
