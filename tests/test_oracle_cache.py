"""Pins of the oracle's KV-cache append (CPU): an element-by-element
pure-Python brute force on tiny caches, the invariant that a dense gather of
the appended cache ends with exactly the new rows while every other token is
unchanged, and the rows the append must not write."""

import random

import numpy as np

import oracle


def _brute(kc, bt, lens, new, ps, num_pages):
    """Every element moved by hand: out[page][slot][g][d] = new[b][i][g][d]."""
    out = [[[[kc[p][s][g][d] for d in range(len(kc[0][0][0]))] for g in range(len(kc[0][0]))]
            for s in range(ps)] for p in range(len(kc))]
    cap = len(bt[0]) * ps
    for b in range(len(new)):
        n = min(max(lens[b], 0), cap)
        for i in range(len(new[b])):
            t = n - len(new[b]) + i
            if t < 0:
                continue
            page = bt[b][t // ps]
            if not 0 <= page < num_pages:
                continue
            for g in range(len(new[b][i])):
                for d in range(len(new[b][i][g])):
                    out[page][t % ps][g][d] = new[b][i][g][d]
    return out


def test_append_brute_force():
    rng = random.Random(7)
    for trial in range(30):
        ps, P, B, Hkv, D = rng.choice([1, 2, 4]), rng.randint(4, 9), rng.randint(1, 3), 2, 3
        mp = rng.randint(1, 4)
        snew = rng.randint(1, 4)
        kc = np.array([[[[rng.random() for _ in range(D)] for _ in range(Hkv)] for _ in range(ps)]
                       for _ in range(P)])
        bt = [[rng.randint(-1, P) for _ in range(mp)] for _ in range(B)]   # includes out-of-range pages
        lens = [rng.randint(-1, mp * ps + 2) for _ in range(B)]
        new = np.array([[[[rng.random() for _ in range(D)] for _ in range(Hkv)] for _ in range(snew)]
                        for _ in range(B)])
        got, _ = oracle.kv_append_ref(kc, kc, np.array(bt), np.array(lens), new, new, page_size=ps,
                                      num_pages=P)
        want = _brute(kc.tolist(), bt, lens, new.tolist(), ps, P)
        assert np.array_equal(got, np.array(want)), trial


def test_append_then_gather_ends_with_new_rows():
    rng = np.random.default_rng(3)
    P, ps, Hkv, D, B, mp, snew = 40, 4, 2, 8, 3, 6, 5
    perm = rng.permutation(P)[: B * mp].reshape(B, mp)       # distinct pages: no two rows collide
    kc = rng.standard_normal((P, ps, Hkv, D))
    lens = np.array([24, 7, 3])                               # 3 < snew: the first rows have no slot
    new = rng.standard_normal((B, snew, Hkv, D))
    kc2, _ = oracle.kv_append_ref(kc, kc, perm, lens, new, new, page_size=ps)
    before = oracle.paged_gather_ref(kc, perm, lens, ps)
    after = oracle.paged_gather_ref(kc2, perm, lens, ps)
    for b in range(B):
        n = int(lens[b])
        k = min(n, snew)
        assert np.array_equal(after[b, n - k:n], new[b, snew - k:])
        assert np.array_equal(after[b, : n - k], before[b, : n - k])
    touched = {(int(perm[b, t // ps]), t % ps) for b in range(B)
               for t in range(max(int(lens[b]) - snew, 0), int(lens[b]))}
    for p in range(P):
        for s_ in range(ps):
            if (p, s_) not in touched:
                assert np.array_equal(kc2[p, s_], kc[p, s_])


def test_append_contiguous_layout():
    rng = np.random.default_rng(5)
    B, S, Hkv, D, snew = 2, 16, 1, 4, 3
    kc = rng.standard_normal((B, S, Hkv, D))
    new = rng.standard_normal((B, snew, Hkv, D))
    lens = np.array([10, 16])
    kc2, _ = oracle.kv_append_ref(kc, kc, None, lens, new, new, page_size=4)
    assert np.array_equal(kc2[0, 7:10], new[0]) and np.array_equal(kc2[1, 13:16], new[1])
    assert np.array_equal(kc2[0, :7], kc[0, :7]) and np.array_equal(kc2[0, 10:], kc[0, 10:])
