"""Head dims other than 64/128/256/512, and key / value head dims that differ,
through the C ABI against the fp64 oracle: prefill (ragged tails, windows,
Sq > Skv), decode and verify over paged and contiguous caches whose slots
past each sequence's end hold NaN, q/k/v cut from one fused projection
buffer, output columns past Dv left untouched, the append followed by a
verify, and the score modifiers on a Dk != Dv cache."""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as fa
import oracle
from tests.gpu_util import DEV, assert_parity

pytestmark = pytest.mark.gpu


def _randn(gen, shape):
    return torch.randn(shape, generator=gen).to(torch.bfloat16)


PREFILL = [
    # B, Sq, Skv, Hq, Hkv, Dk, Dv, causal, window
    (2, 77, 77, 8, 2, 72, 72, True, 0),
    (1, 130, 130, 4, 4, 80, 80, True, 33),
    (2, 100, 160, 6, 2, 96, 96, True, 0),
    (1, 150, 150, 8, 2, 192, 192, True, 0),
    (1, 129, 129, 8, 2, 192, 128, True, 0),
    (1, 90, 90, 4, 2, 320, 256, True, 0),
    (1, 64, 200, 4, 1, 40, 8, False, 0),
    (1, 70, 40, 4, 2, 112, 96, True, 0),            # Sq > Skv: leading rows see no key
    # 576-wide keys with 512-wide values (the 512 tile plus 64 extra key columns)
    (1, 150, 150, 8, 2, 576, 512, True, 0),
    (2, 64, 200, 4, 1, 576, 512, True, 70),
    (1, 70, 40, 4, 2, 576, 512, True, 0),
    (1, 96, 96, 2, 2, 576, 512, False, 0),
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}_S{}x{}_H{}x{}_Dk{}_Dv{}_c{}_w{}".format(*c))
def test_prefill_head_dims(case):
    B, Sq, Skv, Hq, Hkv, Dk, Dv, causal, window = case
    print(f"prefill head dims {case}", flush=True)
    g = torch.Generator().manual_seed(Dk * 7 + Dv + Sq)
    q, k, v = _randn(g, (B, Sq, Hq, Dk)), _randn(g, (B, Skv, Hkv, Dk)), _randn(g, (B, Skv, Hkv, Dv))
    scale = 1.0 / np.sqrt(Dk)
    # O written into the first Dv columns of a wider zeroed buffer: the rest must stay 0
    big = torch.zeros(B, Sq, Hq, Dv + 16, dtype=torch.bfloat16, device=DEV)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, scale=scale,
                        out=big[..., :Dv])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=causal, window=window, scale=scale)
    assert_parity(o, lse, o_ref, lse_ref, f"prefill head dims {case}")
    assert torch.count_nonzero(big[..., Dv:]) == 0


def test_prefill_fused_projection_views():
    """q, k and v as views of one [B, S, Hq*Dk + Hkv*Dk + Hkv*Dv] buffer."""
    B, S, Hq, Hkv, Dk, Dv = 2, 96, 8, 2, 192, 128
    g = torch.Generator().manual_seed(5)
    W = Hq * Dk + Hkv * Dk + Hkv * Dv
    buf = _randn(g, (B, S, W))
    qv = buf[..., :Hq * Dk].unflatten(-1, (Hq, Dk))
    kv_ = buf[..., Hq * Dk:(Hq + Hkv) * Dk].unflatten(-1, (Hkv, Dk))
    vv = buf[..., (Hq + Hkv) * Dk:].unflatten(-1, (Hkv, Dv))
    d = buf.to(DEV)
    o1, l1 = fa.prefill(d[..., :Hq * Dk].unflatten(-1, (Hq, Dk)),
                        d[..., Hq * Dk:(Hq + Hkv) * Dk].unflatten(-1, (Hkv, Dk)),
                        d[..., (Hq + Hkv) * Dk:].unflatten(-1, (Hkv, Dv)), causal=True)
    o2, l2 = fa.prefill(qv.contiguous().to(DEV), kv_.contiguous().to(DEV), vv.contiguous().to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle.attention_ref(qv, kv_, vv, causal=True, scale=1.0 / np.sqrt(Dk))
    assert_parity(o1, l1, o_ref, lse_ref, "fused projection views 192/128")


def _decode_case(B, Sq, Hq, Hkv, Dk, Dv, ps, max_len, lens, seed, paged):
    """Seeded caches with NaN past each length; paged through a random page permutation."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (B, Sq, Hq, Dk))
    kc = _randn(g, (B, max_len, Hkv, Dk))
    vc = _randn(g, (B, max_len, Hkv, Dv))
    for b, n in enumerate(lens):
        kc[b, n:] = float("nan")
        vc[b, n:] = float("nan")
    lens_t = torch.tensor(lens, dtype=torch.int32)
    if not paged:
        return q, kc, vc, None, lens_t, kc, vc
    mp = max_len // ps
    perm = torch.randperm(B * mp, generator=g)
    table = perm.reshape(B, mp).to(torch.int32)
    kp = torch.empty(B * mp, ps, Hkv, Dk, dtype=torch.bfloat16)
    vp = torch.empty(B * mp, ps, Hkv, Dv, dtype=torch.bfloat16)
    for b in range(B):
        for p in range(mp):
            kp[table[b, p]] = kc[b, p * ps:(p + 1) * ps]
            vp[table[b, p]] = vc[b, p * ps:(p + 1) * ps]
    return q, kp, vp, table, lens_t, kc, vc


DECODE = [
    # B, Sq, Hq, Hkv, Dk, Dv, page_size, max_len, lens, chunk, paged
    (3, 1, 16, 4, 192, 128, 16, 1024, [1, 517, 1024], 256, True),
    (2, 8, 32, 4, 80, 80, 16, 768, [8, 700], 128, True),
    (2, 4, 8, 2, 320, 256, 32, 512, [4, 511], 128, True),
    (2, 1, 8, 2, 72, 72, 16, 640, [0, 639], 64, False),
    (2, 3, 8, 8, 96, 64, 16, 512, [300, 3], 96, False),
    (2, 2, 8, 2, 40, 40, 64, 256, [256, 100], 64, True),
    (3, 1, 16, 4, 576, 512, 16, 1024, [1, 517, 1024], 256, True),
    (2, 8, 16, 2, 576, 512, 16, 768, [8, 700], 128, True),   # 64 rows per KV head: two row blocks
    (2, 3, 8, 8, 576, 512, 16, 512, [300, 3], 96, False),
    (2, 2, 8, 2, 576, 512, 64, 256, [0, 200], 64, True),      # an empty sequence
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B{}_Sq{}_H{}x{}_Dk{}_Dv{}_ps{}_L{}_{}_c{}_p{}".format(*c))
def test_decode_head_dims(case):
    B, Sq, Hq, Hkv, Dk, Dv, ps, max_len, lens, chunk, paged = case
    print(f"decode head dims {case}", flush=True)
    q, kc, vc, table, lens_t, kd, vd = _decode_case(B, Sq, Hq, Hkv, Dk, Dv, ps, max_len, lens,
                                                    seed=Dk + Dv + Sq, paged=paged)
    scale = 1.0 / np.sqrt(Dk)
    o, lse = fa.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), None if table is None else table.to(DEV),
                             lens_t.to(DEV), page_size=ps, kv_chunk=chunk, causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, torch.nan_to_num(kd.float()), torch.nan_to_num(vd.float()),
                                          causal=True, scale=scale, seq_lens=lens)
    assert_parity(o, lse, o_ref, lse_ref, f"decode head dims {case}")


def test_verify_dk_dv_all_modifiers():
    B, Sq, Hq, Hkv, Dk, Dv, ps, max_len = 2, 8, 32, 4, 192, 128, 16, 768
    lens = [768, 301]
    q, kc, vc, table, lens_t, kd, vd = _decode_case(B, Sq, Hq, Hkv, Dk, Dv, ps, max_len, lens, seed=21, paged=True)
    g = torch.Generator().manual_seed(22)
    sinks = torch.randn(Hq, generator=g).float()
    mask = (2.0 * torch.randn(B, Sq, max_len, generator=g)).to(torch.bfloat16)
    mask[:, :, 10:20] = -float("inf")
    scale = 1.0 / np.sqrt(Dk)
    o, lse = fa.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), lens_t.to(DEV), page_size=ps,
                             kv_chunk=256, causal=True, scale=scale, softcap=20.0, max_bias=4.0,
                             sinks=sinks.to(DEV), mask=mask.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, torch.nan_to_num(kd.float()), torch.nan_to_num(vd.float()),
                                          causal=True, scale=scale, seq_lens=lens, softcap=20.0, max_bias=4.0,
                                          sinks=sinks.double().numpy(), mask=mask)
    assert_parity(o, lse, o_ref, lse_ref, "verify 192/128 all modifiers")


def test_append_then_verify_dk_dv():
    B, Sq, Hq, Hkv, Dk, Dv, ps, mp = 2, 8, 16, 2, 192, 128, 16, 24
    g = torch.Generator().manual_seed(31)
    P = B * mp
    table = torch.randperm(P, generator=g).reshape(B, mp).to(torch.int32)
    kc, vc = _randn(g, (P, ps, Hkv, Dk)), _randn(g, (P, ps, Hkv, Dv))
    lens = torch.tensor([mp * ps - 3, 200], dtype=torch.int32)
    kn, vn = _randn(g, (B, Sq, Hkv, Dk)), _randn(g, (B, Sq, Hkv, Dv))
    q = _randn(g, (B, Sq, Hq, Dk))
    kd, vd = kc.to(DEV), vc.to(DEV)
    fa.kv_append(kd, vd, table.to(DEV), lens.to(DEV), kn.to(DEV), vn.to(DEV), page_size=ps)
    o, lse = fa.decode_paged(q.to(DEV), kd, vd, table.to(DEV), lens.to(DEV), page_size=ps, kv_chunk=128)
    torch.cuda.synchronize()
    kc2, vc2 = oracle.kv_append_ref(kc, vc, table, lens, kn, vn, page_size=ps)
    assert torch.equal(kd.cpu().view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vd.cpu().view(torch.int16), vc2.view(torch.int16))
    o_ref, lse_ref = oracle.decode_paged_ref(q, kc2, vc2, table, lens, page_size=ps, causal=True,
                                             scale=1.0 / np.sqrt(Dk))
    assert_parity(o, lse, o_ref, lse_ref, "append + verify 192/128")


def test_prefill_padded_with_mask_and_window():
    """The padded kernel with the score transform and a mask (level 4):
    80/64 with softcap, ALiBi, sinks, a mask and a window."""
    B, Sq, Skv, Hq, Hkv, Dk, Dv = 2, 90, 120, 8, 2, 80, 64
    g = torch.Generator().manual_seed(41)
    q, k, v = _randn(g, (B, Sq, Hq, Dk)), _randn(g, (B, Skv, Hkv, Dk)), _randn(g, (B, Skv, Hkv, Dv))
    sinks = torch.randn(Hq, generator=g).float()
    mask = (2.0 * torch.randn(B, Sq, 124, generator=g)).to(torch.bfloat16)
    mask[:, :, 30:40] = -float("inf")
    scale = 1.0 / np.sqrt(Dk)
    kw = dict(softcap=15.0, max_bias=6.0)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, window=50, scale=scale,
                        sinks=sinks.to(DEV), mask=mask.to(DEV)[:, :, :Skv], **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=True, window=50, scale=scale,
                                          sinks=sinks.double().numpy(), mask=mask[:, :, :Skv], **kw)
    assert_parity(o, lse, o_ref, lse_ref, "prefill 80/64 all modifiers window 50")


def test_decode_padded_window():
    B, Sq, Hq, Hkv, Dk, Dv, ps, max_len = 2, 4, 16, 4, 96, 96, 16, 640
    q, kc, vc, table, lens_t, kd, vd = _decode_case(B, Sq, Hq, Hkv, Dk, Dv, ps, max_len, [640, 333],
                                                    seed=51, paged=True)
    scale = 1.0 / np.sqrt(Dk)
    o, lse = fa.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), lens_t.to(DEV), page_size=ps,
                             kv_chunk=128, causal=True, window=70, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, torch.nan_to_num(kd.float()), torch.nan_to_num(vd.float()),
                                          causal=True, window=70, scale=scale, seq_lens=[640, 333])
    assert_parity(o, lse, o_ref, lse_ref, "decode 96/96 window 70")


def test_wide_keys_modifiers_prefill_and_verify():
    """576/512 with every score modifier (softcap, ALiBi, sinks, a mask with a
    hidden band), in prefill (ragged, windowed) and in an 8-row verify over a
    paged cache."""
    Dk, Dv = 576, 512
    g = torch.Generator().manual_seed(576)
    B, S, Hq, Hkv = 1, 100, 4, 2
    q, k, v = _randn(g, (B, S, Hq, Dk)), _randn(g, (B, S, Hkv, Dk)), _randn(g, (B, S, Hkv, Dv))
    sinks = torch.randn(Hq, generator=g).float()
    mask = (2.0 * torch.randn(B, S, S, generator=g)).to(torch.bfloat16)
    mask[:, :, 10:14] = -float("inf")
    kw = dict(softcap=20.0, max_bias=4.0)
    scale = 1.0 / np.sqrt(Dk)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, window=60, scale=scale,
                        sinks=sinks.to(DEV), mask=mask.to(DEV), **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=True, window=60, scale=scale,
                                          sinks=sinks.double().numpy(), mask=mask, **kw)
    assert_parity(o, lse, o_ref, lse_ref, "prefill 576/512 all modifiers")
    B, Sq, Hq, Hkv, ps, L = 2, 8, 16, 2, 16, 512
    q, kc, vc, table, lens_t, kd, vd = _decode_case(B, Sq, Hq, Hkv, Dk, Dv, ps, L, [L, 333], seed=577, paged=True)
    sinks = torch.randn(Hq, generator=g).float()
    mask = (2.0 * torch.randn(B, Sq, L, generator=g)).to(torch.bfloat16)
    o, lse = fa.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), lens_t.to(DEV), page_size=ps,
                             kv_chunk=128, causal=True, scale=scale, sinks=sinks.to(DEV), mask=mask.to(DEV), **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, torch.nan_to_num(kd.float()), torch.nan_to_num(vd.float()),
                                          causal=True, scale=scale, seq_lens=[L, 333],
                                          sinks=sinks.double().numpy(), mask=mask, **kw)
    assert_parity(o, lse, o_ref, lse_ref, "verify 576/512 all modifiers")


def test_wide_keys_append_then_verify():
    """fa_kv_append of 576-wide K and 512-wide V rows into a paged cache, then
    an 8-row verify over it."""
    Dk, Dv = 576, 512
    B, Sq, Hq, Hkv, ps, L = 2, 8, 16, 2, 16, 384
    q, kc, vc, table, lens_t, kd, vd = _decode_case(B, Sq, Hq, Hkv, Dk, Dv, ps, L, [L, 200], seed=578, paged=True)
    g = torch.Generator().manual_seed(579)
    kn, vn = _randn(g, (B, Sq, Hkv, Dk)), _randn(g, (B, Sq, Hkv, Dv))
    kdev, vdev = kc.to(DEV), vc.to(DEV)
    fa.kv_append(kdev, vdev, table.to(DEV), lens_t.to(DEV), kn.to(DEV), vn.to(DEV), page_size=ps)
    o, lse = fa.decode_paged(q.to(DEV), kdev, vdev, table.to(DEV), lens_t.to(DEV), page_size=ps, kv_chunk=128,
                             causal=True)
    torch.cuda.synchronize()
    for b, n in enumerate([L, 200]):
        kd[b, n - Sq:n] = kn[b]
        vd[b, n - Sq:n] = vn[b]
    o_ref, lse_ref = oracle.attention_ref(q, torch.nan_to_num(kd.float()), torch.nan_to_num(vd.float()),
                                          causal=True, scale=1.0 / np.sqrt(Dk), seq_lens=[L, 200])
    assert_parity(o, lse, o_ref, lse_ref, "append + verify 576/512")


def test_wide_keys_prefill_long_sampled():
    """576/512 causal prefill over 2048 keys (64 tiles), sampled query rows
    against the oracle."""
    Dk, Dv = 576, 512
    g = torch.Generator().manual_seed(580)
    B, S, Hq, Hkv = 1, 2048, 4, 2
    q, k, v = _randn(g, (B, S, Hq, Dk)), _randn(g, (B, S, Hkv, Dk)), _randn(g, (B, S, Hkv, Dv))
    scale = 1.0 / np.sqrt(Dk)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 777, 1500, 2046, 2047])
    o_ref, lse_ref = oracle.attention_ref(q, k, v, causal=True, scale=scale, rows=rows)
    o_s = o[:, rows].cpu()
    l_s = lse[:, :, rows].cpu()
    assert_parity(o_s, l_s, o_ref[:, rows], lse_ref[:, :, rows], "prefill 576/512 S2048 sampled rows")
