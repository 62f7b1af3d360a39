"""Pins of the oracle's fp8 (OCP e4m3) KV encoding (CPU): values the format's
definition fixes, torch's float8_e4m3fn dtype as an independent library
decoder and encoder, exact round trips, ties to even at midpoints,
saturation, the per-head dequantisation against torch's decoder times a
scale per head, and the fp8 append's index map against a loop over tokens."""

import math

import numpy as np
import torch

import oracle


def check_e4m3_spot_values(orc):
    v = orc.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0 and v(0x80) == 0.0
    assert v(0x01) == 2.0 ** -9                  # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9              # largest subnormal
    assert v(0x08) == 2.0 ** -6                  # smallest normal
    assert v(0x38) == 1.0 and v(0xB8) == -1.0
    assert v(0x3C) == 1.5 and v(0x40) == 2.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    t = orc.e4m3_table()
    assert np.all(np.diff(t[0:0x7F]) > 0)      # 0 .. 448 strictly increasing
    assert np.array_equal(t[0x80:0xFF], -t[0:0x7F])


def check_e4m3_against_torch_dtype(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = orc.e4m3_table()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    assert np.array_equal(t[fin], ref[fin])
    # encoding: torch's float -> e4m3fn conversion (round to nearest even) on
    # in-range values
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * 10.0, rng.uniform(-448, 448, 4000),
                        rng.standard_normal(2000) * 1e-2, rng.standard_normal(500) * 1e-3])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.quantize_e4m3(x)
    assert np.array_equal(got, want)


def check_quantize_round_trip_ties_saturation(orc):
    t = orc.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(orc.quantize_e4m3(t[codes]), codes)
    # midpoints between neighbouring positive codes go to the even code
    for c in range(0x00, 0x7E):
        mid = (t[c] + t[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert orc.quantize_e4m3(np.array([mid]))[0] == want, c
        assert orc.quantize_e4m3(np.array([-mid]))[0] == (want | 0x80), c
        # just off the midpoint: the nearer code
        eps = (t[c + 1] - t[c]) * 1e-6
        assert orc.quantize_e4m3(np.array([mid - eps]))[0] == c
        assert orc.quantize_e4m3(np.array([mid + eps]))[0] == c + 1
    # saturation and special values
    q = orc.quantize_e4m3(np.array([448.0, 464.0, 1e9, -1e9, np.inf, -np.inf, np.nan, -0.0, 1e-30, -1e-30]))
    assert list(q) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0x80, 0x00, 0x80]


def check_fp8_append_index_map(orc):
    rng = np.random.default_rng(4)
    B, Snew, Hkv, D, ps, mp = 3, 5, 2, 16, 4, 6
    P = B * mp + 2
    table = rng.permutation(P)[: B * mp].reshape(B, mp)
    table[2, 1] = P + 3                          # out of range: tokens 4..7 of sequence 2 skipped
    kc = rng.integers(0, 255, (P, ps, Hkv, D)).astype(np.uint8)
    vc = rng.integers(0, 255, (P, ps, Hkv, D)).astype(np.uint8)
    lens = [mp * ps, 3, 9]
    kn = torch.randn(B, Snew, Hkv, D).to(torch.bfloat16)
    vn = torch.randn(B, Snew, Hkv, D).to(torch.bfloat16)
    ks, vs = np.array([0.02, 0.5], np.float32), np.array([0.1, 3.0], np.float32)
    k2, v2 = orc.kv_append_fp8_ref(kc, vc, table, lens, kn, vn, ks, vs, page_size=ps)
    kexp, vexp = kc.copy(), vc.copy()
    for b in range(B):
        for i in range(Snew):
            tok = lens[b] - Snew + i
            if tok < 0:
                continue
            page = table[b, tok // ps]
            if page >= P:
                continue
            for g in range(Hkv):
                for d in range(D):
                    qk = np.float32(kn[b, i, g, d].item()) / ks[g]
                    qv = np.float32(vn[b, i, g, d].item()) / vs[g]
                    kexp[page, tok % ps, g, d] = orc.quantize_e4m3(np.array([qk]))[0]
                    vexp[page, tok % ps, g, d] = orc.quantize_e4m3(np.array([qv]))[0]
    assert np.array_equal(k2, kexp) and np.array_equal(v2, vexp)
    assert not np.array_equal(k2, kc)


def check_dequantize_per_head(orc):
    """The cached value of a byte of KV head g is e4m3(byte) * scale[g]:
    torch's float8_e4m3fn decoder widened to fp64 times a distinct scale per
    head, on a paged-cache-shaped array [P, 16, Hkv, D] with Hkv != D (so a
    scale broadcast along D, or one head's scale for all, differs)."""
    rng = np.random.default_rng(5)
    P, ps, Hkv, D = 3, 16, 3, 8
    codes = rng.integers(0, 256, (P, ps, Hkv, D)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E                  # keep the comparison finite
    codes[codes == 0xFF] = 0xFE
    scale = np.array([0.25, 3.0, 1.0 / 7.0], dtype=np.float32)
    got = orc.dequantize_e4m3(codes, scale)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = np.empty_like(dec)
    for g in range(Hkv):
        want[:, :, g, :] = dec[:, :, g, :] * float(scale[g])
    assert got.shape == codes.shape
    assert np.array_equal(got, want)
    # a NaN code stays NaN (and only there)
    nan_codes = codes.copy()
    nan_codes[0, 0, 1, 2] = 0x7F
    out = orc.dequantize_e4m3(nan_codes, scale)
    assert np.isnan(out[0, 0, 1, 2]) and np.isnan(out).sum() == 1


FP8_CHECKS = [check_e4m3_spot_values, check_e4m3_against_torch_dtype, check_quantize_round_trip_ties_saturation,
              check_fp8_append_index_map, check_dequantize_per_head]


def test_e4m3_spot_values():
    check_e4m3_spot_values(oracle)


def test_e4m3_against_torch_dtype():
    check_e4m3_against_torch_dtype(oracle)


def test_quantize_round_trip_ties_saturation():
    check_quantize_round_trip_ties_saturation(oracle)


def test_fp8_append_index_map():
    check_fp8_append_index_map(oracle)


def test_dequantize_per_head():
    check_dequantize_per_head(oracle)
