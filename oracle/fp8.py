"""FP8 (OCP e4m3, "e4m3fn") KV-cache encoding for the oracle.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
package smoke check and the benchmark's CPU baseline may use it; the product
path never does, and nothing here is shared with the GPU code.

The quantised KV decode row of the hot path stores K and V as one byte per
element in the OCP 8-bit floating-point format e4m3 (1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; no infinities; exponent field 15 with
mantissa 7 is NaN; largest finite value 448), with one fp32 dequantisation
scale per KV head for K and one for V: the cached value of element x of KV
head g is e4m3(code) * scale[g]. The pages name low-bit KV caches (q8_0 in
the llama.cpp PR 28507 report, KVarN in beellama.cpp PR 149) without fixing
a format; e4m3 with a per-head scale is this build's reading (it is the
8-bit float format the target GPU converts natively).

Quantisation of a bf16 value v of KV head g (the append of new rows): the
fp32 quotient q = fp32(v) / fp32(scale[g]) (one IEEE fp32 division, rounded
to nearest even), then the e4m3 code nearest to q, ties to the code whose
mantissa is even, values beyond +-448 saturating to +-448, NaN to 0x7f. The
sign of q is kept (-0 and negatives that round to zero give 0x80).
"""

from __future__ import annotations

import numpy as np

__all__ = ["e4m3_value", "e4m3_table", "quantize_e4m3", "dequantize_e4m3", "kv_append_fp8_ref"]


def e4m3_value(code: int) -> float:
    """The real value of one e4m3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:                       # subnormal: 0.m x 2^(1 - bias)
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """float64 value of every code 0..255."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def quantize_e4m3(q) -> np.ndarray:
    """Codes (uint8) of float values q (already divided by the scale):
    nearest e4m3 value, ties to the even code, saturating at +-448."""
    q = np.asarray(q, dtype=np.float64)
    table = e4m3_table()
    pos = table[0:0x7F]                          # codes 0x00..0x7E: 0 .. 448, increasing
    mag = np.minimum(np.abs(q), pos[-1])
    # candidates: the largest code whose value is <= mag, and the next one up
    lo = np.searchsorted(pos, mag, side="right") - 1
    hi = np.minimum(lo + 1, len(pos) - 1)
    d_lo = mag - pos[lo]
    d_hi = pos[hi] - mag
    pick = np.where(d_hi < d_lo, hi, lo)
    tie = (d_hi == d_lo) & (hi != lo)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    codes = pick.astype(np.uint8)
    codes = np.where(np.signbit(q), codes | 0x80, codes).astype(np.uint8)
    codes = np.where(np.isnan(q), np.uint8(0x7F), codes).astype(np.uint8)
    return codes


def dequantize_e4m3(codes, scale) -> np.ndarray:
    """Cached values: e4m3(codes) * scale[g], codes [..., Hkv, D] uint8 and
    scale [Hkv] (float64 result)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scale = np.asarray(scale, dtype=np.float64).reshape(-1)
    vals = e4m3_table()[codes]
    return vals * scale[:, None]


def kv_append_fp8_ref(kcache, vcache, block_table, seq_lens, knew, vnew, k_scale, v_scale, *,
                      page_size: int, num_pages: int | None = None):
    """The fp8 form of the KV-cache append: new bf16 rows [B, Snew, Hkv, D]
    are quantised (fp32 quotient by the head's scale, then e4m3 as above) and
    written to token seq_lens[b] - Snew + i of uint8 caches laid out as in
    kv_append_ref (paged [num_pages, page_size, Hkv, D] through block_table,
    or contiguous [B, Smax, Hkv, D]). Rows with a negative token or a page
    outside [0, num_pages) are skipped. Returns (kcache', vcache') as uint8
    numpy arrays."""
    kc = np.array(kcache, dtype=np.uint8, copy=True)
    vc = np.array(vcache, dtype=np.uint8, copy=True)

    def f32(x):
        if hasattr(x, "detach"):
            x = x.detach().to("cpu").float().numpy()
        return np.asarray(x, dtype=np.float32)

    kn, vn = f32(knew), f32(vnew)
    ks = np.asarray(f32(k_scale), dtype=np.float32).reshape(-1)
    vs = np.asarray(f32(v_scale), dtype=np.float32).reshape(-1)
    kq = quantize_e4m3(kn / ks[None, None, :, None])     # fp32 division, then the encoding
    vq = quantize_e4m3(vn / vs[None, None, :, None])
    lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    B, snew = kn.shape[0], kn.shape[1]
    if block_table is None:
        cap = kc.shape[1]
    else:
        bt = np.asarray(block_table, dtype=np.int64)
        cap = bt.shape[1] * page_size
        if num_pages is None:
            num_pages = kc.shape[0]
    for b in range(B):
        n = min(max(int(lens[b]), 0), cap)
        for i in range(snew):
            t = n - snew + i
            if t < 0:
                continue
            if block_table is None:
                kc[b, t] = kq[b, i]
                vc[b, t] = vq[b, i]
            else:
                page = int(bt[b, t // page_size])
                if page < 0 or page >= num_pages:
                    continue
                kc[page, t % page_size] = kq[b, i]
                vc[page, t % page_size] = vq[b, i]
    return kc, vc
