"""The C-ABI library loads, exports every symbol include/gqafa.h declares,
and rejects invalid calls on the host before any launch (no GPU needed: the
validation paths return before touching the device)."""

import ctypes
import os
import re

import pytest

from gqa_flash_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqafa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted(["fa_prefill", "fa_prefill_strided", "fa_decode_workspace_bytes",
                            "fa_decode_paged", "fa_decode_paged_strided", "fa_combine_lse",
                            "fa_kv_append", "fa_status_string", "fa_paged_gather",
                            "fa_decode_paged_fp8", "fa_kv_append_fp8", "fa_decode_paged_noalloc"])
    assert set(names) == set(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(lib):
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, -5, 12345):
        assert lib.fa_status_string(s)


# a fake, 16-byte aligned "device" address: validation must fail before any use
P = 0x10000


def _prefill(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Sq=8, Skv=8, D=128,
             causal=1, window=0, scale=0.125)
    a.update(kw)
    return lib.fa_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Sq"], a["Skv"], a["D"], a["causal"], a["window"], a["scale"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(D=576), UNSUPPORTED), (dict(D=84), UNSUPPORTED), (dict(D=0), UNSUPPORTED),
    (dict(D=96, B=0), OK), (dict(D=32, B=0), OK), (dict(D=8, B=0), OK), (dict(D=72, B=0), OK),
    (dict(Hq=6, Hkv=4), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID),
    (dict(B=-1), INVALID), (dict(Sq=-1), INVALID), (dict(Skv=-2), INVALID),
    (dict(window=4, causal=0), INVALID), (dict(window=-1), INVALID), (dict(causal=2), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(k=None), INVALID),
    (dict(q=P + 2), INVALID), (dict(v=P + 8), INVALID), (dict(lse=P + 2), INVALID),
    (dict(B=0), OK), (dict(Sq=0), OK),
])
def test_prefill_validation(lib, kw, want):
    assert _prefill(lib, **kw) == want


def _decode(lib, **kw):
    a = dict(q=P, k=P, v=P, table=P, lens=P, o=P, lse=P, B=2, Sq=1, Hq=8, Hkv=2, D=128,
             num_pages=64, page_size=16, max_pages=8, chunk=64, causal=1, window=0, scale=0.1,
             ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return lib.fa_decode_paged(a["q"], a["k"], a["v"], a["table"], a["lens"], a["o"], a["lse"],
                               a["B"], a["Sq"], a["Hq"], a["Hkv"], a["D"], a["num_pages"],
                               a["page_size"], a["max_pages"], a["chunk"], a["causal"], a["window"],
                               a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(D=520), UNSUPPORTED), (dict(D=100), UNSUPPORTED), (dict(page_size=12), UNSUPPORTED),
    (dict(page_size=0), UNSUPPORTED), (dict(page_size=1 << 17), UNSUPPORTED), (dict(D=80, B=0), OK),
    (dict(Hq=7), INVALID), (dict(chunk=0), INVALID), (dict(max_pages=-1), INVALID),
    (dict(chunk=48), INVALID), (dict(chunk=100), INVALID), (dict(chunk=33), INVALID),
    (dict(window=3, causal=0), INVALID), (dict(scale=0.0), INVALID),
    (dict(num_pages=0), INVALID), (dict(lens=None), INVALID), (dict(q=None), INVALID),
    (dict(k=P + 4), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE), (dict(ws=P + 4), WORKSPACE),
    (dict(max_pages=1 << 27, page_size=1 << 8), INVALID),
    (dict(B=0), OK), (dict(Sq=0), OK),
])
def test_decode_validation(lib, kw, want):
    assert _decode(lib, **kw) == want


def test_workspace_bytes(lib):
    f = lib.fa_decode_workspace_bytes
    # C3 shape: 16 x 32 rows x (64 chunks + 1 slots) x (128 + 1) fp32
    assert f(16, 1, 32, 128, 16384, 256) == 16 * 32 * 65 * 128 * 4 + 16 * 32 * 65 * 4
    assert f(1, 1, 1, 100, 10, 4) == 0         # unsupported head dim
    assert f(1, 1, 1, 64, 10, 0) == 0          # bad chunk
    assert f(1, 1, 1, 64, 10, 48) == 0         # chunks are whole 32-key tiles
    # head dims below a tile width are sized at the tile width
    assert f(16, 1, 32, 80, 16384, 256) == f(16, 1, 32, 128, 16384, 256)
    # 576-wide keys run on the 512 tile
    assert f(2, 8, 16, 576, 4096, 256) == f(2, 8, 16, 512, 4096, 256)
    assert f(2, 8, 16, 584, 4096, 256) == 0
    assert f(2, 3, 4, 320, 1000, 96) == f(2, 3, 4, 512, 1000, 96)


def test_workspace_bytes_alignment(lib):
    f = lib.fa_decode_workspace_bytes
    rows, slots, D = 1 * 2 * 3, 3 + 1, 64
    o = rows * slots * D * 4
    l = rows * slots * 4
    up = lambda x: (x + 255) // 256 * 256
    assert f(1, 3, 2, 64, 70, 32) == up(o) + up(l)


@pytest.mark.parametrize("kw,want", [
    (dict(D=48), UNSUPPORTED), (dict(D=96), UNSUPPORTED), (dict(B=-1), INVALID), (dict(max_chunks=-1), INVALID),
    (dict(o=None), INVALID), (dict(o_part=None), INVALID), (dict(B=0), OK),
])
def test_combine_validation(lib, kw, want):
    a = dict(o_part=P, lse_part=P, n=None, max_chunks=4, o=P, lse=P, B=1, Sq=1, Hq=2, D=64)
    a.update(kw)
    st = lib.fa_combine_lse(a["o_part"], a["lse_part"], a["n"], a["max_chunks"], a["o"], a["lse"],
                            a["B"], a["Sq"], a["Hq"], a["D"], None)
    assert st == want


@pytest.mark.parametrize("kw,want", [
    (dict(D=44), UNSUPPORTED), (dict(page_size=3), UNSUPPORTED), (dict(table=None), INVALID),
    (dict(num_pages=0), INVALID), (dict(out=P + 2), INVALID), (dict(B=0), OK),
])
def test_gather_validation(lib, kw, want):
    a = dict(cache=P, table=P, lens=P, out=P, B=1, Hkv=1, D=64, num_pages=4, page_size=16, max_pages=4)
    a.update(kw)
    st = lib.fa_paged_gather(a["cache"], a["table"], a["lens"], a["out"], a["B"], a["Hkv"], a["D"],
                             a["num_pages"], a["page_size"], a["max_pages"], None)
    assert st == want


def _st(a, b, c):
    return (ctypes.c_int64 * 3)(a, b, c)


def test_strided_prefill_validation(lib):
    f = lib.fa_prefill_strided
    def call(qs=None, ks=None, B=0):
        return f(P, qs, P, ks, P, None, P, None, None, B, 8, 2, 16, 16, 128, 128, 1, 0, 0.1, None, None)
    assert call() == OK                                   # NULL strides: contiguous
    assert call(qs=_st(16 * 8 * 128, 8 * 128, 128)) == OK  # explicit dense strides
    assert call(qs=_st(16 * 8 * 128, 8 * 128, 12)) == INVALID    # head stride not a multiple of 8
    assert call(qs=_st(-8, 8 * 128, 128)) == INVALID              # negative
    assert call(ks=_st(0, 1 << 24, 128)) == INVALID               # K token stride too large
    assert call(ks=_st(0, (1 << 24) - 8, 128)) == OK


def test_strided_decode_validation(lib):
    f = lib.fa_decode_paged_strided
    def call(ks=None, os_=None, B=0):
        return f(P, None, P, ks, P, None, P, P, P, os_, None, B, 1, 8, 2, 128, 128, 64, 16, 8, 64, 1, 0,
                 0.1, None, P, 1 << 30, None)
    assert call() == OK
    assert call(ks=_st(2 * 16 * 2 * 128, 2 * 2 * 128, 128)) == OK      # K/V interleaved per slot
    assert call(ks=_st(4, 8, 8)) == INVALID
    assert call(os_=_st(8, 8, -8)) == INVALID


@pytest.mark.parametrize("kw,want", [
    (dict(Dk=84), UNSUPPORTED), (dict(Dv=600), UNSUPPORTED), (dict(Dk=80, Dv=72, B=0), OK),
    (dict(page_size=3), UNSUPPORTED), (dict(Hkv=0), INVALID), (dict(num_pages=0), INVALID), (dict(lens=None), INVALID), (dict(kc=P + 4), INVALID),
    (dict(kn=None), INVALID), (dict(ks=_st(0, 12, 8)), INVALID),
    (dict(B=0), OK), (dict(Snew=0), OK), (dict(table=None, num_pages=0, B=0), OK),
])
def test_kv_append_validation(lib, kw, want):
    a = dict(kc=P, ks=None, vc=P, vs=None, table=P, lens=P, kn=P, kns=None, vn=P, vns=None,
             B=2, Snew=4, Hkv=2, Dk=128, Dv=128, num_pages=64, page_size=16, max_pages=8)
    a.update(kw)
    assert lib.fa_kv_append(a["kc"], a["ks"], a["vc"], a["vs"], a["table"], a["lens"], a["kn"], a["kns"],
                            a["vn"], a["vns"], a["B"], a["Snew"], a["Hkv"], a["Dk"], a["Dv"], a["num_pages"],
                            a["page_size"], a["max_pages"], None) == want


def test_score_mods_validation(lib):
    f = lib.fa_prefill_strided
    def call(m):
        return f(P, None, P, None, P, None, P, None, None, 0, 8, 2, 16, 16, 128, 128, 1, 0, 0.1,
                 ctypes.byref(m), None)
    assert call(_lib.ScoreMods(30.0, 8.0, P)) == OK
    assert call(_lib.ScoreMods(-1.0, 0.0, None)) == INVALID
    assert call(_lib.ScoreMods(0.0, float("inf"), None)) == INVALID
    assert call(_lib.ScoreMods(0.0, float("nan"), None)) == INVALID
    assert call(_lib.ScoreMods(0.0, 0.0, P + 2)) == INVALID          # unaligned sinks
    assert call(_lib.ScoreMods(0.0, 0.0, None, P, 0, 4096)) == OK
    assert call(_lib.ScoreMods(0.0, 0.0, None, P + 4, 0, 4096)) == INVALID    # mask not 8-byte aligned
    assert call(_lib.ScoreMods(0.0, 0.0, None, P, 6, 4096)) == INVALID       # stride not a multiple of 4
    assert call(_lib.ScoreMods(0.0, 0.0, None, P, 0, -4)) == INVALID
    assert call(_lib.ScoreMods(0.0, 0.0, None, P, 1 << 40, 4)) == INVALID


@pytest.mark.parametrize("dk,dv,want", [
    (192, 128, OK), (320, 256, OK), (72, 80, OK), (8, 512, OK), (576, 512, OK),
    (576, 576, UNSUPPORTED), (576, 256, UNSUPPORTED), (584, 512, UNSUPPORTED), (512, 576, UNSUPPORTED),
    (128, 12, UNSUPPORTED), (0, 64, UNSUPPORTED),
])
def test_dk_dv_validation(lib, dk, dv, want):
    """Distinct key / value head dims on the strided entry points (B = 0:
    validation only)."""
    f = lib.fa_prefill_strided
    assert f(P, None, P, None, P, None, P, None, None, 0, 8, 2, 16, 16, dk, dv, 1, 0, 0.1, None, None) == want
    g = lib.fa_decode_paged_strided
    assert g(P, None, P, None, P, None, P, P, P, None, None, 0, 1, 8, 2, dk, dv, 64, 16, 8, 64, 1, 0,
             0.1, None, P, 1 << 30, None) == want


def test_fp8_decode_validation(lib):
    f = lib.fa_decode_paged_fp8
    def call(D=128, ks=None, ksc=P, vsc=P, B=0):
        return f(P, None, P, ks, P, None, ksc, vsc, P, P, P, None, None, B, 1, 8, 2, D, 64, 16, 8, 64, 1, 0,
                 0.1, None, P, 1 << 30, None)
    assert call() == OK
    assert call(D=256) == OK and call(D=512) == OK
    assert call(D=64) == UNSUPPORTED and call(D=192) == UNSUPPORTED and call(D=320) == UNSUPPORTED
    assert call(ks=_st(0, 2 * 2 * 128, 128)) == OK           # K/V interleaved per slot, 16-byte rows
    assert call(ks=_st(0, 8 * 2, 8)) == INVALID              # not a multiple of 16 bytes
    assert call(B=2, ksc=None) == INVALID and call(B=2, vsc=P + 2) == INVALID


def test_fp8_append_validation(lib):
    f = lib.fa_kv_append_fp8
    def call(D=128, ksc=P, B=2, kc=P, ks=None):
        return f(kc, ks, P, None, ksc, P, P, P, P, None, P, None, B, 4, 2, D, 64, 16, 8, None)
    assert call(D=72) == UNSUPPORTED and call(D=600) == UNSUPPORTED
    assert call(ksc=None) == INVALID and call(ksc=P + 1) == INVALID
    assert call(kc=P + 8) == INVALID and call(ks=_st(0, 8, 8)) == INVALID
    assert call(B=0) == OK and call(D=80, B=0) == OK
