"""GQA flash attention for MI355X (gfx950): thin Python binding over libgqafa.so.

Every function below marshals torch tensors into device pointers plus the
current HIP stream and calls the C ABI (include/gqafa.h). All computation
runs in the HIP kernels; nothing here falls back to another implementation.
"""

from __future__ import annotations

import ctypes
import math

import torch

from ._lib import FAError, ScoreMods, check, load  # noqa: F401

__all__ = ["prefill", "decode_paged", "decode_paged_noalloc", "decode_paged_fp8", "decode_workspace_bytes",
           "combine_lse", "kv_append", "kv_append_fp8", "paged_gather", "FAError", "load"]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t, name, dtype, device=None, strided=False):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if strided:
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be 4-D with a unit-stride last dimension")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _lse_out(lse, B, Hq, Sq, dev, return_lse=True):
    """The caller's LSE buffer (checked) or a new one; None when not wanted."""
    if lse is None:
        return torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev) if return_lse else None
    _require(lse, "lse", torch.float32, dev)
    _shape(lse, "lse", (B, Hq, Sq))
    return lse


def _workspace(ws, need, dev):
    """The caller's workspace (checked: a contiguous device buffer of at least
    `need` bytes) or a new one, and its size in bytes."""
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if not ws.is_cuda or ws.device != dev:
        raise ValueError(f"workspace must be on {dev}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
    return ws, nbytes


def _lengths_table(seq_lens, block_table, B, dev):
    _require(seq_lens, "seq_lens", torch.int32, dev)
    _shape(seq_lens, "seq_lens", (B,))
    if block_table is not None:
        _require(block_table, "block_table", torch.int32, dev)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError(f"block_table must be [B={B}, max_pages], got {list(block_table.shape)}")


def _strides(t):
    """(outer, token, head) element strides of a 4-D view, as a C int64[3]."""
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def _mods(softcap, max_bias, sinks, mask, B, Sq, Hq, n_keys, dev):
    """A ScoreMods for the call (None when no modifier is on)."""
    if not softcap and not max_bias and sinks is None and mask is None:
        return None, None
    if sinks is not None:
        _require(sinks, "sinks", torch.float32, dev)
        if sinks.shape != (Hq,):
            raise ValueError("sinks must have shape [Hq]")
    msb = mss = 0
    if mask is not None:
        if mask.dtype != torch.bfloat16 or not mask.is_cuda or mask.device != dev:
            raise TypeError("mask must be a bfloat16 tensor on the inputs' device")
        if mask.dim() != 3 or mask.shape[0] not in (1, B) or mask.shape[1] != Sq or mask.shape[2] < n_keys:
            raise ValueError(f"mask must be [B or 1, Sq, >= {n_keys}]")
        if mask.stride(2) != 1:
            raise ValueError("mask keys must be unit-stride")
        msb = mask.stride(0) if mask.shape[0] > 1 else 0
        mss = mask.stride(1)
    m = ScoreMods(float(softcap or 0.0), float(max_bias or 0.0), _ptr(sinks), _ptr(mask), msb, mss)
    return ctypes.byref(m), m


def prefill(q, k, v, *, causal: bool = True, window: int = 0, scale: float | None = None,
            out=None, lse=None, return_lse: bool = True, softcap: float = 0.0,
            max_bias: float = 0.0, sinks=None, mask=None):
    """q [B,Sq,Hq,Dk], k [B,Skv,Hkv,Dk], v [B,Skv,Hkv,Dv] bf16 ->
    (o [B,Sq,Hq,Dv] bf16, lse [B,Hq,Sq] fp32); head dims multiples of 8 up to 512.

    q, k, v and out may be strided views (e.g. slices of one fused QKV
    tensor); only their last dimension must be unit-stride. softcap,
    max_bias, sinks (device fp32 [Hq]) and mask (bf16 [B or 1, Sq, >= Skv],
    additive, shared by the heads) are the score modifiers of fa_score_mods
    (off by default).
    """
    B, Sq, Hq, Dk = q.shape
    _, Skv, Hkv, _ = k.shape
    Dv = v.shape[3]
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, torch.bfloat16, dev, strided=True)
    if v.shape[:3] != k.shape[:3] or k.shape[0] != B or k.shape[3] != Dk:
        raise ValueError("shape mismatch between q, k and v")
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev, strided=True)
    _shape(out, "out", (B, Sq, Hq, Dv))
    lse = _lse_out(lse, B, Hq, Sq, dev, return_lse)
    mref, _keep = _mods(softcap, max_bias, sinks, mask, B, Sq, Hq, Skv, dev)
    check(load().fa_prefill_strided(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                    _ptr(out), _strides(out), _ptr(lse),
                                    B, Hq, Hkv, Sq, Skv, Dk, Dv, int(bool(causal)), int(window),
                                    float(scale), mref, _stream(dev)))
    return out, lse


def decode_workspace_bytes(B, Sq, Hq, D, max_seq_len, kv_chunk) -> int:
    return int(load().fa_decode_workspace_bytes(B, Sq, Hq, D, max_seq_len, kv_chunk))


def decode_paged(q, kcache, vcache, block_table, seq_lens, *, page_size: int = 16,
                 kv_chunk: int = 256, causal: bool = True, window: int = 0,
                 scale: float | None = None, workspace=None, out=None, lse=None,
                 return_lse: bool = True, softcap: float = 0.0, max_bias: float = 0.0,
                 sinks=None, mask=None):
    """Split-KV decode / verify.

    q [B,Sq,Hq,Dk] bf16; with block_table (int32 [B, max_pages]) the caches are
    [num_pages, page_size, Hkv, Dk or Dv]; without it they are contiguous
    [B, Smax, Hkv, Dk or Dv] (Smax a multiple of page_size). seq_lens int32
    [B]. Returns o [B,Sq,Hq,Dv] and lse [B,Hq,Sq].
    q, the caches and out may be strided views with a unit-stride last
    dimension (e.g. K and V interleaved in one allocation). The score
    modifiers are those of prefill; a mask is [B or 1, Sq, >= max_pages *
    page_size], indexed by token position.
    """
    B, Sq, Hq, Dk = q.shape
    dev = q.device
    _require(q, "q", torch.bfloat16, dev, strided=True)
    _require(kcache, "kcache", torch.bfloat16, dev, strided=True)
    _require(vcache, "vcache", torch.bfloat16, dev, strided=True)
    _lengths_table(seq_lens, block_table, B, dev)
    Dv = vcache.shape[3]
    if vcache.shape[:3] != kcache.shape[:3] or kcache.shape[3] != Dk:
        raise ValueError("kcache / vcache shapes do not match q")
    Hkv = kcache.shape[2]
    num_pages, max_pages = _cache_geometry(kcache, vcache, block_table, page_size, dev, B, same_shape=False)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    need = decode_workspace_bytes(B, Sq, Hq, max(Dk, Dv), max_pages * page_size, kv_chunk)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev, strided=True)
    _shape(out, "out", (B, Sq, Hq, Dv))
    lse = _lse_out(lse, B, Hq, Sq, dev, return_lse)
    mref, _keep = _mods(softcap, max_bias, sinks, mask, B, Sq, Hq, max_pages * page_size, dev)
    check(load().fa_decode_paged_strided(_ptr(q), _strides(q), _ptr(kcache), _strides(kcache),
                                         _ptr(vcache), _strides(vcache), _ptr(block_table),
                                         _ptr(seq_lens), _ptr(out), _strides(out), _ptr(lse),
                                         B, Sq, Hq, Hkv, Dk, Dv, num_pages, page_size, max_pages, kv_chunk,
                                         int(bool(causal)), int(window), float(scale), mref,
                                         _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse


def decode_paged_noalloc(q, kcache, vcache, block_table, seq_lens, *, page_size: int = 16,
                         kv_chunk: int = 256, causal: bool = True, window: int = 0,
                         scale: float | None = None, out=None, lse=None, softcap: float = 0.0,
                         max_bias: float = 0.0, sinks=None, mask=None):
    """decode_paged through fa_decode_paged_noalloc: the split partials go to
    the library's static device buffer instead of a workspace, so the C call
    allocates nothing (out and lse must then be given by a caller that cannot
    allocate either). Calls on one GPU share the buffer: order them on one
    stream. Raises FAError(FA_ERR_SCRATCH) when the call's partials exceed
    the buffer (NOALLOC_SCRATCH_BYTES)."""
    from ._lib import NOALLOC_SCRATCH_BYTES  # noqa: F401  (documented limit)

    B, Sq, Hq, Dk = q.shape
    dev = q.device
    _require(q, "q", torch.bfloat16, dev, strided=True)
    _require(kcache, "kcache", torch.bfloat16, dev, strided=True)
    _require(vcache, "vcache", torch.bfloat16, dev, strided=True)
    _lengths_table(seq_lens, block_table, B, dev)
    Dv = vcache.shape[3]
    if vcache.shape[:3] != kcache.shape[:3] or kcache.shape[3] != Dk:
        raise ValueError("kcache / vcache shapes do not match q")
    Hkv = kcache.shape[2]
    num_pages, max_pages = _cache_geometry(kcache, vcache, block_table, page_size, dev, B, same_shape=False)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev, strided=True)
    _shape(out, "out", (B, Sq, Hq, Dv))
    lse = _lse_out(lse, B, Hq, Sq, dev)
    mref, _keep = _mods(softcap, max_bias, sinks, mask, B, Sq, Hq, max_pages * page_size, dev)
    check(load().fa_decode_paged_noalloc(_ptr(q), _strides(q), _ptr(kcache), _strides(kcache),
                                         _ptr(vcache), _strides(vcache), _ptr(block_table),
                                         _ptr(seq_lens), _ptr(out), _strides(out), _ptr(lse),
                                         B, Sq, Hq, Hkv, Dk, Dv, num_pages, page_size, max_pages, kv_chunk,
                                         int(bool(causal)), int(window), float(scale), mref, _stream(dev)))
    return out, lse


def _cache_geometry(kcache, vcache, block_table, page_size, dev, B, same_shape=True):
    """(num_pages, max_pages) of a paged cache [num_pages, page_size, Hkv, D]
    with its block table [B, max_pages], or of a contiguous cache
    [B, Smax, Hkv, D] (num_pages 0)."""
    if same_shape and vcache.shape != kcache.shape:
        raise ValueError("kcache and vcache differ in shape")
    if block_table is not None:
        _require(block_table, "block_table", torch.int32, dev)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError(f"block_table must be [B={B}, max_pages], got {list(block_table.shape)}")
        if kcache.shape[1] != page_size:
            raise ValueError("cache page dimension differs from page_size")
        return kcache.shape[0], block_table.shape[1]
    if kcache.shape[0] != B:
        raise ValueError(f"a contiguous cache must be [B={B}, Smax, Hkv, D], got {list(kcache.shape)}")
    if kcache.shape[1] % page_size:
        raise ValueError("contiguous cache length must be a multiple of page_size")
    return 0, kcache.shape[1] // page_size


def decode_paged_fp8(q, kcache, vcache, k_scale, v_scale, block_table, seq_lens, *, page_size: int = 16,
                     kv_chunk: int = 256, causal: bool = True, window: int = 0,
                     scale: float | None = None, workspace=None, out=None, lse=None,
                     return_lse: bool = True, softcap: float = 0.0, max_bias: float = 0.0,
                     sinks=None, mask=None):
    """Split-KV decode / verify over fp8 (OCP e4m3) caches.

    kcache / vcache: uint8 [num_pages, page_size, Hkv, D] with block_table,
    else [B, Smax, Hkv, D], D = 128, 256 or 512 (views with a unit-stride
    last dimension); k_scale / v_scale: fp32 [Hkv] dequantisation scales
    (value = e4m3(byte) * scale). q and the result are bf16 [B, Sq, Hq, D];
    the rest is as decode_paged.
    """
    B, Sq, Hq, D = q.shape
    dev = q.device
    _require(q, "q", torch.bfloat16, dev, strided=True)
    _require(kcache, "kcache", torch.uint8, dev, strided=True)
    _require(vcache, "vcache", torch.uint8, dev, strided=True)
    _require(k_scale, "k_scale", torch.float32, dev)
    _require(v_scale, "v_scale", torch.float32, dev)
    _lengths_table(seq_lens, block_table, B, dev)
    Hkv = kcache.shape[2]
    if kcache.shape[3] != D or k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
        raise ValueError("cache head dim or scale shape does not match")
    num_pages, max_pages = _cache_geometry(kcache, vcache, block_table, page_size, dev, B)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_bytes(B, Sq, Hq, D, max_pages * page_size, kv_chunk)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev, strided=True)
    _shape(out, "out", (B, Sq, Hq, D))
    lse = _lse_out(lse, B, Hq, Sq, dev, return_lse)
    mref, _keep = _mods(softcap, max_bias, sinks, mask, B, Sq, Hq, max_pages * page_size, dev)
    check(load().fa_decode_paged_fp8(_ptr(q), _strides(q), _ptr(kcache), _strides(kcache),
                                     _ptr(vcache), _strides(vcache), _ptr(k_scale), _ptr(v_scale),
                                     _ptr(block_table), _ptr(seq_lens), _ptr(out), _strides(out), _ptr(lse),
                                     B, Sq, Hq, Hkv, D, num_pages, page_size, max_pages, kv_chunk,
                                     int(bool(causal)), int(window), float(scale), mref,
                                     _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse


def kv_append_fp8(kcache, vcache, k_scale, v_scale, block_table, seq_lens, knew, vnew, *,
                  page_size: int = 16):
    """Quantise knew/vnew (bf16 [B, Snew, Hkv, D]) to e4m3 by the heads'
    scales and write them into the uint8 caches in place (placement as
    kv_append)."""
    B, Snew, Hkv, D = knew.shape
    dev = knew.device
    for t, n in ((knew, "knew"), (vnew, "vnew")):
        _require(t, n, torch.bfloat16, dev, strided=True)
    for t, n in ((kcache, "kcache"), (vcache, "vcache")):
        _require(t, n, torch.uint8, dev, strided=True)
    _require(k_scale, "k_scale", torch.float32, dev)
    _require(v_scale, "v_scale", torch.float32, dev)
    _lengths_table(seq_lens, block_table, B, dev)
    if vnew.shape != knew.shape or kcache.shape[2:] != (Hkv, D):
        raise ValueError("shape mismatch between caches and new rows")
    if k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
        raise ValueError("k_scale and v_scale must be [Hkv]")
    num_pages, max_pages = _cache_geometry(kcache, vcache, block_table, page_size, dev, B)
    check(load().fa_kv_append_fp8(_ptr(kcache), _strides(kcache), _ptr(vcache), _strides(vcache),
                                  _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
                                  _ptr(knew), _strides(knew), _ptr(vnew), _strides(vnew),
                                  B, Snew, Hkv, D, num_pages, page_size, max_pages, _stream(dev)))


def combine_lse(o_part, lse_part, n_chunks=None, *, out=None, lse=None):
    """o_part fp32 [B,Hq,Sq,C,D], lse_part fp32 [B,Hq,Sq,C] -> (o bf16 [B,Sq,Hq,D], lse [B,Hq,Sq])."""
    B, Hq, Sq, C, D = o_part.shape
    dev = o_part.device
    _require(o_part, "o_part", torch.float32, dev)
    _require(lse_part, "lse_part", torch.float32, dev)
    _shape(lse_part, "lse_part", (B, Hq, Sq, C))
    if n_chunks is not None:
        _require(n_chunks, "n_chunks", torch.int32, dev)
        _shape(n_chunks, "n_chunks", (B,))
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    _shape(out, "out", (B, Sq, Hq, D))
    lse = _lse_out(lse, B, Hq, Sq, dev)
    check(load().fa_combine_lse(_ptr(o_part), _ptr(lse_part), _ptr(n_chunks), C, _ptr(out),
                                _ptr(lse), B, Sq, Hq, D, _stream(dev)))
    return out, lse


def kv_append(kcache, vcache, block_table, seq_lens, knew, vnew, *, page_size: int = 16):
    """Write knew/vnew [B, Snew, Hkv, D] into the caches in place.

    Row i of sequence b goes to token seq_lens[b] - Snew + i (seq_lens counts
    the new rows). With block_table the caches are [num_pages, page_size,
    Hkv, D], else contiguous [B, Smax, Hkv, D]. Every tensor may be a strided
    view with a unit-stride last dimension.
    """
    B, Snew, Hkv, Dk = knew.shape
    Dv = vnew.shape[3]
    dev = knew.device
    for t, n in ((kcache, "kcache"), (vcache, "vcache"), (knew, "knew"), (vnew, "vnew")):
        _require(t, n, torch.bfloat16, dev, strided=True)
    _lengths_table(seq_lens, block_table, B, dev)
    if (vnew.shape[:3] != knew.shape[:3] or vcache.shape[:3] != kcache.shape[:3]
            or kcache.shape[2:] != (Hkv, Dk) or vcache.shape[3] != Dv):
        raise ValueError("shape mismatch between caches and new rows")
    num_pages, max_pages = _cache_geometry(kcache, vcache, block_table, page_size, dev, B, same_shape=False)
    check(load().fa_kv_append(_ptr(kcache), _strides(kcache), _ptr(vcache), _strides(vcache),
                              _ptr(block_table), _ptr(seq_lens), _ptr(knew), _strides(knew),
                              _ptr(vnew), _strides(vnew), B, Snew, Hkv, Dk, Dv, num_pages, page_size,
                              max_pages, _stream(dev)))


def paged_gather(cache, block_table, seq_lens, *, out=None):
    """Test hook: dense [B, max_pages*page_size, Hkv, D] copy of a paged cache."""
    P, ps, Hkv, D = cache.shape
    B, max_pages = block_table.shape
    dev = cache.device
    _require(cache, "cache", torch.bfloat16, dev)
    _lengths_table(seq_lens, block_table, B, dev)
    if out is None:
        out = torch.empty((B, max_pages * ps, Hkv, D), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    _shape(out, "out", (B, max_pages * ps, Hkv, D))
    check(load().fa_paged_gather(_ptr(cache), _ptr(block_table), _ptr(seq_lens), _ptr(out),
                                 B, Hkv, D, P, ps, max_pages, _stream(dev)))
    return out
