"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and builds index tables; it holds none
of the attention arithmetic, so both the HIP path and the fp64 oracle can be
fed from it without sharing any of the method.

Recipe (one torch CPU generator per workload, seeded; values drawn as fp32
N(0, 1) and rounded to bfloat16; draw order q, k, v, lengths, page
permutation):

  prefill_c1   B=1  Hq=2  Hkv=1 Sq=Skv=128  D=64  causal               seed 1001
  prefill_c2   B=2  Hq=32 Hkv=8 Sq=Skv=4096 D=128 causal               seed 1002
  decode_c3    B=16 Sq=1 Hq=32 Hkv=8 D=128, contiguous cache of 16384
               slots, lengths uniform in [1024, 16384], 256-token split   seed 1003
  prefill_c4a  B=1  Hq=16 Hkv=8 S=8192 D=256 causal, window 1024        seed 1004
  prefill_c4b  B=1  Hq=16 Hkv=8 S=8192 D=512 causal (drawn after c4a)   seed 1004
  verify_c5    B=4  Sq=8 Hq=64 Hkv=8 D=128, paged cache of 16-token
               pages, 32768 tokens per sequence, block table a random
               permutation of the 8192 physical pages                    seed 1005
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BF16 = torch.bfloat16


@dataclass(frozen=True)
class PrefillShape:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    causal: bool = True
    window: int = 0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


@dataclass(frozen=True)
class DecodeShape:
    name: str
    B: int
    Sq: int
    Hq: int
    Hkv: int
    D: int
    page_size: int          # 0 = contiguous cache (no block table)
    max_len: int            # cache slots per sequence
    len_lo: int             # lengths drawn uniformly in [len_lo, len_hi]
    len_hi: int
    kv_chunk: int
    causal: bool = True
    window: int = 0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


C1 = PrefillShape("prefill_c1", B=1, Hq=2, Hkv=1, Sq=128, Skv=128, D=64, seed=1001)
C2 = PrefillShape("prefill_c2", B=2, Hq=32, Hkv=8, Sq=4096, Skv=4096, D=128, seed=1002)
C4A = PrefillShape("prefill_c4a", B=1, Hq=16, Hkv=8, Sq=8192, Skv=8192, D=256, window=1024, seed=1004)
C4B = PrefillShape("prefill_c4b", B=1, Hq=16, Hkv=8, Sq=8192, Skv=8192, D=512, seed=1004)
C3 = DecodeShape("decode_c3", B=16, Sq=1, Hq=32, Hkv=8, D=128, page_size=0, max_len=16384,
                 len_lo=1024, len_hi=16384, kv_chunk=256, seed=1003)
C5 = DecodeShape("verify_c5", B=4, Sq=8, Hq=64, Hkv=8, D=128, page_size=16, max_len=32768,
                 len_lo=32768, len_hi=32768, kv_chunk=1024, seed=1005)

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4A, C4B, C5)}


def _randn(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(BF16)


def prefill_inputs(shape: PrefillShape, gen: torch.Generator | None = None):
    """q [B,Sq,Hq,D], k and v [B,Skv,Hkv,D], bf16 CPU tensors."""
    if gen is None:
        gen = torch.Generator("cpu").manual_seed(shape.seed)
    q = _randn(gen, (shape.B, shape.Sq, shape.Hq, shape.D))
    k = _randn(gen, (shape.B, shape.Skv, shape.Hkv, shape.D))
    v = _randn(gen, (shape.B, shape.Skv, shape.Hkv, shape.D))
    return q, k, v


def c4_inputs():
    """The two large-head layers are drawn in sequence from one generator."""
    gen = torch.Generator("cpu").manual_seed(C4A.seed)
    a = prefill_inputs(C4A, gen)
    b = prefill_inputs(C4B, gen)
    return a, b


def random_inputs(B, Sq, Skv, Hq, Hkv, D, seed, dist="normal"):
    """Small seeded prefill inputs for parity grids (same recipe, any shape)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _randn(gen, (B, Sq, Hq, D))
    k = _randn(gen, (B, Skv, Hkv, D))
    v = _randn(gen, (B, Skv, Hkv, D))
    return q, k, v


@dataclass
class DecodeInputs:
    q: torch.Tensor               # [B, Sq, Hq, D] bf16
    kcache: torch.Tensor          # contiguous [B, max_len, Hkv, D] or paged [P, page, Hkv, D]
    vcache: torch.Tensor
    block_table: torch.Tensor | None   # int32 [B, max_pages] or None
    seq_lens: torch.Tensor        # int32 [B]
    extra: dict = field(default_factory=dict)


def decode_inputs(shape: DecodeShape, gen: torch.Generator | None = None,
                  poison_tail: bool = False) -> DecodeInputs:
    """Seeded decode / verify inputs.

    For a contiguous cache (page_size 0) the caches are [B, max_len, Hkv, D].
    For a paged cache there are B * max_len / page_size physical pages and the
    block table is one random permutation of them, reshaped to
    [B, max_len / page_size]. With poison_tail, cache slots at or beyond a
    sequence's length are filled with NaN so any read past the end shows.
    """
    if gen is None:
        gen = torch.Generator("cpu").manual_seed(shape.seed)
    B, D, Hkv = shape.B, shape.D, shape.Hkv
    q = _randn(gen, (B, shape.Sq, shape.Hq, D))
    if shape.page_size == 0:
        kc = _randn(gen, (B, shape.max_len, Hkv, D))
        vc = _randn(gen, (B, shape.max_len, Hkv, D))
    else:
        assert shape.max_len % shape.page_size == 0
        n_pages = B * shape.max_len // shape.page_size
        kc = _randn(gen, (n_pages, shape.page_size, Hkv, D))
        vc = _randn(gen, (n_pages, shape.page_size, Hkv, D))
    lens = torch.randint(shape.len_lo, shape.len_hi + 1, (B,), generator=gen, dtype=torch.int64)
    lens = lens.to(torch.int32)
    table = None
    if shape.page_size:
        ppseq = shape.max_len // shape.page_size
        perm = torch.randperm(B * ppseq, generator=gen)
        table = perm.view(B, ppseq).to(torch.int32).contiguous()
    if poison_tail:
        nan = float("nan")
        for b in range(B):
            n = int(lens[b])
            if table is None:
                kc[b, n:] = nan
                vc[b, n:] = nan
            else:
                ps = shape.page_size
                for t in range(n, shape.max_len):
                    pg = int(table[b, t // ps])
                    kc[pg, t % ps] = nan
                    vc[pg, t % ps] = nan
    return DecodeInputs(q, kc, vc, table, lens)
