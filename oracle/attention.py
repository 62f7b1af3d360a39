"""Plain fp64 CPU oracle for grouped-query scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. This module is the independent check on the HIP
path. Only the test suite, the package smoke check and the benchmark's CPU
baseline leg may import it. The product path never calls it, and it imports
nothing from the GPU package.

What it computes: the plain definition of attention, softmax(Q K^T * scale +
mask) V, written as the two passes that the flash-attention pages reduce to
(a row maximum, then an exponent sum and a weighted sum of V). The pages
describe this computation without printing it:

* llama.cpp PR 28507 (Vulkan K/V shared-memory staging on AMD RDNA),
  section Summary: the "scalar flash-attention path"; section Measurements:
  SWA layers with head size 256 and global layers with head size 512; the
  RX 6900 XT test report: GQA 8, and the FLASH_ATTN_EXT case parameters
  (head sizes, head count, broadcast ratio nr23, kv length, mask).
* beellama.cpp PR 149 (Make KVarN usable on ROCm RDNA3), section Overview:
  every tile of the streaming softmax publishes its (max, rowsum) pair, and
  split tiles are merged from those pairs; the review notes that a combine
  kernel merges partial results when the KV range is split
  ("parallel_blocks > 1").

Readings taken where the pages are silent (each one is listed with its reason
in the design notes of the repository):

* Head grouping: query head h reads KV head h // (Hq // Hkv).
* Causal alignment is bottom-right: query row i of a sequence with Skv_b keys
  sits at absolute position p_i = i + Skv_b - Sq.
* Visible keys of row i: 0 <= j < Skv_b, and j <= p_i when causal, and
  p_i - j < window when window > 0 (exactly `window` keys up to and including
  the diagonal). A window is only meaningful with causal masking.
* LSE is the natural log of sum_j exp(scale * q . k_j) over visible keys.
* A row with no visible key has O = 0 and LSE = -inf.
* Split-KV partials are normalised by their own row sum and carry their own
  LSE; the merge is LSE = M + ln sum_c exp(LSE_c - M), O = sum_c
  exp(LSE_c - LSE) O_c, with M = max_c LSE_c. A chunk with LSE_c = -inf has
  weight 0; when every chunk is empty the row is O = 0, LSE = -inf.

Score modifiers, named (without their formulas) by the FLASH_ATTN_EXT case
parameters of the llama.cpp PR 28507 test report (mask, sinks, max_bias,
logit_softcap); the formulas are readings of this build:

* logit_softcap c > 0: the scaled score s = scale * q . k becomes
  c * tanh(s / c).
* max_bias > 0 (ALiBi): query head h adds slope_h * (j - p_i) to the score
  of key j, with n = 2^floor(log2 Hq), m0 = 2^(-max_bias / n),
  m1 = 2^(-max_bias / (2 n)), slope_h = m0^(h + 1) for h < n and
  m1^(2 (h - n) + 1) otherwise (the geometric slopes of ALiBi).
* sinks: one extra logit sink_h per query head joins the softmax
  denominator and carries no value: l = sum_j exp(s_j) + exp(sink_h),
  O = sum_j exp(s_j) v_j / l, LSE = ln l. A row with no visible key then has
  O = 0 and LSE = sink_h.

* mask (the test report's "mask" case parameter; its layout is a reading of
  this build): an additive tensor [B or 1, Sq, >= Skv] of per-(sequence,
  query row, key) values, shared by every head, added to the score of key j
  of query row i (j is the key's index in the sequence, i the row's index
  among the Sq query rows); -inf hides a key. A leading dimension of 1 is
  shared by every sequence. Keys at or beyond a sequence's length stay
  hidden whatever the mask holds.

The softcap applies first, then the ALiBi bias, then the additive mask, and
last the causal / window / length visibility.

Every floating-point value is widened to float64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "to_f64",
    "visible_mask",
    "attention_ref",
    "paged_gather_ref",
    "decode_paged_ref",
    "partial_attention_ref",
    "combine_ref",
    "kv_append_ref",
    "alibi_slopes",
]


def to_f64(x) -> np.ndarray:
    """Widen a numpy array or a CPU torch tensor (any float dtype) to fp64.

    bfloat16 values are exactly representable in float64, so this step adds
    no rounding.
    """
    if hasattr(x, "detach"):  # torch tensor, without importing torch here
        x = x.detach().to("cpu")
        x = x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def visible_mask(rows: np.ndarray, sq: int, skv: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [len(rows), skv] mask of the keys each query row may attend to.

    rows are query-row indices 0..sq-1 of one sequence whose key count is
    skv. Causal masking is bottom-right aligned (row i is at position
    i + skv - sq). With window > 0, key j is visible only if
    position - j < window.
    """
    rows = np.asarray(rows, dtype=np.int64)
    pos = rows + (skv - sq)
    j = np.arange(skv, dtype=np.int64)
    vis = np.ones((rows.size, skv), dtype=bool)
    if causal:
        vis &= j[None, :] <= pos[:, None]
        if window > 0:
            vis &= (pos[:, None] - j[None, :]) < window
    return vis


def alibi_slopes(hq: int, max_bias: float) -> np.ndarray:
    """ALiBi slope of each of hq query heads (all zero when max_bias <= 0)."""
    if max_bias <= 0:
        return np.zeros(hq)
    n = 1 << int(np.floor(np.log2(hq)))
    m0 = 2.0 ** (-max_bias / n)
    m1 = 2.0 ** (-max_bias / (2.0 * n))
    return np.array([m0 ** (h + 1) if h < n else m1 ** (2 * (h - n) + 1) for h in range(hq)])


def _attend_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray, scale: float,
                 softcap: float = 0.0, bias=None, sink: float = -np.inf, mask=None):
    """Two-pass softmax attention for a block of rows of one query head.

    q_rows [R, D], k and v [S, D], vis [R, S] boolean; optional softcap,
    ALiBi bias [R, S], sink logit and additive mask [R, S]. Returns O [R, D]
    and LSE [R], both float64.

    Pass 1 takes the maximum over the visible scores of each row (and the
    sink); pass 2 sums exp(score - max), plus exp(sink - max), and the
    score weights times V.
    """
    s = scale * (q_rows @ k.T)                      # scores, [R, S]
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    if bias is not None:
        s = s + bias
    if mask is not None:
        s = s + mask
    s = np.where(vis, s, -np.inf)
    # pass 1: row maximum over visible keys and the sink (-inf when neither)
    m = np.max(s, axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    m = np.maximum(m, sink)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    # pass 2: exponent sum (with the sink's term) and weighted sum of V
    e = np.exp(s - m_safe[:, None])                 # masked keys give exp(-inf) = 0
    l = e.sum(axis=1) + np.exp(sink - m_safe)
    num = e @ v
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(empty[:, None], 0.0, num / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return o, lse


def attention_ref(q, k, v, *, causal: bool, window: int = 0, scale: float,
                  seq_lens=None, rows=None, heads=None, batches=None, row_block: int = 512,
                  softcap: float = 0.0, max_bias: float = 0.0, sinks=None, mask=None):
    """Reference attention for grouped-query heads.

    q [B, Sq, Hq, Dk]; k [B, Skv, Hkv, Dk]; v [B, Skv, Hkv, Dv] (numpy or
    CPU torch, any float dtype; the key and value head dims may differ). seq_lens (optional, length B) gives the number of valid keys
    Skv_b <= Skv per sequence; keys at or beyond it are ignored. rows, heads
    and batches optionally restrict which query rows / query heads /
    sequences are computed (for sampling at large sizes); the result still
    has the full shape and the rows not computed hold NaN. softcap,
    max_bias, sinks ([Hq] logits or None) and mask ([B or 1, Sq, >= Skv]
    additive, or None) are the score modifiers of the module docstring (all
    off by default).

    Returns O [B, Sq, Hq, Dv] and LSE [B, Hq, Sq] in float64.
    """
    q = to_f64(q)
    k = to_f64(k)
    v = to_f64(v)
    B, Sq, Hq, Dk = q.shape
    _, Skv, Hkv, Dk2 = k.shape
    Dv = v.shape[3]
    assert k.shape[0] == B and v.shape[:3] == k.shape[:3] and Dk2 == Dk
    assert Hq % Hkv == 0
    group = Hq // Hkv
    if seq_lens is None:
        seq_lens = [Skv] * B
    seq_lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    batches = range(B) if batches is None else batches

    slopes = alibi_slopes(Hq, max_bias)
    sink_v = None if sinks is None else to_f64(sinks).reshape(-1)
    mask_v = None if mask is None else to_f64(mask)
    if mask_v is not None:
        assert mask_v.ndim == 3 and mask_v.shape[0] in (1, B) and mask_v.shape[1] == Sq
        assert mask_v.shape[2] >= Skv
    o = np.full((B, Sq, Hq, Dv), np.nan)
    lse = np.full((B, Hq, Sq), np.nan)
    for b in batches:
        skv = seq_lens[b]
        assert 0 <= skv <= Skv
        for h in heads:
            g = h // group                       # KV head shared by this query head
            kb = k[b, :skv, g, :]
            vb = v[b, :skv, g, :]
            for r0 in range(0, rows.size, row_block):
                rr = rows[r0:r0 + row_block]
                vis = visible_mask(rr, Sq, skv, causal, window)
                bias = None
                if max_bias > 0:
                    pos = rr + (skv - Sq)            # absolute positions of the rows
                    bias = slopes[h] * (np.arange(skv)[None, :] - pos[:, None])
                sink = -np.inf if sink_v is None else float(sink_v[h])
                mrows = None
                if mask_v is not None:
                    mrows = mask_v[b if mask_v.shape[0] > 1 else 0][rr, :skv]
                ob, lb = _attend_rows(q[b, rr, h, :], kb, vb, vis, scale, softcap, bias, sink, mrows)
                o[b, rr, h, :] = ob
                lse[b, h, rr] = lb
    return o, lse


def paged_gather_ref(cache, block_table, seq_lens, page_size: int, max_len: int | None = None):
    """Gather a paged KV cache into a dense [B, max_len, Hkv, D] array.

    cache [num_pages, page_size, Hkv, D]; block_table [B, pages_per_seq]
    int; token t of sequence b lives at page block_table[b, t // page_size],
    slot t % page_size. Positions at or beyond seq_lens[b] are left as zero.
    Returns the same dtype as the cache (no arithmetic: a pure index map).
    """
    cache = np.asarray(cache) if not hasattr(cache, "detach") else cache.detach().cpu()
    bt = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    B = bt.shape[0]
    if max_len is None:
        max_len = bt.shape[1] * page_size
    hkv, d = cache.shape[2], cache.shape[3]
    if hasattr(cache, "new_zeros"):
        out = cache.new_zeros((B, max_len, hkv, d))
    else:
        out = np.zeros((B, max_len, hkv, d), dtype=cache.dtype)
    for b in range(B):
        for t in range(int(lens[b])):
            page = int(bt[b, t // page_size])
            out[b, t] = cache[page, t % page_size]
    return out


def decode_paged_ref(q, kcache, vcache, block_table, seq_lens, *, page_size: int,
                     causal: bool, window: int = 0, scale: float, rows=None, heads=None,
                     softcap: float = 0.0, max_bias: float = 0.0, sinks=None, mask=None):
    """Reference decode / speculative verify over a paged (or contiguous) cache.

    q [B, Sq, Hq, D] holds the Sq newest query rows of each sequence (Sq = 1
    for plain decode). When block_table is None the caches are contiguous
    [B, Smax, Hkv, D]; otherwise they are [num_pages, page_size, Hkv, D] and
    are gathered through the table first. Row i of sequence b is at
    position seq_lens[b] - Sq + i. mask, if given, is [B or 1, Sq, M]
    indexed by token position in the sequence, M >= every seq_lens[b].
    """
    lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    if block_table is None:
        k = kcache
        v = vcache
    else:
        max_len = max(lens) if lens else 0
        k = paged_gather_ref(kcache, block_table, lens, page_size, max_len)
        v = paged_gather_ref(vcache, block_table, lens, page_size, max_len)
    if mask is not None:
        # the gathered caches hold max(lens) keys; keys past each length are hidden
        kmax = k.shape[1]
        mask = to_f64(mask)
        assert mask.shape[2] >= max(lens, default=0)
        mask = mask[:, :, :kmax] if mask.shape[2] >= kmax else \
            np.concatenate([mask, np.zeros(mask.shape[:2] + (kmax - mask.shape[2],))], axis=2)
    return attention_ref(q, k, v, causal=causal, window=window, scale=scale,
                         seq_lens=lens, rows=rows, heads=heads, softcap=softcap,
                         max_bias=max_bias, sinks=sinks, mask=mask)


def partial_attention_ref(q, k, v, *, causal: bool, window: int = 0, scale: float,
                          seq_lens=None, chunk: int):
    """Split-KV partials: attention restricted to key chunks [c*chunk, (c+1)*chunk).

    Returns O_c [B, Hq, Sq, n_chunks, D] (each normalised by its own row
    sum) and LSE_c [B, Hq, Sq, n_chunks], computed with the same visibility
    rule as the whole; chunks past a sequence's end are empty (O_c = 0,
    LSE_c = -inf). This is the per-tile (max, rowsum) publication the merge
    consumes.
    """
    q = to_f64(q)
    k = to_f64(k)
    v = to_f64(v)
    B, Sq, Hq, _ = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    D = v.shape[3]
    group = Hq // Hkv
    if seq_lens is None:
        seq_lens = [Skv] * B
    lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    n_chunks = max(1, -(-Skv // chunk))
    o = np.zeros((B, Hq, Sq, n_chunks, D))
    lse = np.full((B, Hq, Sq, n_chunks), -np.inf)
    rows = np.arange(Sq)
    for b in range(B):
        vis_all = visible_mask(rows, Sq, lens[b], causal, window)
        for h in range(Hq):
            g = h // group
            for c in range(n_chunks):
                lo, hi = c * chunk, min((c + 1) * chunk, lens[b])
                if hi <= lo:
                    continue
                ob, lb = _attend_rows(q[b, :, h, :], k[b, lo:hi, g, :], v[b, lo:hi, g, :],
                                      vis_all[:, lo:hi], scale)
                o[b, h, :, c, :] = ob
                lse[b, h, :, c] = lb
    return o, lse


def combine_ref(o_part, lse_part, n_chunks=None, sinks=None):
    """Merge split-KV partials by their log-sum-exp.

    o_part [B, Hq, Sq, C, D], lse_part [B, Hq, Sq, C]; n_chunks (optional,
    length B) limits how many leading chunks of sequence b are merged.
    sinks ([Hq] or None) adds each head's sink as one more partial with
    LSE = sink_h and O = 0 (its logit joins the denominator, no value).
    Returns O [B, Sq, Hq, D] and LSE [B, Hq, Sq] in float64.
    """
    o_part = to_f64(o_part)
    lse_part = to_f64(lse_part)
    B, Hq, Sq, C, D = o_part.shape
    if n_chunks is None:
        n_chunks = [C] * B
    if sinks is not None:
        sk = to_f64(sinks).reshape(1, Hq, 1, 1) * np.ones((B, Hq, Sq, 1))
        o_part = np.concatenate([o_part, np.zeros((B, Hq, Sq, 1, D))], axis=3)
        # the sink goes right after each sequence's merged chunks
        lp = np.full((B, Hq, Sq, C + 1), -np.inf)
        for b in range(B):
            n = max(0, min(int(n_chunks[b]), C))
            lp[b, :, :, :n] = lse_part[b, :, :, :n]
            lp[b, :, :, n] = sk[b, :, :, 0]
            o_part[b, :, :, n, :] = 0.0
            if n < C:
                o_part[b, :, :, n + 1:, :] = 0.0
        lse_part = lp
        n_chunks = [max(0, min(int(x), C)) + 1 for x in n_chunks]
        C = C + 1
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        n = int(n_chunks[b])
        if n <= 0:
            continue
        lp = lse_part[b, :, :, :n]                       # [Hq, Sq, n]
        M = np.max(lp, axis=-1)                          # [Hq, Sq]
        empty = ~np.isfinite(M)
        M_safe = np.where(empty, 0.0, M)
        w = np.exp(lp - M_safe[..., None])               # exp(-inf) = 0 for empty chunks
        tot = w.sum(axis=-1)
        with np.errstate(divide="ignore", invalid="ignore"):
            L = np.where(empty, -np.inf, M_safe + np.log(np.where(empty, 1.0, tot)))
            wn = np.where(empty[..., None], 0.0, w / np.where(empty, 1.0, tot)[..., None])
        ob = np.einsum("hsc,hscd->hsd", wn, o_part[b, :, :, :n, :])
        o[b] = np.transpose(ob, (1, 0, 2))
        lse[b] = L
    return o, lse


def kv_append_ref(kcache, vcache, block_table, seq_lens, knew, vnew, *, page_size: int,
                  num_pages: int | None = None):
    """Write the Snew newest K/V rows of each sequence into copies of the caches.

    A pure index map, the step before a decode call over the same cache.
    seq_lens counts the tokens in each cache after the append (the decode
    convention), so new row i of sequence b lands at token
    t = len_b - Snew + i, with len_b clamped to [0, pages_per_seq *
    page_size]. With block_table [B, pages_per_seq] the caches are
    [num_pages, page_size, Hkv, D] and token t lives at page
    block_table[b, t // page_size], slot t % page_size; with block_table None
    they are [B, Smax, Hkv, D]. Rows with t < 0, and rows whose page is
    outside [0, num_pages), are not written (readings of this build: the
    pages do not describe the append). Returns (kcache', vcache').
    """
    def copy(x):
        return x.clone() if hasattr(x, "clone") else np.array(x, copy=True)

    kc, vc = copy(kcache), copy(vcache)
    lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    B, snew = knew.shape[0], knew.shape[1]
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
                kc[b, t] = knew[b, i]
                vc[b, t] = vnew[b, i]
            else:
                page = int(bt[b, t // page_size])
                if page < 0 or page >= num_pages:
                    continue
                kc[page, t % page_size] = knew[b, i]
                vc[page, t % page_size] = vnew[b, i]
    return kc, vc
