// Flash-attention tile kernel for gfx950: bf16 MFMA with fp32 accumulators,
// K/V tiles streamed into swizzled LDS by direct global->LDS loads, online
// softmax in registers.
//
// Method: the streaming-softmax attention of the scalar flash-attention path
// (llama.cpp PR 28507, Summary) with K/V staged in on-chip memory once per
// workgroup and reused by all its query rows (same page, Measurements: the
// gain grows with context depth). Every partial publishes its row (max,
// rowsum) as an LSE (beellama.cpp PR 149, Overview: whole-tile blocks must
// publish their meta or the merge drops them). fp32 accumulation of both
// products follows the same page (fp16 accumulation compounded over depth into
// a KL-divergence collapse). Every XOR swizzle stays inside its row for every
// head dim (the AstrAI commit log fixed a swizzle mask wider than the chunk
// count of a row).
//
// Layout of the work. For one KV head g of sequence b the "rows" of the
// problem are the pairs (query position i, query head h in g's group),
// numbered r = i * G + (h - g * G). Rows of one position are adjacent in
// memory ([B, Sq, Hq, D]), so a block of 32 rows is a few positions times the
// whole head group, and every row of a workgroup reads the same K/V tile.
//
// Each wave owns 32 rows. It computes S^T = K Q^T for a tile of keys with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T from registers), so
// each lane holds the scores of ONE query row for 16 keys of every 32-key
// block: the row max is an in-lane max plus one exchange with the lane 32
// away, and the row sum needs no cross-lane step until the end. The score
// accumulators, rounded to bf16, are already the B operand of O^T = V^T P^T;
// the V^T operand comes straight from the row-major V tile through the
// transposing LDS read ds_read_b64_tr_b16.
//
// Staging. K and V tiles are copied straight into LDS, 16 bytes per lane
// (global_load_lds_dwordx4 in the split kernels, buffer_load_dwordx4 ... lds
// in prefill): each lane's load lands at (segment base + 16 * lane), so a
// swizzled LDS layout is produced by choosing WHICH global chunk each lane
// fetches. A ring
// of NBUF LDS buffers per operand (separate objects; two for bf16 tiles) lets
// the loads of the next tiles run while tile t is computed, with one barrier
// per tile; no registers hold the tile in flight.
//
// D split (DS = 2, used for the large head dims): two waves share the same 32
// rows; each holds half of Q's head dim and half of O. Each computes the
// partial S^T over its half of the contraction, the pair adds the two halves
// through LDS (in the same order in both waves, so both hold bit-identical
// scores and run identical softmax), and each then accumulates its half of O.
//
// Split-KV mode (decode and speculative verify) is bound by HBM bandwidth. A
// persistent grid of as many workgroups as the GPU holds at once streams the
// K/V tiles of all (sequence, block of rows) in one global order. The grid is
// cut into sets of Hkv workgroups, member g of a set taking KV head g, and
// each set takes an equal contiguous range of tiles, so every slot streams
// until the end and none idles in a tail (the Stream-K way of balancing a
// split reduction), and the Hkv workgroups of a set read the same token rows
// ([.., Hkv, D] is token-major) side by side. Keys are cut into chunks of
// kv_chunk tokens, the unit of the split: tiles never straddle a chunk and a
// range holds at least one chunk. A range merges the chunks it holds in its
// online softmax (an incremental LSE combine) and writes one partial per
// block of rows it touches, in slot r - r0 of those rows (r the range, r0 the
// range of the rows' first tile); the LSE combine merges the partials.
//
// Forms. MODS selects what the score path does: 0 plain (the softmax scale
// rides in the exponent FMA; sinks, when given, are folded in by the prefill
// epilogue or the combine); 1 the score transform (logit softcap, ALiBi
// slope); 2 the transform plus an additive bf16 mask; 3 and 4 are 0 and 2 on
// head dims below the tile width D (Q columns past Dk load as 0, K/V chunks
// past Dk / Dv are filled from chunk 0 of the same key row, O columns past
// Dv are not stored). KV8 (split kernels at D = 128, 256, 512) reads one-byte OCP e4m3
// K/V tiles and widens each fragment to bf16 just before its MFMA; the K/V
// scales of the workgroup's KV head fold into the exponent factor and the
// partial's normalisation.
#pragma once

#include "fa_device.h"
#include "fa_launch.h"

namespace gqafa {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;            // final output (prefill)
  float* lse;             // final LSE (prefill), may be null
  float* o_part;          // split mode: fp32 [B, Hq, Sq, n_slots, D]
  float* lse_part;        // split mode: fp32 [B, Hq, Sq, n_slots]
  const int32_t* seq_lens;  // split mode: keys per sequence
  const int32_t* table;     // split mode: block table or null
  int page_shift, max_pages, num_pages;
  // element strides; the head dim is unit-stride. K/V: (sequence, token,
  // head) for a dense cache, (page, slot, head) for a paged one. The token
  // strides of K and V are below 2^24 (checked by the caller).
  int64_t q_sb, q_ss, q_sh;
  int64_t o_sb, o_ss, o_sh;   // prefill output
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int B, Sq, Hq, Hkv, G;
  int skv;                // prefill: keys per sequence
  int causal, window;
  float sl2;              // scale * log2(e)
  int n_rb;               // row blocks per (b, g)
  int chunk, n_slots;     // split mode: keys per chunk, partial slots per row (chunks + 1)
  // score modifiers (kernels whose MODS level includes the score transform;
  // the mask needs a level that includes it; sinks are read by every prefill
  // kernel): softcap > 0 maps the
  // scaled score s to softcap * tanh(s / softcap); alibi_k0 / alibi_k1 > 0
  // add slope_h * (key - position) with slope_h = 2^(-alibi_k0 (h + 1)) for
  // h < alibi_n and 2^(-alibi_k1 (2 (h - alibi_n) + 1)) above; sinks
  // (prefill only; the split path's combine adds them) is a per-query-head
  // logit in the softmax denominator, or null; mask (bf16, or null) adds
  // mask[b * mask_sb + i * mask_ss + key] to the score of query row i of
  // sequence b (every head), after the softcap and the slope term.
  float scale;            // the softmax scale (used by MODS kernels)
  float softcap, alibi_k0, alibi_k1;
  int alibi_n;
  const float* sinks;
  const uint16_t* mask;
  int64_t mask_sb, mask_ss;
  // key and value head dims when they are below the tile's D (multiples of
  // 8): Q columns at or past dk load as 0; a K or V tile chunk past dk / dv
  // is filled with a copy of chunk 0 of the same key row (finite data that
  // meets only zero Q columns, or lands in O columns that are never
  // stored); O columns at or past dv are not stored
  // (all of this in the padded kernels, MODS levels 3 and 4, which are used
  // exactly when dk < D or dv < D)
  int dk, dv;
  // fp8 (OCP e4m3) K and V caches (kernels instantiated with KV8): the value
  // of an element of KV head g is e4m3(byte) * k_scale[g] (v_scale[g] for V);
  // device [Hkv]
  const float* k_scale;
  const float* v_scale;
};

// Fill the score-modifier fields of the kernel arguments (host side).
// ALiBi slopes: n = 2^floor(log2 Hq), m0 = 2^(-max_bias / n),
// m1 = 2^(-max_bias / (2 n)); head h < n gets m0^(h + 1), the others
// m1^(2 (h - n) + 1) -- kept as exponents k0 = max_bias / n and k1 = k0 / 2.
inline void set_mods(AttnArgs& a, float scale, float softcap, float max_bias, const float* sinks, int Hq,
                     const void* mask, int64_t mask_sb, int64_t mask_ss) {
  a.mask = static_cast<const uint16_t*>(mask);
  a.mask_sb = mask_sb;
  a.mask_ss = mask_ss;
  a.scale = scale;
  a.softcap = softcap > 0.f ? softcap : 0.f;
  a.alibi_k0 = a.alibi_k1 = 0.f;
  a.alibi_n = 1;
  if (max_bias > 0.f) {
    int n = 1;
    while (n * 2 <= Hq) n *= 2;
    a.alibi_n = n;
    a.alibi_k0 = max_bias / (float)n;
    a.alibi_k1 = max_bias / (2.0f * (float)n);
  }
  a.sinks = sinks;
}

// Spread a 1-D grid over the 8 XCDs so that logical neighbours (row blocks of
// one (b, KV head), which read the same K/V) share an XCD and its L2.
// Workgroup i is dispatched to XCD i % 8; this returns the logical index.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  constexpr int X = 8;
  const int per = n / X, rem = n % X;
  const int x = i % X, k = i / X;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + k;
}

// XOR swizzles (16-byte chunk index within a row). Both stay below the chunk
// count of a row.
//
// K is read as the A operand of S^T: sixteen consecutive lanes read sixteen
// consecutive rows at the same logical chunk, so the XOR takes four bits of
// the row (spreading them over 16 distinct 16-byte bank groups; any 8
// consecutive lanes also land in 8 distinct groups).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D >= 128) return row & 15;
  else return (row >> 1) & 7;          // 128-byte rows: two rows per 256 bytes
}
// V is read by ds_read_b64_tr_b16: a 16-lane group reads 4 consecutive rows x
// 2 consecutive chunks, the two groups of a half-wave the next 2 chunks of
// the same rows. The XOR (bits 1-3) separates the 4 rows both in bits 2-3
// (16 distinct groups across the half-wave) and in bits 1-2 (8 distinct
// groups within one 16-lane group).
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  const int rr = row & 3;
  if constexpr (D >= 128) return (rr << 2) ^ (((rr ^ (rr >> 1)) & 1) << 1);
  else return rr << 1;
}

// The keys any row of one block of rows may attend to, as tiles of BN keys
// laid out chunk by chunk: tile k of chunk c starts at key c * chunk + k * BN
// and never crosses the chunk's end. Chunks c_lo .. c_hi hold visible keys;
// the first holds tiles k0 .. tpc - 1 (tpc tiles per chunk), the last tiles
// 0 .. k1 (k0 .. k1 when they are the same chunk).
struct RowSpan {
  int c_lo, k0, c_hi, k1;
  int nt;                    // tiles in all (0: no visible key)
};
template <int BN, int BM>
__device__ __forceinline__ RowSpan row_span(const AttnArgs& a, int len, int rb, int tpc) {
  RowSpan s{0, 0, 0, 0, 0};
  const int rows = a.Sq * a.G;
  const int r_lo = rb * BM, r_hi = min(r_lo + BM, rows);
  const int shift = len - a.Sq;               // bottom-right causal alignment
  int lo = 0, hi = len;
  if (a.causal) {
    hi = min(hi, (r_hi - 1) / a.G + shift + 1);
    if (a.window > 0) lo = max(lo, r_lo / a.G + shift - a.window + 1);
  }
  if (hi <= lo) return s;
  s.c_lo = lo / a.chunk;
  s.c_hi = (hi - 1) / a.chunk;
  s.k0 = (lo - s.c_lo * a.chunk) / BN;
  s.k1 = (hi - 1 - s.c_hi * a.chunk) / BN;
  s.nt = s.c_lo == s.c_hi ? s.k1 - s.k0 + 1 : (tpc - s.k0) + (s.c_hi - s.c_lo - 1) * tpc + s.k1 + 1;
  return s;
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) x += __shfl_xor(x, s, 64);
  return x;
}
__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int y = __shfl_up(x, s, 64);
    if (lane >= s) x += y;
  }
  return x;
}

template <int D, int NW, int BN, int DS, int NBUF, bool PAGED, bool SPLIT, int WPE, int MODS, bool KV8 = false,
          bool KX = false>
__global__ void __launch_bounds__(NW * 64, WPE) attn_kernel(const AttnArgs a) {
  static_assert(D % 64 == 0 && BN % 32 == 0, "tile shape");
  static_assert((DS == 1 || DS == 2 || DS == 4) && NW % DS == 0, "a D split groups 2 or 4 waves");
  constexpr int BM = NW * 32 / DS;
  // Prefill with eight full-D waves runs them as two groups in ping-pong
  // (the main loop below); head dim 128 without score modifiers.
  constexpr bool PP = !SPLIT && DS == 1 && NW == 8;
  static_assert(!PP || (NBUF == 3 && BN == 64 && !KV8 && !KX && (MODS == 0 || MODS == 1)), "ping-pong prefill");
  // Prefill at head dim 256 holds one workgroup per CU, so nothing covers a
  // block of rows' start (its Q from HBM, the first tiles) and end (O out):
  // measured on MI355X ~12 us per block against ~0.9 us per 32-key tile.
  // This kernel runs a persistent grid instead: each workgroup takes several
  // blocks of rows in turn and loads the next block's Q fragments and first
  // tiles before writing the current block's O. (At head dim 512 the same
  // loop, with its copy lambdas forced inline so that it does not spill,
  // measured 1 % slower: 2048 causal blocks of one wave per SIMD balance
  // better under the hardware's own dispatch.)
  constexpr bool PERS = !SPLIT && !PP && D == 256 && !KX;
  // MODS level: 0 plain, 1 score transform (softcap, ALiBi), 2 transform +
  // mask, 3 plain with head dims below D, 4 transform + mask + head dims
  // below D
  static_assert(MODS >= 0 && MODS <= 4, "modifier level");
  constexpr bool kXform = MODS == 1 || MODS == 2 || MODS == 4;
  constexpr bool kMask = MODS == 2 || MODS == 4;
  constexpr bool kPad = MODS >= 3;
  // fp8 K/V (one byte per element) only in the one-wave-per-32-rows split
  // kernels at D = 128 (8 chunks of 16 bytes per key row)
  // fp8 K/V (one byte per element): split kernels at head dims 128, 256 and
  // 512 (register-staged one wave per 32 rows at 128, a D split above)
  static_assert(!KV8 || (SPLIT && D >= 128 && !kPad && (D == 128) == (DS == 1)), "fp8 K/V: split kernels");
  constexpr int ES = KV8 ? 1 : 2;             // bytes per K/V element
  constexpr int KCH = D * ES / 16;            // 16-byte chunks per row
  constexpr int NSEG = BN * KCH / 64;         // 1 KiB segments per tile
  static_assert(NSEG % NW == 0, "every wave loads whole segments");
  constexpr int SEGW = NSEG / NW;             // segments per wave per operand
  constexpr int NKB = BN / 32;                // 32-key score blocks per tile
  constexpr int NKS = BN / 16;                // 16-key steps of the PV product
  constexpr int NDB = D / 32 / DS;            // 32-wide d blocks of O per wave
  constexpr int NQC = D / 16 / DS;            // 16-wide d steps of Q K^T per wave
  static_assert(NBUF >= 2 && NBUF <= 4, "ring of 2 to 4 tile buffers per operand");
  // Split mode: a window of block-table entries staged in LDS (none at
  // D = 512, where the tile ring and the score exchange fill LDS). The
  // contiguous-cache kernel reserves the same space, so both kernels hold
  // the same number of workgroups per CU and split the work identically.
  constexpr int TAB = (SPLIT && D < 512) ? 512 : 0;
  // KX: a key head dim of D + 64 (576 at D = 512; the value head dim is D).
  // The 64 extra key columns have a small tile of their own (32 rows x 64,
  // one 1 KiB copy segment per wave), and each wave of a D split takes 64 / DS
  // of them as NQX more 16-wide steps of the score contraction. The score
  // exchange then has one slot (LDS: 128 KiB of tiles + 8 KiB of extra key
  // columns + 16 KiB of exchange).
  static_assert(!KX || (D == 512 && !KV8 && !kPad && (MODS == 0 || MODS == 2) && NW == 4 && NBUF == 2 && BN == 32),
                "576-wide keys: the head-dim-512 kernels");
  constexpr int DXK = KX ? 64 : 0;
  constexpr int NQX = KX ? 4 / DS : 1;
  constexpr int XSLOTS = KX ? 1 : 2;

  // A ring of NBUF tile buffers per operand, each its own object: the copies
  // into one never alias reads of another, so no read waits on a copy it does
  // not need.
  constexpr int TU = BN * D * ES / 2;          // 16-bit slots of one tile buffer
  constexpr int B2 = NBUF > 2 ? TU : 8, B3 = NBUF > 3 ? TU : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[TU];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[TU];
  __shared__ __attribute__((aligned(1024))) uint16_t sK2[B2];
  __shared__ __attribute__((aligned(1024))) uint16_t sK3[B3];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[TU];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[TU];
  __shared__ __attribute__((aligned(1024))) uint16_t sV2[B2];
  __shared__ __attribute__((aligned(1024))) uint16_t sV3[B3];
  int* sT = nullptr;
  if constexpr (TAB > 0) {
    __shared__ int sT_buf[TAB > 0 ? TAB : 1];
    sT = sT_buf;
    asm volatile("" ::"v"(sT_buf));           // keeps the reservation in the dense kernel
  }
  // partial scores exchanged by the waves of a D split, [slot][wave][value][lane]
  __shared__ float sX[DS > 1 ? XSLOTS : 1][DS > 1 ? NW : 1][DS > 1 ? NKB * 16 : 1][64];
  // O staging of the persistent prefill at head dims up to 256 (the tile
  // buffers then already hold the next block's first tiles)
  __shared__ __attribute__((aligned(1024))) uint16_t sO[(PERS && D <= 256) ? BM * D : 8];
  // extra key columns (KX), one buffer per K tile buffer
  __shared__ __attribute__((aligned(1024))) uint16_t sKx0[KX ? BN * DXK : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sKx1[KX ? BN * DXK : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps LDS bases scalar
  const int j = lane & 31;     // this lane's query row inside the wave
  const int hl = lane >> 5;    // lane half
  const int rg = wave / DS;    // row group (32 rows) of this wave
  const int dh = wave % DS;    // which half of the head dim this wave holds

  // ---- staging geometry: global -> LDS ---------------------------------------
  // Segment s (1 KiB) of a tile holds chunk positions 64 s .. 64 s + 63 of
  // the row-major tile: lane L writes position 64 s + L = row * KCH + pc,
  // holding logical chunk pc ^ swizzle(row) of that key row.
  const int k_rs = (int)a.k_ss, v_rs = (int)a.v_ss;   // token strides (elements)
  // Per-lane segment geometry. With few segments per wave it is kept in
  // registers; with many (large head dims, few waves) it is recomputed at
  // each copy, which costs a few integer operations instead of 3 registers
  // per segment.
  constexpr bool KEEP_SEG = SEGW <= 8;
  constexpr int NKEEP = KEEP_SEG ? SEGW : 1;
  auto seg_row = [&](int i) -> int { return ((wave * SEGW + i) * 64 + lane) / KCH; };
  // fp8 tiles: rows of 8 chunks, the chunk XORed with the row's low 3 bits
  auto swzk = [](int row) -> int { return KV8 ? (row & 7) : swz_k<D>(row); };
  auto swzv = [](int row) -> int { return KV8 ? (row & 7) : swz_v<D>(row); };
  auto seg_koff = [&](int i) -> uint32_t {
    const int pos = (wave * SEGW + i) * 64 + lane, row = pos / KCH, pc = pos % KCH;
    return (uint32_t)(ES * row * k_rs + 16 * (pc ^ swzk(row)));
  };
  auto seg_voff = [&](int i) -> uint32_t {
    const int pos = (wave * SEGW + i) * 64 + lane, row = pos / KCH, pc = pos % KCH;
    return (uint32_t)(ES * row * v_rs + 16 * (pc ^ swzv(row)));
  };
  int srow[NKEEP];         // key row (inside the tile) of each of this lane's segments
  uint32_t koff[NKEEP];    // byte offset of its K chunk inside an unclamped tile
  uint32_t voff[NKEEP];
  if constexpr (KEEP_SEG) {
#pragma unroll
    for (int i = 0; i < SEGW; ++i) {
      srow[i] = seg_row(i);
      koff[i] = seg_koff(i);
      voff[i] = seg_voff(i);
    }
  }
  // Prefill copy geometry: a 1 KiB segment covers RPS = 64 / KCH key rows;
  // lane L fetches row p_lr = L / KCH of its segment into physical chunk
  // L % KCH, i.e. logical chunk (L % KCH) ^ swizzle(row). Since RPS is a
  // power of two and p_lr < RPS, both swizzles of row sg RPS + p_lr split
  // into a per-lane part and a per-segment (uniform) part.
  constexpr int RPS = 64 / KCH;
  const int p_lr = lane / KCH, p_pc = lane % KCH;
  const uint32_t p_lrk = (uint32_t)(p_lr * ES * k_rs);
  const uint32_t p_lrv = (uint32_t)(p_lr * ES * v_rs);
  // K: swz_k(sg RPS + lr) = swz_k-bits of (sg RPS) ^ those of lr (disjoint)
  const int p_kx = D >= 128 ? (p_pc ^ p_lr) : (p_pc ^ (p_lr >> 1));
  auto p_kchunk = [&](int sg) -> int {
    const int c = D >= 128 ? ((sg * RPS) & 15) : ((sg * 4) & 7);
    return p_kx ^ c;
  };
  // V: swz_v depends on row & 3 only
  const int p_vx0 = p_pc ^ swz_v<D>(p_lr & 3);
  const int p_vx1 = p_pc ^ swz_v<D>((2 + p_lr) & 3);
  auto p_vchunk = [&](int sg) -> int {
    if constexpr (RPS == 1) return lane ^ swz_v<D>(sg & 3);
    else if constexpr (RPS == 2) return (sg & 1) ? p_vx1 : p_vx0;
    else return p_vx0;
  };

  // Head dims below D: the byte distance from this lane's chunk of segment i
  // back to chunk 0 of its key row when the chunk lies past the real K or V
  // head dim, else 0 (recomputed at each copy of a padded call: a few integer
  // operations). Every copy keeps its instruction count, which the copy
  // waits count on. Only the padded kernels use it.
  auto seg_pad = [&](int i, bool is_v) -> uint32_t {
    const int pos = (wave * SEGW + i) * 64 + lane, row = pos / KCH, pc = pos % KCH;
    const int lc = pc ^ (is_v ? swz_v<D>(row) : swz_k<D>(row));
    return 8 * lc >= (is_v ? a.dv : a.dk) ? 16u * (uint32_t)lc : 0u;
  };

  // Paged split: a window of one sequence's block-table row, clamped into
  // [0, num_pages), staged in LDS so that no tile copy waits on a table
  // load. A tile outside the window restages it (all waves together).
  int tw_b = -1, tw_p0 = 0;
  auto stage_table = [&](int b_t, int pf) {
    lds_barrier();                          // every wave is done with the old window
    const int np = min(TAB, a.max_pages - pf);
    for (int i = tid; i < np; i += NW * 64) sT[i] = clamp_page(a.table[(int64_t)b_t * a.max_pages + pf + i], a.num_pages);
    lds_barrier();
    tw_b = b_t;
    tw_p0 = pf;
  };

  // Prefill (dense K/V) copy of segment sg of one operand of the tile of
  // keys [tb, tb + BN) into dst, buffer form: segment sg holds rows sg RPS ..
  // sg RPS + RPS - 1 of the tile; this lane fetches logical chunk lc of row
  // sg RPS + p_lr. The row part of the source offset is uniform (soffset);
  // the lane part is one per-lane constant plus the chunk. Rows at or past
  // ke_t, the sequence's end, read its last key's row (their
  // scores are masked, their V rows get weight 0), and for head dims below
  // D a chunk past the real one reads chunk 0 of its row; both are written
  // without branches (whole tiles subtract 0), so copies placed between
  // MFMAs stay in the MFMA block's one basic block.
  auto prefill_seg = [&](int tb, int ke_t, const uint16_t* kv_base, bool is_v, uint16_t* dst, int sg)
      __attribute__((always_inline)) {
    const int lim = ke_t - 1 - tb;
    const int rs = is_v ? v_rs : k_rs;
    const int rsb = ES * rs;                          // bytes per key row
    const char* tbase = reinterpret_cast<const char*>(kv_base) + (int64_t)ES * tb * rs;
    const int lc = is_v ? p_vchunk(sg) : p_kchunk(sg);
    const int over = max(sg * RPS + p_lr - lim, 0);
    uint32_t o = (is_v ? p_lrv : p_lrk) + 16u * (uint32_t)lc - (uint32_t)(over * rsb);
    if constexpr (kPad) o -= 8 * lc >= (is_v ? a.dv : a.dk) ? 16u * (uint32_t)lc : 0u;
    dma16_buf_s<false>(tbase, o, (uint32_t)(sg * RPS * rsb), dst + sg * 512);
  };

  // Copy one operand of the tile of keys [tb, tb + BN) of a sequence whose
  // keys end at ke_t (exclusive) into dst. kv_base is the K or V cache at
  // this KV head (and, for a contiguous cache, at this sequence). Keys past
  // ke_t are clamped onto its last key: their scores are masked and their V
  // rows get weight exactly 0, so the data read there never matters (and is
  // always finite in-range data). A block-table entry outside [0, num_pages)
  // is clamped into range: every load stays inside the cache.
  auto issue = [&](int tb, int ke_t, const uint16_t* kv_base, int b_t, bool is_v, uint16_t* dst) {
    const int lim = ke_t - 1 - tb;            // last valid row of this tile
    const bool tail = lim < BN - 1;           // uniform
    const int rs = is_v ? v_rs : k_rs;
    if constexpr (KX) {
      if (!is_v) {
        // the 64 extra key columns of the tile: wave w copies rows 8 w ..
        // 8 w + 7 (8 chunks of 16 bytes each), logical chunk (lane & 7) ^
        // (row & 7) into physical chunk lane & 7 of its row
        uint16_t* dx = (dst == sK0 ? sKx0 : sKx1) + wave * 512;
        const int rowx = 8 * wave + (lane >> 3);
        const int lcx = (lane & 7) ^ (rowx & 7);
        const int rx = min(rowx, lim);            // rows past the last valid one read that row
        if constexpr (!SPLIT) {
          const char* tbx = reinterpret_cast<const char*>(kv_base) + (int64_t)ES * tb * rs;
          dma16_buf_s<false>(tbx, (uint32_t)(rx * ES * rs + ES * D + 16 * lcx), 0u, dx);
        } else if constexpr (PAGED) {
          const int t = tb + rx;
          const int page = clamp_page(a.table[(int64_t)b_t * a.max_pages + (t >> a.page_shift)], a.num_pages);
          const char* src = reinterpret_cast<const char*>(kv_base) +
                            ES * (paged_row(page, t & ((1 << a.page_shift) - 1), a.k_sb, rs) + D) + 16 * lcx;
          dma16<SPLIT>(reinterpret_cast<const uint16_t*>(src), dx);
        } else {
          const char* src = reinterpret_cast<const char*>(kv_base) + ES * ((int64_t)(tb + rx) * rs + D) + 16 * lcx;
          dma16<SPLIT>(reinterpret_cast<const uint16_t*>(src), dx);
        }
      }
    }
    if constexpr (!SPLIT) {
      // one segment as prefill_seg above, with the tile's row base, row
      // pitch and lane offset computed once for all segments
      const int rsb = ES * rs;                          // bytes per key row
      const char* tbase = reinterpret_cast<const char*>(kv_base) + (int64_t)ES * tb * rs;
      const uint32_t lro = is_v ? p_lrv : p_lrk;        // p_lr * rsb
      auto seg_copy = [&](int i, bool clamp_rows) {
        const int sg = wave * SEGW + i;                 // uniform
        const int lc = is_v ? p_vchunk(sg) : p_kchunk(sg);
        uint32_t o = lro + 16u * (uint32_t)lc;
        if (clamp_rows) {
          const int r = sg * RPS + p_lr;
          if (r > lim) o -= (uint32_t)((r - lim) * rsb);
        }
        if constexpr (kPad) {
          if (8 * lc >= (is_v ? a.dv : a.dk)) o -= 16u * (uint32_t)lc;
        }
        dma16_buf_s<false>(tbase, o, (uint32_t)(sg * RPS * rsb), dst + sg * 512);
      };
      // At head dim 512 whole tiles (all but a sequence's last) take a
      // straight-line path (the per-copy tail test became a branch per copy
      // there); elsewhere one loop keeps the register budget.
      if (D < 512 || tail) {
#pragma unroll
        for (int i = 0; i < SEGW; ++i) seg_copy(i, tail);
      } else {
#pragma unroll
        for (int i = 0; i < SEGW; ++i) seg_copy(i, false);
      }
      return;
    }
    if constexpr (PAGED && TAB > 0) {
      const int pf = tb >> a.page_shift, pl = (tb + min(lim, BN - 1)) >> a.page_shift;
      if (b_t != tw_b || pf < tw_p0 || pl >= tw_p0 + TAB) stage_table(b_t, pf);
    }
    if constexpr (PAGED && TAB > 0 && BN == 32 && !kPad) {
      // A whole tile starting on a 16-token boundary with pages of 16 tokens
      // or more: rows 0-15 lie in one page and rows 16-31 in one page (the
      // same one for larger pages), so both row bases are wave-uniform
      // (scalar arithmetic) and a lane only picks one and adds its 32-bit
      // offset inside the tile.
      if (!tail && a.page_shift >= 4 && (tb & 15) == 0) {
        const int mask = (1 << a.page_shift) - 1;
        const int p0 = __builtin_amdgcn_readfirstlane(sT[(tb >> a.page_shift) - tw_p0]);
        const int p1 = __builtin_amdgcn_readfirstlane(sT[((tb + 16) >> a.page_shift) - tw_p0]);
        const int64_t sb = is_v ? a.v_sb : a.k_sb;
        const char* base0 = reinterpret_cast<const char*>(kv_base) + ES * paged_row(p0, tb & mask, sb, rs);
        const char* base1 = reinterpret_cast<const char*>(kv_base) +
                            ES * (paged_row(p1, (tb + 16) & mask, sb, rs) - 16 * (int64_t)rs);
#pragma unroll
        for (int i = 0; i < SEGW; ++i) {
          const int row = KEEP_SEG ? srow[i] : seg_row(i);
          const uint32_t off0 = KEEP_SEG ? (is_v ? voff[i] : koff[i]) : (is_v ? seg_voff(i) : seg_koff(i));
          const char* src = (row >= 16 ? base1 : base0) + off0;
          dma16<SPLIT>(reinterpret_cast<const uint16_t*>(src), dst + (wave * SEGW + i) * 512);
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < SEGW; ++i) {
      const int row = KEEP_SEG ? srow[i] : seg_row(i);
      const uint32_t off0 = KEEP_SEG ? (is_v ? voff[i] : koff[i]) : (is_v ? seg_voff(i) : seg_koff(i));
      const char* src;
      if constexpr (PAGED) {
        const int t = tb + min(row, lim);
        int page;
        if constexpr (TAB > 0) {
          page = sT[(t >> a.page_shift) - tw_p0];     // clamped when staged
        } else {
          page = clamp_page(a.table[(int64_t)b_t * a.max_pages + (t >> a.page_shift)], a.num_pages);
        }
        // the lane's offset inside the tile (off0) already holds row * rs,
        // so the slot passed here is the token's slot minus the row
        const int64_t base = paged_row(page, (t & ((1 << a.page_shift) - 1)) - row, is_v ? a.v_sb : a.k_sb, rs);
        src = reinterpret_cast<const char*>(kv_base) + ES * base + off0;
      } else {
        // uniform tile base + 32-bit per-lane byte offset
        uint32_t o = off0;
        if (tail && row > lim) o -= (uint32_t)(ES * (row - lim) * rs);
        if constexpr (!SPLIT) {
          // prefill: the buffer form, which keeps its operand reads in flight
          // (measured slower for the split kernels' streams)
          if constexpr (kPad) o -= seg_pad(i, is_v);
          dma16_buf<SPLIT>(reinterpret_cast<const char*>(kv_base) + ES * ((int64_t)tb * rs), o,
                           dst + (wave * SEGW + i) * 512);
          continue;
        }
        src = reinterpret_cast<const char*>(kv_base) + ES * ((int64_t)tb * rs) + o;
      }
      if constexpr (kPad) src -= seg_pad(i, is_v);
      dma16<SPLIT>(reinterpret_cast<const uint16_t*>(src), dst + (wave * SEGW + i) * 512);
    }
  };
  // K and V cache bases of (sequence b, KV head g)
  auto kv_bases = [&](int b_t, int g_t, const uint16_t*& kb_out, const uint16_t*& vb_out) {
    int64_t koff = (int64_t)g_t * a.k_sh, voff = (int64_t)g_t * a.v_sh;
    if constexpr (!PAGED) {
      koff += (int64_t)b_t * a.k_sb;
      voff += (int64_t)b_t * a.v_sb;
    }
    kb_out = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.k) + ES * koff);
    vb_out = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.v) + ES * voff);
  };

  // ---- the rows being worked on: one block of rows of one (b, KV head) ------
  // In split mode they change as the workgroup moves through its tiles.
  int b = 0;
  int p = 0, wpmin = 0, wpmax = 0, qi = 0, qh = 0;
  bool row_ok = false;
  float slope = 0.f;           // ALiBi slope of this lane's query head (MODS)
  const uint16_t* mrow = nullptr;  // this lane's mask row (MODS with a mask)
  int mlen = 0;                // keys of the sequence (the mask is read below it)
  int ke = 0;                  // end (exclusive) of the keys the current tile may hold
  bf16x8 qf[NQC];
  bf16x8 qfx[NQX];     // KX: this wave's share of the 64 extra query columns
  // This lane's Q fragments of row block rb_ of (sequence b_, KV head g_),
  // as set_rows loads them (the persistent prefill's prefetch of the next
  // block)
  auto load_q = [&](int b_, int g_, int rb_) {
    const int rows = a.Sq * a.G;
    const int r_lo = rb_ * BM;
    const int r_hi = min(r_lo + BM, rows);
    const int r = r_lo + 32 * rg + j;
    const bool ok = r < r_hi;
    const int qi_ = ok ? r / a.G : 0;
    const int qh_ = g_ * a.G + (ok ? r % a.G : 0);
    const int64_t qoff = (int64_t)b_ * a.q_sb + (int64_t)qi_ * a.q_ss + (int64_t)qh_ * a.q_sh +
                         8 * hl + dh * (D / DS);
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      const bool in_d = !kPad || 8 * hl + dh * (D / DS) + 16 * c < a.dk;
      if (ok && in_d) w = *reinterpret_cast<const u32x4*>(a.q + qoff + 16 * c);
      qf[c] = as_bf16x8(w);
    }
  };
  auto set_rows = [&](int b_, int g_, int rb_, int n_keys, bool with_q = true) {
    b = b_;
    const int rows = a.Sq * a.G;
    const int r_lo = rb_ * BM;
    const int r_hi = min(r_lo + BM, rows);
    const int shift = n_keys - a.Sq;           // bottom-right causal alignment
    const int wr_lo = r_lo + 32 * rg;
    const int wr_hi = min(wr_lo + 32, r_hi);
    wpmin = wr_lo / a.G + shift;
    wpmax = (wr_hi - 1) / a.G + shift;
    const int r = wr_lo + j;
    row_ok = r < r_hi;
    qi = row_ok ? r / a.G : 0;
    qh = g_ * a.G + (row_ok ? r % a.G : 0);
    p = qi + shift;                            // absolute position of this lane's row
    if constexpr (kXform) {
      slope = 0.f;
      if (a.alibi_k0 > 0.f)
        slope = fast_exp2(qh < a.alibi_n ? -a.alibi_k0 * (float)(qh + 1)
                                         : -a.alibi_k1 * (float)(2 * (qh - a.alibi_n) + 1));
    }
    if constexpr (kMask) {
      if (a.mask != nullptr) mrow = a.mask + (int64_t)b_ * a.mask_sb + (int64_t)qi * a.mask_ss;
      mlen = n_keys;
    }
    const int64_t qoff = (int64_t)b_ * a.q_sb + (int64_t)qi * a.q_ss + (int64_t)qh * a.q_sh +
                         8 * hl + dh * (D / DS);
    if (with_q) {
#pragma unroll
      for (int c = 0; c < NQC; ++c) {
        u32x4 w = {0u, 0u, 0u, 0u};
        const bool in_d = !kPad || 8 * hl + dh * (D / DS) + 16 * c < a.dk;
        if (row_ok && in_d) w = *reinterpret_cast<const u32x4*>(a.q + qoff + 16 * c);
        qf[c] = as_bf16x8(w);
      }
    }
    if constexpr (KX) {
      // columns D + 16 (dh NQX + c) + 8 hl .. + 7
      const int64_t qx = qoff - dh * (D / DS) + D + 16 * dh * NQX;
#pragma unroll
      for (int c = 0; c < NQX; ++c) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (row_ok) w = *reinterpret_cast<const u32x4*>(a.q + qx + 16 * c);
        qfx[c] = as_bf16x8(w);
      }
    }
  };

  // ---- LDS read addresses --------------------------------------------------
  // K (A operand of S^T): row 32 kb + j, logical chunk 2 (c + dh NQC) + hl.
  // V^T (A operand of O^T): the 16-lane group m = lane % 16 supplies rows
  // key_base + m / 4 at d = d_base + 4 (m % 4); lane i of the group receives
  // (V[key_base + e][d_base + i], e = 0..3).
  const int m16 = lane & 15;
  const int g1 = (lane >> 4) & 1;
  // Element offset of this lane's V^T read inside a tile buffer, per 32-wide
  // d block; the read of 16-key step ks and half h adds (16 ks + 8 h) D (the
  // V swizzle depends on row & 3, the same for every ks and h). The offsets
  // are opaque to the optimiser, so every read address stays one constant
  // away from its buffer and the compiler can tell which buffer a read
  // touches: otherwise it loses track on long address chains and makes the
  // read wait for every tile copy in flight, whatever buffer they fill.
  // The kernels for head dims below D, short of registers, compute each
  // address in full instead.
  int vlo[kPad ? 1 : NDB];
  if constexpr (!kPad) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * (db + dh * NDB) + 16 * g1 + 4 * (m16 & 3);
      const int r0 = 4 * hl + (m16 >> 2);
      vlo[db] = r0 * D + 8 * ((d >> 3) ^ swz_v<D>(r0)) + (d & 7);
    }
  }
  auto v_elem = [&](int ks, int half, int db) -> int {
    if constexpr (kPad) {
      const int d = 32 * (db + dh * NDB) + 16 * g1 + 4 * (m16 & 3);
      const int row = 16 * ks + 8 * half + 4 * hl + (m16 >> 2);
      return row * D + 8 * ((d >> 3) ^ swz_v<D>(row)) + (d & 7);
    } else {
      return (16 * ks + 8 * half) * D + vlo[db];
    }
  };

  // ---- running state -----------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;   // reference max of the row (raw score units)
  float nb_ref = 0.f;        // its exponent offset -m_run * sl2 (0 while m_run is -inf)
  float l_run = 0.f;         // this lane's part of the row sum
  // exponent factor: scores are raw q.k (scale folded in here), or with
  // score modifiers already scaled and modified (natural units)
  // (fp8 K: times the KV head's K scale, set once the head is known)
  float sl2 = kXform ? kLog2e : a.sl2;
  float thr = kRescaleLog2 / sl2;
  float xscale = a.scale;    // the score scale of the score transform
  float vsc = 1.f;           // fp8 V: the KV head's V scale

  // KX: this wave's NQX steps of the contraction over the extra key columns
  // of the tile whose main part is in bk (row j, logical chunk 2 (dh NQX +
  // c) + hl, stored at physical chunk lc ^ (row & 7))
  auto score_extra = [&](const uint16_t* bk, f32x16& acc) {
    if constexpr (KX) {
      const uint16_t* bx = bk == sK0 ? sKx0 : sKx1;
#pragma unroll
      for (int c = 0; c < NQX; ++c) {
        const int lc = 2 * (dh * NQX + c) + hl;
        const u32x4 kw = *reinterpret_cast<const u32x4*>(&bx[j * DXK + 8 * (lc ^ (j & 7))]);
        acc = mfma32(as_bf16x8(kw), qfx[c], acc);
      }
    }
  };

  // S^T (this wave's part of the contraction) for the tile in bk
  auto scores = [&](const uint16_t* bk, f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {          // alternate accumulators
        const int row = 32 * kb + j;
        if constexpr (KV8) {
          // fp8 tile: this lane's 8 bytes (d = 16 c' + 8 hl ..) of its key
          // row in 16-byte chunk c' = c + dh NQC, widened to bf16
          const unsigned char* b8 = reinterpret_cast<const unsigned char*>(bk);
          const u32x2 kw =
              *reinterpret_cast<const u32x2*>(b8 + row * D + 16 * ((c + dh * NQC) ^ swzk(row)) + 8 * hl);
          s[kb] = mfma32(as_bf16x8(fp8x8_to_bf16x8(kw)), qf[c], s[kb]);
        } else {
          const int ch = 2 * (c + dh * NQC) + hl;
          const u32x4 kw = *reinterpret_cast<const u32x4*>(&bk[row * D + 8 * (ch ^ swz_k<D>(row))]);
          s[kb] = mfma32(as_bf16x8(kw), qf[c], s[kb]);
        }
      }
    }
    if constexpr (KX) score_extra(bk, s[0]);
  };

  // S^T as scores, with the first NPRE operand fragments already in kpre
  // (read before the softmax bookkeeping that precedes the MFMA block, so
  // their LDS latency is hidden behind it). Reads then run NPRE ahead of
  // their MFMAs: at head dim 256 four measured 1-2 % faster than six and
  // 3 % faster than eight (two and three: 8 % slower).
  constexpr int NPRE = 4 < NQC * NKB ? 4 : NQC * NKB;
  auto k_frag = [&](const uint16_t* bk, int idx) -> u32x4 {
    const int c = idx / NKB, kb = idx % NKB;
    const int row = 32 * kb + j;
    const int ch = 2 * (c + dh * NQC) + hl;
    return *reinterpret_cast<const u32x4*>(&bk[row * D + 8 * (ch ^ swz_k<D>(row))]);
  };
  auto scores_pre = [&](const uint16_t* bk, f32x16 (&s)[NKB], const u32x4 (&kpre)[NPRE]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int idx = c * NKB + kb;
        const u32x4 kw = idx < NPRE ? kpre[idx < NPRE ? idx : 0] : k_frag(bk, idx);
        s[kb] = mfma32(as_bf16x8(kw), qf[c], s[kb]);
      }
    }
  };

  // Mask values of the tile starting at key tb (MODS with a mask): for each
  // 8-key group r of block kb, the 4 bf16 at keys tb + 32 kb + 8 r + 4 hl ..
  // + 3 of this lane's row (the keys its score registers hold). Issued at the
  // start of a step, ahead of the step's tile copies, so waiting for them
  // leaves the copies in flight. Keys at or past the sequence's end read 0.
  u32x2 mv[NKB][4];
  auto load_mask = [&](int tb) {
    if constexpr (kMask) {
      if (a.mask != nullptr) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = tb + 32 * kb + 8 * r + 4 * hl;
            if (key + 4 <= mlen) {
              mv[kb][r] = *reinterpret_cast<const u32x2*>(mrow + key);
            } else {
              uint32_t w[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = key + e < mlen ? (uint32_t)mrow[key + e] : 0u;
              mv[kb][r] = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
            }
          }
      }
    }
  };

  // Mask the boundary tiles, update the reference max (lazily), and return
  // the exponent offset -m*c for the tile starting at key tb.
  auto mask_scores = [&](f32x16 (&s)[NKB], int tb) {
    if constexpr (kXform) {
      // s -> softcap(scale * s) + slope * (key - p) + mask, before the
      // causal / window / length mask
      const float inv_cap = a.softcap > 0.f ? 1.0f / a.softcap : 0.f;
      const float pb = (float)(tb + 4 * hl - p);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          float v = s[kb][x] * xscale;
          if (a.softcap > 0.f) {
            // tanh y = 1 - 2 / (1 + e^(2y)), finite for every y
            const float e2 = fast_exp2(2.0f * kLog2e * v * inv_cap);
            v = a.softcap * (1.0f - 2.0f * fast_rcp(1.0f + e2));
          }
          const int rel = 32 * kb + 8 * (x >> 2) + (x & 3);
          v = fmaf(slope, pb + (float)rel, v);
          if (kMask && a.mask != nullptr) {
            const uint32_t w = mv[kb][x >> 2][(x & 3) >> 1];
            v += __uint_as_float((x & 1) ? (w & 0xffff0000u) : (w << 16));
          }
          s[kb][x] = v;
        }
    }
    const bool full = (tb + BN <= ke) && (!a.causal || tb + BN - 1 <= wpmin) &&
                      (!a.causal || a.window <= 0 || wpmax - tb < a.window);
    if (!full) {
      // visible iff lo_lim <= key - tb - 4*hl <= hi_lim; the left side is a
      // per-element constant
      const int base = tb + 4 * hl;
      const int hi_lim = min(ke - 1, a.causal ? p : INT_MAX) - base;
      const int lo_lim = (a.causal && a.window > 0) ? p - a.window + 1 - base : INT_MIN;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int rel = 32 * kb + 8 * (x >> 2) + (x & 3);
          s[kb][x] = (rel <= hi_lim && rel >= lo_lim) ? s[kb][x] : -INFINITY;
        }
    }
  };
  auto update_ref = [&](const f32x16 (&s)[NKB]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[kb][x]);
    mx = pair_max(mx);
    // Lazy rescale: the running reference max only moves when a row's max
    // grows by more than kRescaleLog2 in the exponent. exp(s - m_ref) then
    // stays below 2^kRescaleLog2, the final O / l and LSE are unchanged,
    // and most tiles skip the O rescale entirely (wave-uniform branch).
    const bool grow = mx > m_run + thr;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2((m_run - m_new) * sl2) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = m_new;
      nb_ref = m_run == -INFINITY ? 0.f : -m_run * sl2;
    }
    return nb_ref;
  };
  auto prepare = [&](f32x16 (&s)[NKB], int tb) -> float {
    mask_scores(s, tb);
    return update_ref(s);
  };

  // P = exp2(s*c - m*c) as bf16 pairs: already the B operand of O^T += V^T P^T.
  // The row sum adds the fp32 values: with few visible keys, summing the
  // bf16-rounded P would put bf16's 2^-9 relative error straight into LSE.
  auto exp_sum = [&](const f32x16 (&s)[NKB], float nb, u32x4 (&pf)[NKS]) -> float {
    float ls;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kb = ks >> 1, base = 8 * (ks & 1);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float e0 = fast_exp2(fmaf(s[kb][base + 2 * w], sl2, nb));
        const float e1 = fast_exp2(fmaf(s[kb][base + 2 * w + 1], sl2, nb));
        ls = (ks == 0 && w == 0) ? e0 + e1 : ls + (e0 + e1);
        pf[ks][w] = pack_bf16(e0, e1);
      }
    }
    return ls;
  };
  auto exponentiate = [&](const f32x16 (&s)[NKB], float nb, u32x4 (&pf)[NKS]) { l_run += exp_sum(s, nb, pf); };

  // The softmax of one tile without the row max in the common case: once
  // every row of the wave has a reference max, the tile is exponentiated
  // against it first. Every weight is at most this lane's part of the row
  // sum, so a part of at most 2^kRescaleLog2 (not NaN) means no weight
  // exceeds the bound the lazy rescale keeps, and the tile needs neither the
  // max nor a rescale. Otherwise (any lane of the wave; rare once the first
  // tiles are done) the row max is taken, the reference updated as in
  // prepare, and the tile exponentiated again. Saves the max reduction's
  // VALU work (~20 of ~130 instructions per 64-key tile and lane) on most
  // tiles; used by the ping-pong prefill, whose softmax slot is VALU work
  // only (in the other kernels the extra live scores cost more registers
  // than the saved instructions gain).
  auto softmax_tile = [&](f32x16 (&s)[NKB], int tb, u32x4 (&pf)[NKS]) {
    mask_scores(s, tb);
    bool slow = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    float ls = 0.f;
    if (!slow) {
      ls = exp_sum(s, nb_ref, pf);
      slow = __builtin_amdgcn_ballot_w64(!(ls <= kRescaleSum)) != 0;
    }
    if (slow) ls = exp_sum(s, update_ref(s), pf);
    l_run += ls;
  };

  // O^T += V^T P^T for the tile in bv
  auto accumulate = [&](const uint16_t* bv, const u32x4 (&pf)[NKS]) {
    if constexpr (KV8) {
      // fp8 tile: V^T from ds_read_b64_tr_b8 (lane layout as read_v8 below,
      // the d block offset by this wave's part of the head dim), widened to
      // bf16 just before the MFMA
      const unsigned char* b8 = reinterpret_cast<const unsigned char*>(bv);
      const int grp = lane >> 4, r16 = lane & 15, aa = r16 & 1, kk = r16 >> 1;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int row = 16 * ks + 8 * (kk >> 2) + 4 * (grp >> 1) + (kk & 3);
          const int lc = 2 * (db + dh * NDB) + (grp & 1);
          const u32x2 vw = read_tr8(b8 + row * D + 16 * (lc ^ swzv(row)) + 8 * aa);
          oacc[db] = mfma32(as_bf16x8(fp8x8_to_bf16x8(vw)), as_bf16x8(pf[ks]), oacc[db]);
        }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // consecutive MFMAs feed different accumulators
        u32x4 vw;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x2 t = read_tr16(&bv[v_elem(ks, half, db)]);
          vw[2 * half] = t[0];
          vw[2 * half + 1] = t[1];
        }
        oacc[db] = mfma32(as_bf16x8(vw), as_bf16x8(pf[ks]), oacc[db]);
      }
    }
  };

  // Register-staged forms, used by the one-wave split kernel: a tile's operand
  // fragments are first read out of LDS, so its buffer can be refilled before
  // the MFMAs run. Same addresses as scores/accumulate above.
  auto read_k = [&](const uint16_t* bk, u32x4 (&kr)[NQC][NKB]) {
#pragma unroll
    for (int c = 0; c < NQC; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = 32 * kb + j;
        const int ch = 2 * (c + dh * NQC) + hl;
        kr[c][kb] = *reinterpret_cast<const u32x4*>(&bk[row * D + 8 * (ch ^ swz_k<D>(row))]);
      }
  };
  // S^T from registers; even and odd d steps feed two accumulators so that
  // the dependent MFMA chain is half as long.
  auto scores_regs = [&](const u32x4 (&kr)[NQC][NKB], f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s0{}, s1{};
#pragma unroll
      for (int c = 0; c < NQC; c += 2) {
        s0 = mfma32(as_bf16x8(kr[c][kb]), qf[c], s0);
        if (c + 1 < NQC) s1 = mfma32(as_bf16x8(kr[c + 1][kb]), qf[c + 1], s1);
      }
      s[kb] = s0 + s1;
    }
  };
  auto read_v = [&](const uint16_t* bv, u32x4 (&vr)[NKS][NDB]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x2 t = read_tr16(&bv[v_elem(ks, half, db)]);
          vr[ks][db][2 * half] = t[0];
          vr[ks][db][2 * half + 1] = t[1];
        }
      }
  };
  // fp8 tiles (KV8): K rows are read 8 bytes (8 d values) per lane and
  // widened to bf16; V^T comes from ds_read_b64_tr_b8: the lane in position
  // (group G, r = 2 k + a) of each 16-lane group addresses key 16 ks +
  // 8 (k / 4) + 4 (G / 2) + k % 4 at d 32 db + 16 (G % 2) + 8 a, so that lane
  // l receives V[key][32 db + l % 32] for its 8 keys in the order of the P^T
  // operand (keys 4 hl + 0..3, then 8 + 4 hl + 0..3 of the 16-key step).
  // The fragments stay as fp8 bytes in registers (half the registers of
  // bf16) and are widened just before their MFMA.
  auto read_k8 = [&](const uint16_t* bk, u32x2 (&kr)[NQC][NKB]) {
    const unsigned char* b8 = reinterpret_cast<const unsigned char*>(bk);
#pragma unroll
    for (int c = 0; c < NQC; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = 32 * kb + j;
        kr[c][kb] = *reinterpret_cast<const u32x2*>(b8 + row * D + 16 * (c ^ swzk(row)) + 8 * hl);
      }
  };
  auto scores_regs8 = [&](const u32x2 (&kr)[NQC][NKB], f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s0{}, s1{};
#pragma unroll
      for (int c = 0; c < NQC; c += 2) {
        s0 = mfma32(as_bf16x8(fp8x8_to_bf16x8(kr[c][kb])), qf[c], s0);
        if (c + 1 < NQC) s1 = mfma32(as_bf16x8(fp8x8_to_bf16x8(kr[c + 1][kb])), qf[c + 1], s1);
      }
      s[kb] = s0 + s1;
    }
  };
  auto read_v8 = [&](const uint16_t* bv, u32x2 (&vr)[NKS][NDB]) {
    const unsigned char* b8 = reinterpret_cast<const unsigned char*>(bv);
    const int grp = lane >> 4, r16 = lane & 15, aa = r16 & 1, kk = r16 >> 1;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int row = 16 * ks + 8 * (kk >> 2) + 4 * (grp >> 1) + (kk & 3);
        const int lc = 2 * db + (grp & 1);
        vr[ks][db] = read_tr8(b8 + row * D + 16 * (lc ^ swzv(row)) + 8 * aa);
      }
  };
  auto accumulate_regs8 = [&](const u32x2 (&vr)[NKS][NDB], const u32x4 (&pf)[NKS]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(as_bf16x8(fp8x8_to_bf16x8(vr[ks][db])), as_bf16x8(pf[ks]), oacc[db]);
  };
  auto accumulate_regs = [&](const u32x4 (&vr)[NKS][NDB], const u32x4 (&pf)[NKS]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(as_bf16x8(vr[ks][db]), as_bf16x8(pf[ks]), oacc[db]);
  };

  // D split: publish this wave's partial scores, and add the group's.
  auto publish = [&](const f32x16 (&s)[NKB], int slot) {
    if constexpr (DS > 1) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) sX[slot % XSLOTS][wave][kb * 16 + x][lane] = s[kb][x];
    }
  };
  auto combine_partner = [&](f32x16 (&s)[NKB], int slot) {
    if constexpr (DS > 1) {
      // every wave of the group adds the DS parts in the same order (part 0
      // first), so all of them hold bit-identical scores; only the other
      // waves' parts are read back
      const int w0 = rg * DS;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          if constexpr (DS == 2) {
            const float other = sX[slot % XSLOTS][wave ^ 1][kb * 16 + x][lane];
            s[kb][x] = dh == 0 ? s[kb][x] + other : other + s[kb][x];
          } else {
            float part[DS];
#pragma unroll
            for (int k = 0; k < DS; ++k) part[k] = s[kb][x];
#pragma unroll
            for (int k = 0; k < DS; ++k)
              if (k != dh) part[k] = sX[slot % XSLOTS][w0 + k][kb * 16 + x][lane];
            float acc = part[0];
#pragma unroll
            for (int k = 1; k < DS; ++k) acc += part[k];
            s[kb][x] = acc;
          }
        }
    }
  };

  // VALU instructions of one tile's exponentiation per lane: an FMA and an
  // exp per score, one add per score and one pack per pair
  constexpr int kExpValuPerTile = NKB * 16 * 3 + NKB * 8;

  auto kbuf = [&](int i) -> uint16_t* { return i == 0 ? sK0 : i == 1 ? sK1 : i == 2 ? sK2 : sK3; };
  auto vbuf = [&](int i) -> uint16_t* { return i == 0 ? sV0 : i == 1 ? sV1 : i == 2 ? sV2 : sV3; };

  if constexpr (SPLIT) {
    // ======================= split-KV: persistent Stream-K =====================
    const int C = a.chunk;
    const int tpc = (C + BN - 1) / BN;          // tiles per chunk
    const int W = gridDim.x, w = blockIdx.x;
    const int64_t cap = (int64_t)a.max_pages << a.page_shift;
    auto clamp_len = [&](int v) -> int { return (int)min(max((int64_t)v, (int64_t)0), cap); };
    // tiles of every block of rows of one sequence (per KV head)
    auto seq_tiles = [&](int len) -> int {
      int n = 0;
      for (int r = 0; r < a.n_rb; ++r) n += row_span<BN, BM>(a, len, r, tpc).nt;
      return n;
    };

    // Partial slot of query row (qi, head qh) of sequence b.
    auto slot_index = [&](int s_) -> int64_t {
      return (((int64_t)b * a.Hq + qh) * a.Sq + qi) * a.n_slots + s_;
    };
    // Normalised partial output and LSE of the current state into slot s_.
    auto write_partial = [&](int s_) {
      const float l_tot = pair_sum(l_run);
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : fast_rcp(l_tot) * vsc;
      const float lse_v = empty ? -INFINITY : (m_run * sl2 + fast_log2(l_tot)) * kLn2;
      if (row_ok) {
        const int64_t prow = slot_index(s_);
        float* dst = a.o_part + prow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int d0 = 32 * (db + dh * NDB) + 8 * rr + 4 * hl;
            f32x4 val = {oacc[db][4 * rr + 0] * inv, oacc[db][4 * rr + 1] * inv,
                         oacc[db][4 * rr + 2] * inv, oacc[db][4 * rr + 3] * inv};
            *reinterpret_cast<f32x4*>(dst + d0) = val;
          }
        if (hl == 0 && dh == 0) a.lse_part[prow] = lse_v;
      }
    };
    // Slots [s0, s1) of the current rows hold no key (LSE -inf; the combine
    // never reads their O).
    auto write_empty = [&](int s0, int s1) {
      if (row_ok && hl == 0 && dh == 0)
        for (int s_ = s0; s_ < s1; ++s_) a.lse_part[slot_index(s_)] = -INFINITY;
    };
    auto reset_state = [&]() {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
      m_run = -INFINITY;
      nb_ref = 0.f;
      l_run = 0.f;
    };

    // ---- total tile count T, lane-parallel over sequences -------------------
    // The lengths of sequences bc0 + lane + 64 r stay in lane registers: the
    // tile iterators read them with readlane, so moving to the next sequence
    // costs no memory access (a global load would wait for every copy in
    // flight).
    int lenc[4] = {0, 0, 0, 0};
    int bc0 = 0;
    int T = 0;
    for (int b0 = 0; b0 < a.B; b0 += 256) {
      int lv[4];
      int part_sum = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int bb = b0 + lane + 64 * r;
        lv[r] = bb < a.B ? clamp_len(a.seq_lens[bb]) : 0;
        part_sum += bb < a.B ? seq_tiles(lv[r]) : 0;
      }
      if (b0 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) lenc[r] = lv[r];
      }
      T += wave_sum_i32(part_sum);
    }
    auto len_of = [&](int bb) -> int {
      const int d = bb - bc0;
      if (d >= 0 && d < 256) {
        const int r = d >> 6, l = d & 63;
        const int v = r == 0 ? lenc[0] : r == 1 ? lenc[1] : r == 2 ? lenc[2] : lenc[3];
        return __builtin_amdgcn_readlane(v, l);
      }
      return __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens[bb]));
    };

    // ---- block rows with no visible key: every slot of their rows is empty ---
    for (int bb = w; bb < a.B; bb += W) {
      const int len = len_of(bb);
      const int nch = (int)(((int64_t)len + C - 1) / C);
      if (nch == 0) continue;
      for (int r = 0; r < a.n_rb; ++r) {
        if (row_span<BN, BM>(a, len, r, tpc).nt > 0) continue;
        for (int gg = 0; gg < a.Hkv; ++gg) {
          set_rows(bb, gg, r, len);
          write_empty(0, nch + 1);
        }
      }
    }

    // ---- this workgroup's KV head and tile range [x0, x1) -------------------
    // (the grid is a multiple of Hkv workgroups)
    const int g_w = w % a.Hkv;
    const int sets = W / a.Hkv;
    if constexpr (KV8) {
      // fold the head's K scale into the exponent factor (or the score scale)
      const float ksc = a.k_scale[g_w];
      vsc = a.v_scale[g_w];
      if constexpr (kXform) xscale = a.scale * ksc;
      else sl2 = a.sl2 * ksc;
      thr = kRescaleLog2 / sl2;
    }
    // a range holds at least one chunk, so the rows of a sequence meet at
    // most (its chunks + 1) ranges
    const int per = (int)max(((int64_t)T + sets - 1) / sets, (int64_t)tpc);
    const int64_t x0l = (int64_t)(w / a.Hkv) * per;
    if (x0l >= T) return;
    const int x0 = (int)x0l;
    const int x1 = (int)min(x0l + per, (int64_t)T);
    const int n_loc = x1 - x0;

    // Tile iterator over the global order (sequence, block of rows, tile);
    // all fields are uniform.
    struct It {
      int b, len, rb, i, nt, c, k, c_lo, k0, c_hi, k1;
    };
    auto it_span = [&](It& t, const RowSpan& sp) {
      t.nt = sp.nt; t.c_lo = sp.c_lo; t.k0 = sp.k0; t.c_hi = sp.c_hi; t.k1 = sp.k1;
      t.i = 0; t.c = sp.c_lo; t.k = sp.k0;
    };
    auto it_next = [&](It& t) {
      if (++t.i < t.nt) {
        if (++t.k == tpc) { t.k = 0; ++t.c; }
        return;
      }
      for (;;) {
        if (++t.rb == a.n_rb) {
          t.rb = 0;
          if (++t.b >= a.B) { t.nt = 0; return; }   // past the last tile
          t.len = len_of(t.b);
        }
        const RowSpan sp = row_span<BN, BM>(a, t.len, t.rb, tpc);
        if (sp.nt > 0) { it_span(t, sp); return; }
      }
    };

    // ---- locate tile x0 -------------------------------------------------------
    It cu;
    {
      int bx = 0, sx = 0, base = 0;
      bool found = false;
      for (int b0 = 0; b0 < a.B && !found; b0 += 256) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int bb = b0 + lane + 64 * r;
          const int len = b0 == 0 ? lenc[r] : (bb < a.B ? clamp_len(a.seq_lens[bb]) : 0);
          const int t = bb < a.B ? seq_tiles(len) : 0;
          const int incl = wave_incl_scan_i32(t, lane) + base;
          const uint64_t m = __builtin_amdgcn_ballot_w64(!found && bb < a.B && incl > x0);
          if (m != 0) {
            const int L = __builtin_ctzll(m);
            bx = b0 + 64 * r + L;
            sx = __builtin_amdgcn_readlane(incl - t, L);
            found = true;
          }
          base = __builtin_amdgcn_readlane(incl, 63);
        }
      }
      if (!found) return;                      // (x0 < T always finds it)
      cu.b = bx;
      cu.len = len_of(bx);
      int o = x0 - sx;
      RowSpan sp{0, 0, 0, 0, 0};
      for (cu.rb = 0; cu.rb < a.n_rb; ++cu.rb) {
        sp = row_span<BN, BM>(a, cu.len, cu.rb, tpc);
        if (o < sp.nt) break;
        o -= sp.nt;
      }
      if (cu.rb == a.n_rb || sp.nt == 0) return;
      it_span(cu, sp);
      cu.i = o;
      if (cu.i < tpc - cu.k0) {
        cu.k = cu.k0 + cu.i;
      } else {
        const int i2 = cu.i - (tpc - cu.k0);
        cu.c = cu.c_lo + 1 + i2 / tpc;
        cu.k = i2 % tpc;
      }
    }
    auto tile_tb = [&](const It& t) -> int { return t.c * C + t.k * BN; };
    auto tile_ke = [&](const It& t) -> int { return (int)min((int64_t)(t.c + 1) * C, (int64_t)t.len); };
    auto n_chunks = [&](const It& t) -> int { return (int)(((int64_t)t.len + C - 1) / C); };

    set_rows(cu.b, g_w, cu.rb, cu.len);
    // a row's first tile also marks the chunks before its visible keys empty
    // This range's slot in the rows' partials: ranges are [r per, (r + 1)
    // per); the rows' first tile (global index x_first) lies in range r0.
    int slot = x0 / per - (x0 - cu.i) / per;
    // ---- copy pipeline --------------------------------------------------------
    // The loop keeps as many copies in flight as the ring holds instead of
    // overlapping MFMA and softmax. Each buffer is refilled as soon as its
    // tile is consumed: K(t + NBUF) right after the scores of tile t,
    // V(t + NBUF) right after its PV product, so at every wait 2 (NBUF - 1) of
    // the 2 NBUF buffers are still being filled. Copy order: K0 V0 K1 V1 ..
    // K(NBUF-1) V(NBUF-1), then per step t V(t + NBUF - 1) (refilling tile
    // t-1's V buffer) and K(t + NBUF). The tiles in flight may belong to later
    // rows: the V copy of step t is for the tile whose K was copied one step
    // earlier, so one descriptor (key start, key end, V base, sequence) of
    // that tile is kept.
    constexpr int AHEAD_CP = 2 * (NBUF - 1) * SEGW < 63 ? 2 * (NBUF - 1) * SEGW : 63;
    // Without a D split the waves read each tile into registers as soon as
    // it lands and the buffer is refilled once all have read it (the refill
    // then does not wait for the tile's MFMAs and softmax): per step
    // K(t + NBUF) right after K(t) is read, V(t + NBUF) right after V(t) is
    // read, so with the ring kept full 2 NBUF - 1 of the 2 NBUF buffers are
    // being filled at every wait (how far the waits let copies run ahead is
    // chosen per kernel below).
    constexpr bool EARLY = DS == 1;
    constexpr int AHEAD_E = (2 * NBUF - 1) * SEGW < 63 ? (2 * NBUF - 1) * SEGW : 63;
    // Stores count in vmcnt too, in issue order with the copies: after a
    // partial output is written, the next few waits also wait for some
    // copies newer than their target (rare: once per range or block of rows).
    // The waits take exactly two forms, so the compiler can tell that a
    // tile's copies are complete and adds no wait of its own.
    // Except in the multi-wave kernels over a paged cache, each wait drains
    // every copy instead. Measured on MI355X, the cache then streams faster:
    // decode over 16 sequences of 1k-16k tokens 85 us against 92 us with the
    // ring kept full (the KV-head workgroups that read the same tokens stay
    // in step), the same over 16-token pages 2 % faster, while the 64-row
    // verify over 32k tokens in 16-token pages is 2-5 % faster with the ring
    // kept full.
    constexpr bool DRAIN = !(PAGED && NW > 1);
    auto wait_e = [&](bool deep) {
      if (!deep || DRAIN) wait_vm<0>();
      else wait_vm<AHEAD_E>();
    };
    It pf = cu;
    int d_tb = 0, d_ke = 0, d_b = 0;
    const uint16_t* d_vb = nullptr;
    auto issue_next_k = [&](uint16_t* dst) {   // K of the prefetch iterator's tile
      const uint16_t* kb_;
      kv_bases(pf.b, g_w, kb_, d_vb);
      d_tb = tile_tb(pf);
      d_ke = tile_ke(pf);
      d_b = pf.b;
      issue(d_tb, d_ke, kb_, d_b, false, dst);
    };
#pragma unroll
    for (int jj = 0; jj < NBUF; ++jj) {
      if (jj < n_loc) {
        issue_next_k(kbuf(jj));
        issue(d_tb, d_ke, d_vb, d_b, true, vbuf(jj));
        if (jj + 1 < n_loc) it_next(pf);
      }
    }
    // Wait for the rows' Q fragments and this first ring together. While
    // loads into registers and copies into LDS are both outstanding, the
    // compiler makes any wait it needs a wait for everything; waiting here,
    // once per workgroup, costs about the first tiles' latency (which the
    // first step waits for anyway) and leaves the loop with copies only, so
    // its waits stay the explicit ones below.
    wait_vm<0>();
    // ---- after a tile: close the partial if its chunk or rows end here ------
    // The rows change exactly after their last tile; inside the rows the
    // chunk changes exactly after its last tile.
    // ---- after a tile: close the partial if the range or the rows end here --
    // The chunks of a range merge in the running softmax; the rows change
    // exactly after their last tile.
    auto finish_tile = [&](int it) {
      const bool range_end = it + 1 == n_loc;
      const bool rows_end = cu.i == cu.nt - 1;
      if (range_end || rows_end) {
        write_partial(slot);
        // the range holding the rows' last tile marks their unused slots
        // (up to chunks + 1) empty
        if (rows_end) write_empty(slot + 1, n_chunks(cu) + 1);
        reset_state();
      }
      if (!range_end) {
        it_next(cu);
        if (rows_end) {
          set_rows(cu.b, g_w, cu.rb, cu.len);
          // the new rows' Q fragments are the newest loads in flight: wait
          // for them here, on this rare path, so the compiler need not make
          // the next scores wait for every copy in flight on every path
          wait_vm<0>();
          slot = 0;                                // the rows start inside this range
        }
      }
    };
    auto sstep = [&](int it, int u) {
      const int tb = tile_tb(cu);
      if constexpr (EARLY) {
        // K(t) landed (copies issued after it: V(t) and the tiles behind)
        wait_e(it + NBUF - 1 < n_loc);
        lds_barrier();
        load_mask(tb);
        // K(t) fragments in registers (raw fp8 bytes for an fp8 cache)
        u32x4 kr[KV8 ? 1 : NQC][KV8 ? 1 : NKB];
        u32x2 kr8[KV8 ? NQC : 1][KV8 ? NKB : 1];
        if constexpr (KV8) read_k8(kbuf(u), kr8);
        else read_k(kbuf(u), kr);
        wait_lgkm0();
        if constexpr (NW > 1) lds_barrier();     // every wave has read K(t)
        __builtin_amdgcn_sched_barrier(0);
        if (it + NBUF < n_loc) {
          issue_next_k(kbuf(u));
          if (it + NBUF + 1 < n_loc) it_next(pf);
        }
        ke = tile_ke(cu);
        f32x16 sc[NKB];
        if constexpr (KV8) scores_regs8(kr8, sc);
        else scores_regs(kr, sc);
        const float nb = prepare(sc, tb);
        u32x4 pv[NKS];
        exponentiate(sc, nb, pv);
        // V(t) landed (copies issued after it: the tiles behind and K(t + NBUF))
        wait_e(it + NBUF < n_loc);
        lds_barrier();
        u32x4 vr[KV8 ? 1 : NKS][KV8 ? 1 : NDB];
        u32x2 vr8[KV8 ? NKS : 1][KV8 ? NDB : 1];
        if constexpr (KV8) read_v8(vbuf(u), vr8);
        else read_v(vbuf(u), vr);
        wait_lgkm0();
        if constexpr (NW > 1) lds_barrier();     // every wave has read V(t)
        __builtin_amdgcn_sched_barrier(0);
        if (it + NBUF < n_loc) issue(d_tb, d_ke, d_vb, d_b, true, vbuf(u));
        if constexpr (KV8) accumulate_regs8(vr8, pv);
        else accumulate_regs(vr, pv);
      } else {
        // The copy order after the prologue is, per step t, V(t + NBUF - 1)
        // (refilling tile t-1's V buffer) then K(t + NBUF).
        // uniform: a full ring behind this tile (the 576-wide-key kernel, whose
        // K groups carry one more copy, waits for every copy instead)
        const bool deep = !KX && it + NBUF - 1 < n_loc;
        // K(t) landed in every wave's share; every wave is done with the PV
        // product of tile t-1, whose V buffer is refilled next
        if (deep) wait_vm<AHEAD_CP>(); else wait_vm<0>();
        lds_barrier();
        load_mask(tb);
        if (it >= 1 && it + NBUF - 1 < n_loc) issue(d_tb, d_ke, d_vb, d_b, true, vbuf((u + NBUF - 1) % NBUF));
        ke = tile_ke(cu);
        f32x16 sc[NKB];
        scores(kbuf(u), sc);
        if constexpr (DS > 1) {
          publish(sc, it & 1);
          lds_barrier();
          combine_partner(sc, it & 1);
        }
        const float nb = prepare(sc, tb);
        u32x4 pv[NKS];
        exponentiate(sc, nb, pv);
        // V(t) landed; every wave is done with K(t), whose buffer is refilled
        if (deep) wait_vm<AHEAD_CP>(); else wait_vm<0>();
        lds_barrier();
        if (it + NBUF < n_loc) {
          issue_next_k(kbuf(u));
          if (it + NBUF + 1 < n_loc) it_next(pf);
        }
        accumulate(vbuf(u), pv);
      }
      finish_tile(it);
    };
    for (int it = 0; it < n_loc; it += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        if (it + u >= n_loc) break;
        sstep(it + u, u);
      }
    }
  } else {
    // ======================= prefill: blocks of rows ==========================
    // One block of rows per workgroup, or (PERS) a persistent grid: the
    // workgroups on XCD x (workgroup w runs on XCD w % 8) take, in zig-zag
    // rounds, the blocks a one-block-per-workgroup grid would give that XCD
    // (xcd_remap), heaviest first within each (b, KV head). Consecutive
    // rounds pair heavy with light blocks, so the workgroups of an XCD get
    // nearly equal work, and the blocks sharing K/V share an L2.
    const int n = a.B * a.Hkv * a.n_rb;
    const int n_keys = a.skv;
    ke = n_keys;
    const int rows = a.Sq * a.G;
    const int shift = n_keys - a.Sq;
    auto pers_item = [&](int r) -> int {
      constexpr int X = 8;
      const int G = gridDim.x, w = blockIdx.x;
      // fewer workgroups than XCDs (a small grid): some XCD would have no
      // workgroup for its chunk, so the blocks are dealt round-robin instead
      if (G < X) {
        const int64_t Lr = (int64_t)r * G + w;
        return Lr < n ? (int)Lr : -1;
      }
      const int x = w % X, k = w / X;
      const int P = G / X + (x < G % X ? 1 : 0);
      const int per = n / X, rem = n % X;
      const int cnt = per + (x < rem ? 1 : 0);
      const int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
      const int jl = r * P + ((r & 1) ? P - 1 - k : k);
      return jl < cnt ? base + jl : -1;
    };
    // the whole tiles holding the keys block rb_ may attend to
    auto block_tiles = [&](int rb_, int& t_start_, int& n_tiles_) {
      const int r_lo_ = rb_ * BM, r_hi_ = min(r_lo_ + BM, rows);
      const int pmin = r_lo_ / a.G + shift, pmax = (r_hi_ - 1) / a.G + shift;
      int kv_lo = 0, kv_hi = n_keys;
      if (a.causal) {
        kv_hi = min(kv_hi, pmax + 1);
        if (a.window > 0) kv_lo = max(kv_lo, pmin - a.window + 1);
      }
      t_start_ = (max(kv_lo, 0) / BN) * BN;
      n_tiles_ = kv_hi > kv_lo ? (kv_hi - t_start_ + BN - 1) / BN : 0;
    };
    int L = PERS ? pers_item(0) : xcd_remap(blockIdx.x, n);
    bool pre = false;    // PERS: this block's Q fragments and first tiles are already loading
    for (int round = 0; L >= 0; ++round) {
    const int bg = L / a.n_rb;
    const int rb = a.n_rb - 1 - (L % a.n_rb);   // heaviest causal row blocks first
    const int bq = bg / a.Hkv;
    const int g = bg % a.Hkv;
    const int r_lo = rb * BM;
    const int r_hi = min(r_lo + BM, rows);
    int t_start = 0, n_tiles = 0;
    block_tiles(rb, t_start, n_tiles);
    set_rows(bq, g, rb, n_keys, !pre);
    if constexpr (PERS) {
      if (round > 0) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
        m_run = -INFINITY;
        nb_ref = 0.f;
        l_run = 0.f;
      }
    }
    const uint16_t* kseq;
    const uint16_t* vseq;
    kv_bases(bq, g, kseq, vseq);
    auto issue_k = [&](int tb, uint16_t* dst) { issue(tb, n_keys, kseq, bq, false, dst); };
    auto issue_v = [&](int tb, uint16_t* dst) { issue(tb, n_keys, vseq, bq, true, dst); };
    int L_next = -1;

    if constexpr (PP) {
      // ---- main loop, two wave groups in ping-pong -----------------------------
      // Waves w and w + 4 share a SIMD. Group 0 (waves 0-3) holds rows 0-127
      // of the block and group 1 rows 128-255; both read the same K/V tiles.
      // Every wave runs the same program: the scores of tile 0, then per
      // tile t a softmax slot (mask, max, exponentiate tile t) and an MFMA
      // slot (the scores of tile t+1, then O += P V with tile t), each ended
      // by a workgroup barrier. Group 1 passes one extra barrier first, so it
      // runs one slot behind: while group 0 exponentiates, group 1 runs its
      // MFMA block, and the other way round. Each SIMD then always has one
      // wave feeding its matrix core and one on the VALU. (Measured on
      // MI355X: a VALU wave beside an MFMA wave leaves the MFMA rate
      // unchanged, while VALU work inside the MFMA wave's own stream slows
      // it once there are more than ~4 VALU instructions per 32x32x16 MFMA;
      // the softmax needs ~4.)
      //
      // Copies: a ring of three buffers per operand; every wave copies two
      // 1 KiB segments of each tile of K and V. Issuing a copy stalls the
      // issuing wave (the CU's vector memory unit takes ~10 cycles per 1 KiB
      // copy, more under load: measured ~75 cycles per copy per wave), so
      // the copies are split between the slots: in its softmax slot of tile
      // t a wave copies its segments of K(t+2) into the buffer of K(t-1),
      // and in its MFMA slot of tile t, between MFMAs, those of V(t+2) into
      // the buffer of V(t-1); both buffers' last readers are the MFMA slots
      // of the tile before, done by then in either group. At the end of its
      // MFMA slot of tile t a wave waits until only that slot's two copies
      // are in flight: for group 0 that covers K(t+2) (needed from the
      // second slot of tile t+1 on) and V(t+1); for group 1, one slot behind,
      // the same. Past the last tile the copies repeat the last tile into
      // the same, free, buffers, so that every slot issues the same number
      // of copies and the waits are exact (which also lets the compiler's
      // own LDS hazard tracking see that no MFMA slot reads a buffer with a
      // copy in flight).
      static_assert(NBUF == 3 && SEGW == 2, "three tile buffers; two segments per wave and operand");
      const int grp = wave >> 2;          // uniform
      f32x16 sc[NKB];
      u32x4 pf[NKS];
      // this wave's two segments of one operand of the tile at key tb, as
      // prefill_seg, with the per-lane parts of the source offsets (fixed
      // for a wave) computed once: the softmax slot is the later one of the
      // two, and each copy there then costs three VALU instructions instead
      // of about seven
      uint32_t kof[SEGW], vof[SEGW];
      int crow[SEGW];
#pragma unroll
      for (int i = 0; i < SEGW; ++i) {
        const int sg = wave * SEGW + i;
        kof[i] = p_lrk + 16u * (uint32_t)p_kchunk(sg);
        vof[i] = p_lrv + 16u * (uint32_t)p_vchunk(sg);
        crow[i] = sg * RPS + p_lr;
      }
      auto copy2 = [&](int tb, const uint16_t* kv_base, bool is_v, uint16_t* dst) __attribute__((always_inline)) {
        const int lim = n_keys - 1 - tb;
        const int rsb = ES * (is_v ? v_rs : k_rs);
        const char* tbase = reinterpret_cast<const char*>(kv_base) + (int64_t)tb * rsb;
#pragma unroll
        for (int i = 0; i < SEGW; ++i) {
          const int sg = wave * SEGW + i;
          const uint32_t o = (is_v ? vof[i] : kof[i]) - (uint32_t)(max(crow[i] - lim, 0) * rsb);
          dma16_buf_s<false>(tbase, o, (uint32_t)(sg * RPS * rsb), dst + sg * 512);
        }
      };
      // softmax slot of tile t (ring position u = t % 3), at raised
      // priority: the issue arbiter then serves its VALU stream before the
      // partner's MFMA and LDS issue (measured +0.6 %; raising the MFMA slot
      // instead gained nothing)
      auto vphase = [&](int t, int u) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        copy2(t_start + min(t + 2, n_tiles - 1) * BN, kseq, false, kbuf((u + 2) % 3));
        softmax_tile(sc, t_start + t * BN, pf);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) pin_vgpr(pf[ks]);
        pin_vgpr(l_run);
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();
      };
      // MFMA slot of tile t: the next tile's scores (after the last tile, of
      // whatever the buffer holds: unused), then O^T += V^T P^T with V(t)
      auto mphase = [&](int t, int u) __attribute__((always_inline)) {
        scores(kbuf((u + 1) % 3), sc);
        copy2(t_start + min(t + 2, n_tiles - 1) * BN, vseq, true, vbuf((u + 2) % 3));
        accumulate(vbuf(u), pf);
        // operand reads six ahead of their MFMAs (measured against 4, 8 and
        // 10 ahead: +1.0 %, +0.6 %, +0.8 % for 6 over each)
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        sched_cont<NKB * NQC, 1, NDB * NKS, 2, 6, 0, 3, 9, 0>();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) pin_vgpr(sc[kb]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) pin_vgpr(oacc[db]);
        wait_vm<SEGW>();
        lds_barrier();
      };
      if (n_tiles > 0) {
        issue_k(t_start, kbuf(0));
        issue_v(t_start, vbuf(0));
        if (n_tiles > 1) {
          issue_k(t_start + BN, kbuf(1));
          issue_v(t_start + BN, vbuf(1));
        }
        wait_vm<0>();
        lds_barrier();
        if (grp == 1) lds_barrier();      // group 1: one slot behind
        scores(kbuf(0), sc);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) pin_vgpr(sc[kb]);
        lds_barrier();
        for (int t = 0; t < n_tiles; t += 3) {
          vphase(t, 0);
          mphase(t, 0);
          if (t + 1 < n_tiles) {
            vphase(t + 1, 1);
            mphase(t + 1, 1);
          }
          if (t + 2 < n_tiles) {
            vphase(t + 2, 2);
            mphase(t + 2, 2);
          }
        }
        wait_vm<0>();                     // no copy lands in the staging below
        if (grp == 0) lds_barrier();      // matches group 1's extra barrier
      }
    } else {
      // ---- main loop, software-pipelined ---------------------------------------
      // Step t: the scores of tile t are already in registers. After the
      // barrier (tile t+1's K and tile t's V have landed in LDS, and every wave
      // is done with step t-1), the wave starts the copies of K(t+NBUF) and
      // V(t+NBUF-1) into the buffers step t-1 released, runs the S^T MFMAs of
      // tile t+1 while the VALU exponentiates tile t, then accumulates O with
      // tile t's V. The MFMA work of S(t+1) overlaps the softmax of tile t
      // inside one wave, and NBUF-1 tiles of copies stay in flight. The copies
      // of one step (K(t+1+j), V(t+j)) form a group; the wait before step t
      // lets the groups issued after group t stay outstanding. Buffer indices
      // are compile-time constants in the unrolled ring.
      constexpr int GROUP = 2 * SEGW + (KX ? 1 : 0);          // copy instructions per group
      // Where a step issues its copies. Issuing a copy stalls the issuing
      // wave (measured ~40-75 cycles per copy with several waves of a CU
      // issuing), so the copies go where the stall hides best:
      // * head dim 512 (one wave per SIMD, 16 copies per wave and step):
      //   after the first two batches of MFMAs, eight after each. At the
      //   top of the step the stalls left the matrix cores idle, and copies
      //   spread to the end of the step made the next step wait for them
      //   (measured, C4B: top of the step 1.61 ms, two after every batch
      //   1.58, four after each score batch 1.55, eight after each of the
      //   first two 1.47-1.52; the batches are now two MFMAs each, and the
      //   copies go out after the first two of them);
      // * head dim 256: inside the MFMA block, after the scores' MFMAs are
      //   issued (C4A 0.215 -> 0.205 ms; after the softmax bookkeeping
      //   instead: no change);
      // * otherwise, and for 576-wide key tiles: at the top of the step.
      // The first two place copies with the branch-free segment copy and,
      // past the last tile, repeat the last tile into the same free
      // buffers, so every step issues the same copies and the waits stay
      // exact; a last wait after the loop drains them.
      constexpr bool kCopyBatched = D >= 512 && !KX;
      constexpr bool kCopyInBlock = D == 256;
      constexpr bool kPrioMfma = D <= 128;
      constexpr int LATER_STEP = (NBUF - 2) * GROUP < 63 ? (NBUF - 2) * GROUP : 63;
      constexpr int LATER_PRO = (NBUF - 1) * GROUP < 63 ? (NBUF - 1) * GROUP : 63;
      f32x16 sc[NKB];
      // the first tiles: K(0 .. NBUF-1), V(0 .. NBUF-2) of the block starting at key ts_
      auto issue_first = [&](int ts_, int nt_, const uint16_t* kb_, const uint16_t* vb_, int b_) {
        issue(ts_, n_keys, kb_, b_, false, kbuf(0));
#pragma unroll
        for (int jj = 0; jj < NBUF - 1; ++jj) {
          if (jj + 1 < nt_) issue(ts_ + (jj + 1) * BN, n_keys, kb_, b_, false, kbuf(jj + 1));
          if (jj < nt_) issue(ts_ + jj * BN, n_keys, vb_, b_, true, vbuf(jj));
        }
      };
      if (n_tiles > 0) {
        if (!pre) issue_first(t_start, n_tiles, kseq, vseq, bq);
        // (a block whose first tiles were issued during the previous block's
        // end waits for everything: that block's O stores followed them)
        if (pre || NBUF - 1 >= n_tiles) wait_vm<0>(); else wait_vm<LATER_PRO>();
        lds_barrier();
        scores(kbuf(0), sc);
        publish(sc, 0);
      }
      auto step = [&](int it, int u) {
        const int tb = t_start + it * BN;
        if (it + NBUF - 1 < n_tiles) wait_vm<LATER_STEP>(); else wait_vm<0>();
        lds_barrier();
        // At head dim 512 (one wave per SIMD) the partner's scores are read
        // first, so their LDS latency overlaps the copy issue below (measured:
        // 1.79 -> 1.63 ms for the head-dim-512 causal workload; at head dim 256,
        // two waves per SIMD, the other order is 2 % faster); they are added
        // in once the first MFMAs of S(t+1) are under way.
        constexpr bool kBig = D >= 512;
        float oth[kBig ? 16 : 1];
        if constexpr (kBig) {
          static_assert(DS == 2 && NKB == 1, "head dim 512: two waves share the scores of a 32-key tile");
#pragma unroll
          for (int x = 0; x < 16; ++x) oth[x] = sX[(it & 1) % XSLOTS][wave ^ 1][x][lane];
        }
        load_mask(tb);
        if constexpr (!kCopyBatched && !kCopyInBlock) {
          if (it + NBUF < n_tiles) issue_k(tb + NBUF * BN, kbuf(u));
          if (it + NBUF - 1 < n_tiles) issue_v(tb + (NBUF - 1) * BN, vbuf((u + NBUF - 1) % NBUF));
        }
        float nb = 0.f;
        u32x4 kpre[kBig ? 1 : NPRE];
        if constexpr (!kBig) {
#pragma unroll
          for (int x = 0; x < NPRE; ++x) kpre[x] = k_frag(kbuf((u + 1) % NBUF), x);
          combine_partner(sc, it & 1);
          nb = prepare(sc, tb);
        }
        f32x16 sn[NKB];
        // Up to D = 128 two workgroups share a CU, so each SIMD runs waves of
        // both. A wave raises its priority for its MFMA block and drops it for
        // the softmax bookkeeping and barrier that follow, so the issue
        // arbiter feeds the matrix cores first (measured +2.4 % at head dim
        // 128; with one workgroup per CU it gains nothing).
        if constexpr (kPrioMfma) __builtin_amdgcn_s_setprio(1);
        if constexpr (D >= 512) {
          // Head dim 512 runs one wave per SIMD, so nothing covers a wave's
          // own LDS latency, and its registers are too full for the compiler
          // to keep more than one operand read in flight on its own. The step
          // is written in explicit batches instead: the reads of the next
          // batch are issued before the MFMAs of the current one (a schedule
          // fence between batches); the first batch of S(t+1) is issued before
          // tile t's exchange and softmax bookkeeping, which then run while it
          // computes, and tile t's exponentiation is spread over the other
          // S(t+1) batches.
          const uint16_t* bk = kbuf((u + 1) % NBUF);
          const uint16_t* bv = vbuf(u);
          // MFMAs per batch: two (measured against one, four and eight:
          // C4B 1.461 -> 1.429 ms against four; one and eight 12-14 % slower)
          constexpr int KB = 2;
          constexpr int NSB = NQC / KB;            // S batches
          constexpr int NPAIR = NKS * 4;           // exponentiated pairs per lane
          static_assert(NKB == 1 && NQC % KB == 0 && (NKS * NDB) % KB == 0, "head dim 512 tile shape");
          auto kread = [&](int c) -> u32x4 {
            const int ch = 2 * (c + dh * NQC) + hl;
            return *reinterpret_cast<const u32x4*>(&bk[j * D + 8 * (ch ^ swz_k<D>(j))]);
          };
          static_assert(NSB >= 2, "the exponentiation needs a batch after the first");
          static_assert(NBUF == 2 && SEGW % 2 == 0 && NSB >= 2, "copies per batch");
          auto copies = [&](int bi, bool is_v, int nb_batches) __attribute__((always_inline)) {
            if constexpr (kCopyBatched) {
              const int per = SEGW / nb_batches;
              const int tc = t_start + min(it + (is_v ? 1 : 2), n_tiles - 1) * BN;
#pragma unroll
              for (int x = 0; x < per; ++x)
                prefill_seg(tc, n_keys, is_v ? vseq : kseq, is_v, is_v ? vbuf(u ^ 1) : kbuf(u),
                            wave * SEGW + bi * per + x);
            }
          };
          u32x4 kf[2][KB];
          constexpr int NPV = NKS * NDB;
          auto vread = [&](int m, u32x4& out) {
            const int ks = m / NDB, db = m % NDB;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const u32x2 t = read_tr16(&bv[v_elem(ks, half, db)]);
              out[2 * half] = t[0];
              out[2 * half + 1] = t[1];
            }
          };
          u32x4 vf[2][KB];
#pragma unroll
          for (int x = 0; x < KB; ++x) kf[0][x] = kread(x);
          sn[0] = f32x16{};
          u32x4 pf[NKS];
          float ls = 0.f;
#pragma unroll
          for (int bi = 0; bi < NSB; ++bi) {
            __builtin_amdgcn_sched_barrier(0);
            if (bi + 1 < NSB) {
#pragma unroll
              for (int x = 0; x < KB; ++x) kf[(bi + 1) & 1][x] = kread((bi + 1) * KB + x);
            } else {
              // the first PV batch's V^T reads beside the last score batch
              // (V(t) landed before this step's barrier)
#pragma unroll
              for (int x = 0; x < KB; ++x) vread(x, vf[0][x]);
            }
#pragma unroll
            for (int x = 0; x < KB; ++x) sn[0] = mfma32(as_bf16x8(kf[bi & 1][x]), qf[bi * KB + x], sn[0]);
            if (bi < 2) {
              copies(bi, false, 2);
              copies(bi, true, 2);
            }
            if (bi == 0) {
              __builtin_amdgcn_sched_barrier(0);
              // the partner's half of tile t's scores (same order in both
              // waves, so the pair holds bit-identical sums), then the mask and
              // the running max
#pragma unroll
              for (int x = 0; x < 16; ++x) sc[0][x] = dh == 0 ? sc[0][x] + oth[x] : oth[x] + sc[0][x];
              nb = prepare(sc, tb);
              continue;
            }
            // pairs q with q (NSB - 1) / NPAIR == bi - 1: an even share per
            // batch after the first
#pragma unroll
            for (int q = 0; q < NPAIR; ++q) {
              if (q * (NSB - 1) / NPAIR != bi - 1) continue;
              const int ks = q / 4, w = q % 4, base = 8 * (ks & 1);
              const float e0 = fast_exp2(fmaf(sc[ks >> 1][base + 2 * w], sl2, nb));
              const float e1 = fast_exp2(fmaf(sc[ks >> 1][base + 2 * w + 1], sl2, nb));
              ls += e0 + e1;
              pf[ks][w] = pack_bf16(e0, e1);
            }
          }
          l_run += ls;
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (KX) {
            score_extra(bk, sn[0]);
            // one exchange slot: every wave has read the partner's scores of
            // tile t (at the top of this step) before any overwrites its slot
            lds_barrier();
          }
          publish(sn, (it + 1) & 1);
          // O^T += V^T P^T in batches of KB MFMAs, two transposing reads each
          // (the first batch's reads went out with the last score batch)
#pragma unroll
          for (int bi = 0; bi < NPV / KB; ++bi) {
            __builtin_amdgcn_sched_barrier(0);
            if (bi + 1 < NPV / KB) {
#pragma unroll
              for (int x = 0; x < KB; ++x) vread((bi + 1) * KB + x, vf[(bi + 1) & 1][x]);
            }
#pragma unroll
            for (int x = 0; x < KB; ++x) {
              const int m = bi * KB + x, ks = m / NDB, db = m % NDB;
              oacc[db] = mfma32(as_bf16x8(vf[bi & 1][x]), as_bf16x8(pf[ks]), oacc[db]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
          scores_pre(kbuf((u + 1) % NBUF), sn, kpre);    // tile t+1 (unused after the last tile)
          if constexpr (kCopyInBlock) {
            static_assert(NBUF == 2, "copies into the buffers the step frees");
#pragma unroll
            for (int x = 0; x < SEGW; ++x) {
              prefill_seg(t_start + min(it + 2, n_tiles - 1) * BN, n_keys, kseq, false, kbuf(u), wave * SEGW + x);
              prefill_seg(t_start + min(it + 1, n_tiles - 1) * BN, n_keys, vseq, true, vbuf(u ^ 1), wave * SEGW + x);
            }
          }
          u32x4 pf[NKS];
          exponentiate(sc, nb, pf);
          publish(sn, (it + 1) & 1);
          accumulate(vbuf(u), pf);
          // one schedule for the whole step: S(t+1) MFMAs each followed by the
          // next K read and a share of tile t's exponentiation, then the PV
          // MFMAs each followed by the next two V^T reads; reads run NPRE
          // ahead of their MFMAs
          {
            // the operand reads as one stream over both phases (the PV
            // phase's first reads beside the last score MFMAs)
            // (the first NPRE reads went out before the softmax bookkeeping)
            sched_cont<NKB * NQC, 1, NDB * NKS, 2, NPRE, kExpValuPerTile / (NKB * NQC), -1, -1, 0>();
          }
        }
        if constexpr (kPrioMfma) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sc[kb] = sn[kb];
      };
      for (int it = 0; it < n_tiles; it += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          if (it + u >= n_tiles) break;
          step(it + u, u);
        }
      }
      if constexpr (kCopyBatched || kCopyInBlock) wait_vm<0>();   // the repeated copies after the last tile
      if constexpr (PERS) {
        static_assert(kCopyBatched || kCopyInBlock, "the loop leaves no copy in flight");
        // the next block: its Q fragments (qf is free once the last scores
        // are done) and, once every wave is past the last tiles, its first
        // tiles, all in flight while this block's O goes out
        L_next = pers_item(round + 1);
        pre = false;
        if (L_next >= 0) {
          const int bg2 = L_next / a.n_rb, rb2 = a.n_rb - 1 - (L_next % a.n_rb);
          const int bq2 = bg2 / a.Hkv, g2 = bg2 % a.Hkv;
          int ts2 = 0, nt2 = 0;
          block_tiles(rb2, ts2, nt2);
          load_q(bq2, g2, rb2);
          lds_barrier();
          const uint16_t* k2;
          const uint16_t* v2;
          kv_bases(bq2, g2, k2, v2);
          if (nt2 > 0) issue_first(ts2, nt2, k2, v2, bq2);
          pre = true;
        }
      }

    }

    // ---- epilogue ------------------------------------------------------------
    // O leaves through LDS up to D = 256 (below); at D = 512 one workgroup
    // holds the CU with one wave per SIMD, nothing hides the staging's two
    // barriers (measured 7 % slower), and a lane's fragments go straight out.
    constexpr bool kStageO = D <= 256;
    const float l_tot = pair_sum(l_run);
    if constexpr (!kStageO && !PERS) {
      if (!row_ok) return;
    }
    const bool empty = !(l_tot > 0.f);
    float inv = empty ? 0.f : fast_rcp(l_tot);
    float lse_v = empty ? -INFINITY : (m_run * sl2 + fast_log2(l_tot)) * kLn2;
    if (a.sinks != nullptr) {
      // the head's sink logit joins the denominator: LSE' = logaddexp(LSE,
      // sink), O' = O exp(LSE - LSE')
      const float sk = a.sinks[qh];
      const float mx = fmaxf(lse_v, sk);
      if (mx != -INFINITY) {
        const float el = empty ? 0.f : fast_exp2((lse_v - mx) * kLog2e);
        const float tot = el + fast_exp2((sk - mx) * kLog2e);
        inv *= el / tot;
        lse_v = mx + fast_log2(tot) * kLn2;
      }
    }
    if constexpr (!kStageO) {
      uint16_t* dst = a.o + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)qh * a.o_sh;
      if (row_ok)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * (db + dh * NDB) + 8 * rr + 4 * hl;
          u32x2 val = {pack_bf16(oacc[db][4 * rr + 0] * inv, oacc[db][4 * rr + 1] * inv),
                       pack_bf16(oacc[db][4 * rr + 2] * inv, oacc[db][4 * rr + 3] * inv)};
          if (!kPad || d0 < a.dv) *reinterpret_cast<u32x2*>(dst + d0) = val;
        }
    } else {
      // A lane holds 4 consecutive d of one row per fragment, so direct stores
      // would put 8 bytes in each of 32 rows per instruction (measured: the O
      // stores then cost 3 % of the head-dim-128 prefill and 12 % of the
      // head-dim-256 windowed one). The normalised bf16 rows are staged
      // row-major in the tile buffers (free once every wave is past its last
      // tile; 16-byte chunks XOR-swizzled by the row) and written back 16 bytes
      // per lane, a row's chunks in consecutive lanes.
      constexpr int CH = D / 8;                 // 16-byte chunks per row
      static_assert(BM <= 4 * BN && NBUF >= 2, "the staged block fits four tile buffers");
      auto stage = [&](int row) -> uint16_t* {
        if constexpr (PERS) return sO + row * D;
        const int r = row % BN;
        uint16_t* base = row < BN ? sK0 : row < 2 * BN ? sK1 : row < 3 * BN ? sV0 : sV1;
        return base + r * D;
      };
      lds_barrier();                            // every wave is done reading the last tiles
      {
        const int srow = 32 * rg + j;
        uint16_t* sp = stage(srow);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int c = 4 * (db + dh * NDB) + rr;   // chunk of d = 32 (db + dh NDB) + 8 rr
            u32x2 val = {pack_bf16(oacc[db][4 * rr + 0] * inv, oacc[db][4 * rr + 1] * inv),
                         pack_bf16(oacc[db][4 * rr + 2] * inv, oacc[db][4 * rr + 3] * inv)};
            *reinterpret_cast<u32x2*>(sp + 8 * (c ^ (srow & (CH - 1))) + 4 * hl) = val;
          }
      }
      lds_barrier();
      constexpr int PER = NW * 64;              // chunks per pass of the workgroup
      static_assert((BM * CH) % PER == 0, "whole passes");
#pragma unroll
      for (int idx = tid; idx < BM * CH; idx += PER) {
        const int row = idx / CH, c = idx % CH;
        const int r = r_lo + row;
        if (r < r_hi && (!kPad || 8 * c < a.dv)) {
          const int qi_r = r / a.G, qh_r = g * a.G + r % a.G;
          const u32x4 v = *reinterpret_cast<const u32x4*>(stage(row) + 8 * (c ^ (row & (CH - 1))));
          *reinterpret_cast<u32x4*>(a.o + (int64_t)b * a.o_sb + (int64_t)qi_r * a.o_ss + (int64_t)qh_r * a.o_sh +
                                    8 * c) = v;
        }
      }
      if constexpr (!PERS) {
        if (!row_ok) return;
      }
    }
    if (a.lse != nullptr && hl == 0 && dh == 0 && row_ok) a.lse[((int64_t)b * a.Hq + qh) * a.Sq + qi] = lse_v;
    if constexpr (!PERS) break;
    L = L_next;
    }  // rounds of the persistent grid
  }
}

}  // namespace gqafa
