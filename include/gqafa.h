/*
 * gqafa.h - C ABI of the MI355X (gfx950) GQA flash-attention library.
 *
 * The library computes scaled-dot-product attention, softmax(Q K^T * scale +
 * mask) V, with a streaming (online) softmax over K/V tiles, for grouped-query
 * heads, causal and sliding-window masks and head dims 64, 128, 256 and 512.
 * The computation is the "scalar flash-attention path" of llama.cpp PR 28507
 * (Vulkan K/V shared-memory staging on AMD RDNA, section Summary), whose SWA
 * layers use head size 256 and global layers 512 (section Measurements); the
 * split-KV partials publish a per-row (max, rowsum) pair that a combine step
 * merges (beellama.cpp PR 149, Make KVarN usable on ROCm RDNA3, section
 * Overview and the first review).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer, 16-byte aligned, owned by the
 *     caller. The library never allocates, frees or synchronizes. Its only
 *     process state is a per-(kernel, device) count of the workgroups a
 *     device holds at once (the grid size of the split-KV kernels and of the
 *     persistent head-dim-256 prefill), computed on a kernel's first call on
 *     a device from the runtime's occupancy query; it is a pure function of
 *     the kernel and the device, so no result depends on call history.
 *   - bf16 tensors are passed as raw 16-bit storage (bfloat16 bit patterns).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream). Results are ready when the stream reaches the call.
 *   - Arguments are validated on the host before anything is launched. An
 *     invalid call returns a negative status and launches nothing. The
 *     library never aborts and never prints.
 *   - Query head h reads KV head h / (Hq / Hkv) (consecutive query heads
 *     share a KV head).
 *   - Causal masking is bottom-right aligned: query row i of a sequence with
 *     n keys sits at position i + n - Sq and sees keys j <= that position.
 *     With window > 0 it only sees keys with position - j < window (exactly
 *     `window` keys ending at the diagonal). window > 0 requires causal.
 *   - LSE is the natural log of sum_j exp(scale * q . k_j) over the visible
 *     keys, in fp32. A row with no visible key gets O = 0 and LSE = -inf.
 *   - Arithmetic: bf16 inputs, fp32 accumulation of Q K^T and P V, fp32
 *     softmax state, P rounded to bf16 as the second product's operand.
 */
#ifndef GQAFA_H
#define GQAFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, bad mask or scale, misaligned pointer */
  FA_ERR_UNSUPPORTED = -2,  /* head dims not multiples of 8 in [8, 512] (nor 576/512), page size not a power of two */
  FA_ERR_WORKSPACE = -3,    /* decode workspace missing or smaller than fa_decode_workspace_bytes */
  FA_ERR_LAUNCH = -4,       /* the HIP runtime rejected a kernel launch */
  FA_ERR_SCRATCH = -5       /* fa_decode_paged_noalloc: the call needs more than FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/*
 * Score modifiers (the FLASH_ATTN_EXT case parameters logit_softcap,
 * max_bias and sinks of the llama.cpp PR 28507 test report name them; the
 * formulas are the readings stated here). With s = scale * q . k_j for the
 * query row at position p of query head h and key j:
 *   logit_softcap c > 0: s -> c * tanh(s / c)   (0: off)
 *   max_bias > 0 (ALiBi): s -> s + slope_h * (j - p), with n =
 *     2^floor(log2 Hq), slope_h = 2^(-max_bias (h + 1) / n) for h < n and
 *     2^(-max_bias (2 (h - n) + 1) / (2 n)) otherwise   (0: off)
 *   sinks: device fp32 [Hq]; sink_h joins the softmax denominator with no
 *     value: l = sum_j exp(s_j) + exp(sink_h), LSE = ln l; a row with no
 *     visible key gets O = 0 and LSE = sink_h   (NULL: off)
 *   mask: device bf16, additive, shared by every head: the score of key j
 *     for query row i of sequence b gains mask[b * mask_batch_stride +
 *     i * mask_row_stride + j] (elements; batch stride 0 shares one mask
 *     among the sequences). j is the key's token index: 0 .. Skv-1 in
 *     prefill, 0 .. seq_lens[b]-1 in decode/verify; every such entry must
 *     exist. Values finite or -inf (-inf hides the key). 8-byte aligned,
 *     strides >= 0, multiples of 4 and below 2^40   (NULL: off)
 * The softcap applies first, then the ALiBi term, then the mask; causal,
 * window and length masking come last. softcap and max_bias must be finite
 * and >= 0; sinks 4-byte aligned. Invalid fields: FA_ERR_INVALID_ARG.
 */
typedef struct fa_score_mods {
  float logit_softcap;
  float max_bias;
  const float* sinks;
  const void* mask;
  int64_t mask_batch_stride;
  int64_t mask_row_stride;
} fa_score_mods;

/*
 * Prefill attention (many query rows per sequence).
 *
 *   q   bf16 [B, Sq, Hq, D]   contiguous
 *   k   bf16 [B, Skv, Hkv, D] contiguous
 *   v   bf16 [B, Skv, Hkv, D] contiguous
 *   o   bf16 [B, Sq, Hq, D]   output (round-to-nearest-even)
 *   lse fp32 [B, Hq, Sq]      output, may be NULL (not written)
 *
 * B, Sq, Skv >= 0 (an empty batch or Sq = 0 writes nothing; Skv = 0 gives
 * O = 0 and LSE = -inf); Hq, Hkv > 0 with Hq % Hkv == 0; D a multiple of 8
 * in [8, 512] (FA_ERR_UNSUPPORTED otherwise); causal 0/1; window >= 0;
 * scale finite and > 0. A head dim runs on the smallest tile of 64, 128,
 * 256 or 512 columns that holds it; the columns past it are zeros in the
 * tiles and never stored.
 */
int fa_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Sq, int Skv, int D,
               int causal, int window, float scale, void* stream);

/*
 * fa_prefill on strided views, so that callers need not copy slices (for
 * example q, k and v cut from one fused QKV projection) into contiguous
 * tensors first. Inputs are read and the output written by stride (ATOM
 * PR 2938, Summary: the kernel reads by token and block strides and only the
 * innermost dimension must be unit-stride).
 *
 *   q_stride, k_stride, v_stride, o_stride: host arrays of three int64
 *   element strides (batch, token, head) of the [B, S, H, D] tensors; the
 *   head dim D is unit-stride. NULL means the contiguous layout. Each stride
 *   is a non-negative multiple of 8 below 2^40 (every row 16-byte aligned);
 *   the token strides of k and v are below 2^24. o must not overlap itself
 *   or the inputs. Returns FA_ERR_INVALID_ARG otherwise; the rest is as
 *   fa_prefill, and the results are bitwise those of fa_prefill on
 *   contiguous copies of the same values.
 *   mods: host pointer to score modifiers (see fa_score_mods), NULL = none.
 *   Dk, Dv: the key and value head dims, which may differ (each a multiple
 *   of 8 in [8, 512], or the pair Dk = 576, Dv = 512): q and k are [.., Dk],
 *   v and o [.., Dv]; the tile is the smallest of 64, 128, 256, 512 that
 *   holds both (512 for 576/512: the 64 key columns past 512 are a small
 *   tile of their own, taken in extra steps of the score contraction; the
 *   FLASH_ATTN_EXT case grid of the llama.cpp PR 28507 report lists the
 *   576/512 pair). FA_ERR_UNSUPPORTED otherwise. fa_prefill is Dk = Dv = D.
 */
int fa_prefill_strided(const void* q, const int64_t* q_stride, const void* k, const int64_t* k_stride,
                       const void* v, const int64_t* v_stride, void* o, const int64_t* o_stride,
                       float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int Dk, int Dv,
                       int causal, int window, float scale, const fa_score_mods* mods, void* stream);

/*
 * Bytes of device workspace fa_decode_paged needs: fp32 partial outputs
 * [B, Hq, Sq, n_slots, W] and their LSEs [B, Hq, Sq, n_slots], with W the
 * tile width for head dim D (the smallest of 64, 128, 256, 512 that holds
 * it, 512 for D = 576; with Dk != Dv pass the larger of the two), and
 * n_slots = ceil(max_seq_len / kv_chunk) + 1 (a sequence's keys meet at most
 * that many workgroup ranges of the balanced split), each region 256-byte
 * aligned. Returns 0 for invalid sizes.
 */
size_t fa_decode_workspace_bytes(int B, int Sq, int Hq, int D, int max_seq_len, int kv_chunk);

/*
 * Decode (Sq = 1) and speculative verify (a few query rows, causal among
 * them) over a paged KV cache, split over the KV sequence in chunks of
 * kv_chunk tokens and merged by LSE (split-KV, "parallel blocks" + combine:
 * beellama.cpp PR 149, Overview). The split kernel is a persistent grid that
 * gives every workgroup an equal, contiguous range of all K/V tiles (at least
 * one chunk; tiles never straddle a chunk); a range merges its chunks in its
 * online softmax and leaves one partial per block of rows it touches.
 *
 *   q           bf16 [B, Sq, Hq, D]: the Sq newest rows of each sequence
 *   kcache      bf16 [num_pages, page_size, Hkv, D] when block_table != NULL;
 *   vcache           bf16 [B, max_pages_per_seq * page_size, Hkv, D] (a
 *                    contiguous cache, i.e. the identity table) when NULL
 *   block_table int32 [B, max_pages_per_seq]: token t of sequence b is in
 *               physical page block_table[b][t / page_size], slot
 *               t % page_size. May be NULL (contiguous cache).
 *   seq_lens    int32 [B] on the device: tokens in each sequence's cache,
 *               including the Sq query rows' own keys; values are clamped to
 *               [0, max_pages_per_seq * page_size].
 *   o           bf16 [B, Sq, Hq, D] output
 *   lse         fp32 [B, Hq, Sq] output, may be NULL
 *   num_pages   physical pages in the cache; ignored when block_table is
 *               NULL. A block_table entry outside [0, num_pages) that covers
 *               tokens below seq_lens[b] is a caller error that is not
 *               detected: the entry is clamped into range, so every load
 *               stays inside the cache, and that sequence's output is
 *               unspecified. Entries past a sequence's last page are never
 *               used.
 *   page_size   a power of two in [1, 65536]
 *   kv_chunk    tokens per chunk, a positive multiple of 32 (the split's
 *               32-key tiles never straddle a chunk); FA_ERR_INVALID_ARG
 *               otherwise
 *   workspace   device buffer of at least
 *               fa_decode_workspace_bytes(B, Sq, Hq, D, max_pages_per_seq*page_size, kv_chunk)
 *
 * Two kernels run on `stream`: the split kernel writes partials into the
 * workspace, then the combine kernel writes o and lse. Calls that share a
 * workspace must be ordered on one stream. Results are deterministic: the
 * work split depends only on the shapes, seq_lens and the GPU's size.
 * Returns FA_ERR_INVALID_ARG when the K/V tile count of one call does not
 * fit 32 bits (B * Hkv * ceil(Sq * Hq / Hkv / 32) * (ceil(max_len / 32) +
 * ceil(max_len / kv_chunk)) > 2^31 - 1, max_len = max_pages_per_seq *
 * page_size).
 */
int fa_decode_paged(const void* q, const void* kcache, const void* vcache,
                    const int32_t* block_table, const int32_t* seq_lens,
                    void* o, float* lse,
                    int B, int Sq, int Hq, int Hkv, int D,
                    int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                    int causal, int window, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_paged on strided views (ATOM PR 2938, Summary: read by stride,
 * only the innermost dimension unit-stride). q_stride and o_stride are the
 * (batch, row, head) element strides of q and o; k_stride and v_stride the
 * (page, slot, head) strides of a paged cache, or (sequence, token, head) of
 * a contiguous one, so K and V may for example be interleaved in one
 * allocation. Each is a host array of three int64, NULL for the contiguous
 * layout, with the rules of fa_prefill_strided. The results are bitwise
 * those of fa_decode_paged on contiguous copies of the same values. mods:
 * host pointer to score modifiers (see fa_score_mods), NULL = none. Dk and
 * Dv are the key and value head dims as in fa_prefill_strided: q and kcache
 * are [.., Dk], vcache and o [.., Dv]; the workspace is sized with
 * max(Dk, Dv).
 */
int fa_decode_paged_strided(const void* q, const int64_t* q_stride,
                            const void* kcache, const int64_t* k_stride,
                            const void* vcache, const int64_t* v_stride,
                            const int32_t* block_table, const int32_t* seq_lens,
                            void* o, const int64_t* o_stride, float* lse,
                            int B, int Sq, int Hq, int Hkv, int Dk, int Dv,
                            int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                            int causal, int window, float scale, const fa_score_mods* mods,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode / verify over an fp8 KV cache: fa_decode_paged_strided with K and V
 * stored one byte per element in the OCP e4m3 format (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; no infinities; largest finite 448) and
 * one fp32 dequantisation scale per KV head: the cached value of an element
 * of KV head g is e4m3(byte) * k_scale[g] (v_scale[g] for V). Halving the
 * bytes of the cache halves the HBM traffic of the memory-bound split
 * kernel. (The pages name low-bit KV caches, q8_0 in the llama.cpp PR 28507
 * report and KVarN in beellama.cpp PR 149, without fixing a format; e4m3
 * with a per-head scale is the format gfx950 converts natively.)
 *
 *   kcache, vcache  uint8 [num_pages, page_size, Hkv, D] with block_table,
 *                   else [B, max_pages_per_seq * page_size, Hkv, D]
 *   k_stride, v_stride  host int64[3] strides in elements (= bytes), NULL
 *                   for the contiguous layout; multiples of 16 below 2^40,
 *                   token strides below 2^24
 *   k_scale, v_scale    device fp32 [Hkv], 4-byte aligned
 *   D               128, 256 or 512 (FA_ERR_UNSUPPORTED otherwise): the head
 *                   sizes of the pages' quantised-cache layers (llama.cpp
 *                   PR 28507, Measurements: q8_0 caches on head-256 SWA and
 *                   head-512 global layers)
 * Everything else (q and o bf16, seq_lens, block table, workspace, score
 * modifiers, outputs) is as fa_decode_paged_strided with Dk = Dv = D. The
 * arithmetic is that of the bf16 cache path on the dequantised values: the
 * K scale multiplies the exponent factor, the V scale the normalisation.
 */
int fa_decode_paged_fp8(const void* q, const int64_t* q_stride,
                        const void* kcache, const int64_t* k_stride,
                        const void* vcache, const int64_t* v_stride,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        void* o, const int64_t* o_stride, float* lse,
                        int B, int Sq, int Hq, int Hkv, int D,
                        int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                        int causal, int window, float scale, const fa_score_mods* mods,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Merge split-KV partials by their LSE (the combine step that runs after the
 * split blocks on the same stream when a KV range is cut into parallel
 * blocks: beellama.cpp PR 149, first review; every partial publishes its
 * row max and sum as an LSE, same page, Overview):
 *   M = max_c LSE_c,  LSE = M + ln sum_c exp(LSE_c - M),
 *   O = sum_c exp(LSE_c - LSE) * O_c.
 * Chunks with LSE_c = -inf have weight 0; a row whose chunks are all empty
 * gets O = 0, LSE = -inf.
 *
 *   D        64, 128, 256 or 512 (the partial width of the split path)
 *   o_part   fp32 [B, Hq, Sq, max_chunks, D] (each normalised by its own sum)
 *   lse_part fp32 [B, Hq, Sq, max_chunks]
 *   n_chunks int32 [B] on the device: leading chunks of sequence b to merge
 *            (clamped to [0, max_chunks]); NULL merges all max_chunks
 *   o        bf16 [B, Sq, Hq, D] output
 *   lse      fp32 [B, Hq, Sq] output, may be NULL
 */
int fa_combine_lse(const float* o_part, const float* lse_part, const int32_t* n_chunks,
                   int max_chunks, void* o, float* lse,
                   int B, int Sq, int Hq, int D, void* stream);

/*
 * KV-cache append: the step before a decode or verify call, which writes the
 * Snew newest K/V rows of each sequence into the cache.
 *
 *   kcache, vcache  bf16 [num_pages, page_size, Hkv, Dk or Dv] with block_table
 *                   (int32 [B, max_pages_per_seq]), or contiguous
 *                   [B, max_pages_per_seq * page_size, Hkv, D] when
 *                   block_table is NULL; written in place
 *   seq_lens        int32 [B] on the device: tokens in each cache AFTER the
 *                   append (the convention of fa_decode_paged); clamped to
 *                   [0, max_pages_per_seq * page_size]
 *   knew, vnew      bf16 [B, Snew, Hkv, Dk] and [B, Snew, Hkv, Dv]: row i of
 *                   sequence b goes to token seq_lens[b] - Snew + i; the
 *                   caches have the same head dims (multiples of 8 in
 *                   [8, 512])
 *   *_stride        host int64[3] element strides (outer, token, head) of the
 *                   four tensors, NULL for the contiguous layout, with the
 *                   rules of fa_prefill_strided (head dim unit-stride)
 *
 * Rows whose token would be negative (a sequence shorter than Snew) and rows
 * whose block-table entry is outside [0, num_pages) are not written. Two new
 * rows mapped to the same physical slot race (a caller error). The copy is
 * bit-exact.
 */
int fa_kv_append(void* kcache, const int64_t* k_stride, void* vcache, const int64_t* v_stride,
                 const int32_t* block_table, const int32_t* seq_lens,
                 const void* knew, const int64_t* knew_stride, const void* vnew, const int64_t* vnew_stride,
                 int B, int Snew, int Hkv, int Dk, int Dv, int num_pages, int page_size,
                 int max_pages_per_seq, void* stream);

/*
 * fa_kv_append into an fp8 cache (see fa_decode_paged_fp8): each new bf16
 * value v of KV head g is stored as the e4m3 code nearest to the fp32
 * quotient v / scale[g] (one IEEE fp32 division, rounded to nearest even),
 * ties to the even code, saturating at +-448 (NaN -> 0x7f; the sign of the
 * quotient is kept, so -0 and negatives that round to 0 give 0x80).
 *
 *   kcache, vcache  uint8 caches as in fa_decode_paged_fp8, written in place;
 *                   strides multiples of 16 (bytes)
 *   k_scale, v_scale    device fp32 [Hkv] (the dequantisation scales)
 *   knew, vnew      bf16 [B, Snew, Hkv, D], strides as fa_kv_append
 *   D               a multiple of 16 in [16, 512]
 * Placement, skipped rows and races are as in fa_kv_append.
 */
int fa_kv_append_fp8(void* kcache, const int64_t* k_stride, void* vcache, const int64_t* v_stride,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_table, const int32_t* seq_lens,
                     const void* knew, const int64_t* knew_stride, const void* vnew, const int64_t* vnew_stride,
                     int B, int Snew, int Hkv, int D, int num_pages, int page_size, int max_pages_per_seq,
                     void* stream);

/*
 * fa_decode_paged_strided for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, with the split partials written to a static
 * device array of FA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends, instead of a caller workspace.
 * Every argument is as fa_decode_paged_strided without the workspace; the
 * results are bitwise those of fa_decode_paged_strided.
 *
 *   - A call whose fa_decode_workspace_bytes(B, Sq, Hq, max(Dk, Dv),
 *     max_pages_per_seq * page_size, kv_chunk) exceeds
 *     FA_NOALLOC_SCRATCH_BYTES returns FA_ERR_SCRATCH and launches nothing.
 *   - Nothing here allocates: the array's address on a device is looked up
 *     (hipGetSymbolAddress) on the first call for that device and kept.
 *   - The array is shared by every call on its GPU and keeps the last call's
 *     partials; a call writes every slot it reads before reading it, so
 *     nothing needs clearing. Calls that overlap on one GPU (on different
 *     streams, or from different threads, without ordering) race on the
 *     array: order them on one stream.
 *   - The array used is that of the stream's device (the current device for
 *     the NULL stream).
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)
int fa_decode_paged_noalloc(const void* q, const int64_t* q_stride,
                            const void* kcache, const int64_t* k_stride,
                            const void* vcache, const int64_t* v_stride,
                            const int32_t* block_table, const int32_t* seq_lens,
                            void* o, const int64_t* o_stride, float* lse,
                            int B, int Sq, int Hq, int Hkv, int Dk, int Dv,
                            int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                            int causal, int window, float scale, const fa_score_mods* mods,
                            void* stream);

/* Static text for a status code (never NULL). */
const char* fa_status_string(int status);

/*
 * Test hook: gathers a paged cache into a dense tensor through the split-KV
 * kernel's own page address rule (clamp_page and paged_row in the library's
 * device header: a table entry is clamped into [0, num_pages), then token t
 * is slot t % page_size of that page), so that a byte-exact comparison with
 * a CPU gather pins the decode path's address arithmetic (vLLM PR 32,
 * Validation: the paged indexer's picks are checked for identity against a
 * reference).
 *   cache [num_pages, page_size, Hkv, D] bf16 -> out [B, max_pages_per_seq*page_size, Hkv, D]
 *   seq_lens int32 [B] on the device, clamped to [0, max_pages_per_seq*page_size]
 * Slots at or beyond seq_lens[b] are written as zero; a slot whose table
 * entry is outside [0, num_pages) holds the row of the page the entry clamps
 * to, as the decode kernel reads it.
 */
int fa_paged_gather(const void* cache, const int32_t* block_table, const int32_t* seq_lens,
                    void* out, int B, int Hkv, int D, int num_pages, int page_size,
                    int max_pages_per_seq, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQAFA_H */
