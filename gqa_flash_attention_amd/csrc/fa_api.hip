// C ABI: host-side validation and dispatch. Nothing here allocates, frees,
// synchronizes, prints or aborts; an invalid call launches nothing.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/gqafa.h"
#include "fa_launch.h"

using namespace gqafa;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tile widths the kernels are built for; partials of the split path have one
// of these widths.
bool tile_dim_ok(int D) { return D == 64 || D == 128 || D == 256 || D == 512; }

// Head dims: multiples of 8 (16-byte rows) from 8 to 512.
bool head_dim_ok(int D) { return D >= 8 && D <= 512 && D % 8 == 0; }

// Key head dim 576 with value head dim 512: the 512 tile plus 64 extra key
// columns (the 576/512 pair of the llama.cpp PR 28507 report's case grid).
constexpr int kWideK = 576;
bool wide_pair(int dk, int dv) { return dk == kWideK && dv == 512; }

// (Dk, Dv) pairs the attention kernels run.
bool dims_ok(int dk, int dv) { return (head_dim_ok(dk) && head_dim_ok(dv)) || wide_pair(dk, dv); }

// The tile width that runs key / value head dims dk and dv: the smallest of
// 64, 128, 256, 512 that holds both (512 for the 576-wide keys).
int tile_dim(int dk, int dv) {
  const int m = dk > dv ? dk : dv;
  return m <= 64 ? 64 : (m <= 128 ? 128 : (m <= 256 ? 256 : 512));
}

int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t n_chunks_for(int64_t len, int chunk) { return (len + chunk - 1) / chunk; }

int to_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

// Upper bound on grid sizes and element counts (all kernels index in 64 bits;
// this keeps the 1-D grids below 2^31 workgroups).
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

// Element strides (outer, token, head) from a caller's host array, or the
// dense layout when it is NULL. Every stride is a non-negative multiple of 8
// elements (each row stays 16-byte aligned) below 2^40; a K/V token stride is
// below 2^24 (the kernels keep a tile's per-lane offsets in 32 bits).
// Score modifiers from the caller's struct (NULL: none).
struct Mods {
  float softcap = 0.f, max_bias = 0.f;
  const float* sinks = nullptr;
  const void* mask = nullptr;
  int64_t mask_sb = 0, mask_ss = 0;
};

bool get_mods(const fa_score_mods* m, Mods& out) {
  out = Mods{};
  if (m == nullptr) return true;
  if (!std::isfinite(m->logit_softcap) || m->logit_softcap < 0.f) return false;
  if (!std::isfinite(m->max_bias) || m->max_bias < 0.f) return false;
  if (m->sinks != nullptr && (reinterpret_cast<uintptr_t>(m->sinks) & 3u) != 0) return false;
  if (m->mask != nullptr) {
    // 8-byte vector reads of 4 keys: an 8-byte aligned base and strides in
    // whole groups of 4 elements
    if ((reinterpret_cast<uintptr_t>(m->mask) & 7u) != 0) return false;
    if (m->mask_batch_stride < 0 || m->mask_row_stride < 0) return false;
    if ((m->mask_batch_stride & 3) != 0 || (m->mask_row_stride & 3) != 0) return false;
    if (m->mask_batch_stride >= (int64_t(1) << 40) || m->mask_row_stride >= (int64_t(1) << 40)) return false;
  }
  out.softcap = m->logit_softcap;
  out.max_bias = m->max_bias;
  out.sinks = m->sinks;
  out.mask = m->mask;
  out.mask_sb = m->mask_batch_stride;
  out.mask_ss = m->mask_row_stride;
  return true;
}

bool get_strides(const int64_t* st, Strides dense, bool kv, Strides& out, int align = 8) {
  if (st == nullptr) {
    out = dense;
    return true;
  }
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % align != 0 || st[i] >= (int64_t(1) << 40)) return false;
  out = Strides{st[0], st[1], st[2]};
  return !(kv && out.token >= (int64_t(1) << 24));
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED:
      return "unsupported shape (head dims must be multiples of 8 up to 512, or 576 keys with 512 values; "
             "page size a power of two)";
    case FA_ERR_WORKSPACE: return "decode workspace missing or too small";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH:
      return "the call needs more device scratch than fa_decode_paged_noalloc's static buffer holds "
             "(FA_NOALLOC_SCRATCH_BYTES); use fa_decode_paged_strided with a caller workspace";
    default: return "unknown status";
  }
}

int fa_prefill_strided(const void* q, const int64_t* q_stride, const void* k, const int64_t* k_stride,
                       const void* v, const int64_t* v_stride, void* o, const int64_t* o_stride,
                       float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int Dk, int Dv,
                       int causal, int window, float scale, const fa_score_mods* mods, void* stream) {
  if (B < 0 || Sq < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  Mods md;
  if (!get_mods(mods, md)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (!dims_ok(Dk, Dv)) return FA_ERR_UNSUPPORTED;
  Strides qs, ks, vs, os;
  const Strides qd{(int64_t)Sq * Hq * Dk, (int64_t)Hq * Dk, Dk};
  const Strides od{(int64_t)Sq * Hq * Dv, (int64_t)Hq * Dv, Dv};
  const Strides kd{(int64_t)Skv * Hkv * Dk, (int64_t)Hkv * Dk, Dk};
  const Strides vd{(int64_t)Skv * Hkv * Dv, (int64_t)Hkv * Dv, Dv};
  if (!get_strides(q_stride, qd, false, qs) || !get_strides(o_stride, od, false, os) ||
      !get_strides(k_stride, kd, true, ks) || !get_strides(v_stride, vd, true, vs))
    return FA_ERR_INVALID_ARG;
  if (B == 0 || Sq == 0) return FA_OK;
  if (!q || !o || !aligned16(q) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (Skv > 0 && (!k || !v || !aligned16(k) || !aligned16(v))) return FA_ERR_INVALID_ARG;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)Sq * (Hq / Hkv);
  if ((int64_t)B * Hkv * ((rows + 127) / 32) > kMaxGrid) return FA_ERR_INVALID_ARG;
  PrefillDesc d{q, k, v, o, lse, qs, ks, vs, os, B, Hq, Hkv, Sq, Skv, tile_dim(Dk, Dv), causal, window,
                Dk, Dv, scale, md.softcap, md.max_bias, md.sinks, md.mask, md.mask_sb, md.mask_ss};
  return to_status(launch_prefill(d, static_cast<hipStream_t>(stream)));
}

int fa_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Sq, int Skv, int D,
               int causal, int window, float scale, void* stream) {
  return fa_prefill_strided(q, nullptr, k, nullptr, v, nullptr, o, nullptr, lse, B, Hq, Hkv, Sq, Skv, D, D,
                            causal, window, scale, nullptr, stream);
}

size_t fa_decode_workspace_bytes(int B, int Sq, int Hq, int D, int max_seq_len, int kv_chunk) {
  if (B < 0 || Sq < 0 || Hq <= 0 || !(head_dim_ok(D) || D == kWideK) || max_seq_len < 0 || kv_chunk <= 0 ||
      kv_chunk % 32 != 0)
    return 0;
  const int64_t slots = n_chunks_for(max_seq_len, kv_chunk) + 1;
  const int64_t rows = (int64_t)B * Hq * Sq;
  const int64_t width = tile_dim(D, D);     // partials are as wide as the tile
  const size_t o_bytes = align256((size_t)(rows * slots * width) * sizeof(float));
  const size_t l_bytes = align256((size_t)(rows * slots) * sizeof(float));
  return o_bytes + l_bytes;
}

}  // extern "C"

namespace {

// Decode / verify behind fa_decode_paged_strided (bf16 caches) and
// fa_decode_paged_fp8 (one-byte e4m3 caches with per-head scales, D = 128,
// 256 or 512).
int decode_impl(const void* q, const int64_t* q_stride,
                const void* kcache, const int64_t* k_stride,
                const void* vcache, const int64_t* v_stride,
                const float* k_scale, const float* v_scale, bool kv8,
                const int32_t* block_table, const int32_t* seq_lens,
                void* o, const int64_t* o_stride, float* lse,
                int B, int Sq, int Hq, int Hkv, int Dk, int Dv,
                int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                int causal, int window, float scale, const fa_score_mods* mods,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || Sq < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (kv8 && (Dk != Dv || (Dk != 128 && Dk != 256 && Dk != 512))) return FA_ERR_UNSUPPORTED;
  Mods md;
  if (!get_mods(mods, md)) return FA_ERR_INVALID_ARG;
  // chunks are whole 32-key tiles
  if (max_pages_per_seq < 0 || kv_chunk <= 0 || kv_chunk % 32 != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (!dims_ok(Dk, Dv)) return FA_ERR_UNSUPPORTED;
  const int D = tile_dim(Dk, Dv);
  const int page_shift = log2_exact(page_size);
  if (page_shift < 0 || page_shift > 16) return FA_ERR_UNSUPPORTED;
  const int64_t max_len = (int64_t)max_pages_per_seq << page_shift;
  if (max_len > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (block_table != nullptr && num_pages <= 0) return FA_ERR_INVALID_ARG;
  Strides qs, ks, vs, os;
  const Strides qd{(int64_t)Sq * Hq * Dk, (int64_t)Hq * Dk, Dk};
  const Strides od{(int64_t)Sq * Hq * Dv, (int64_t)Hq * Dv, Dv};
  auto cache_dense = [&](int64_t d) {
    return block_table != nullptr ? Strides{(int64_t)page_size * Hkv * d, (int64_t)Hkv * d, d}
                                  : Strides{max_len * Hkv * d, (int64_t)Hkv * d, d};
  };
  // fp8 cache rows are 16-byte aligned at 16 one-byte elements
  const int calign = kv8 ? 16 : 8;
  if (!get_strides(q_stride, qd, false, qs) || !get_strides(o_stride, od, false, os) ||
      !get_strides(k_stride, cache_dense(Dk), true, ks, calign) ||
      !get_strides(v_stride, cache_dense(Dv), true, vs, calign))
    return FA_ERR_INVALID_ARG;
  if (B == 0 || Sq == 0) return FA_OK;
  if (!q || !o || !seq_lens || !aligned16(q) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (max_len > 0 && (!kcache || !vcache || !aligned16(kcache) || !aligned16(vcache)))
    return FA_ERR_INVALID_ARG;
  if (kv8 && (!k_scale || !v_scale || (reinterpret_cast<uintptr_t>(k_scale) & 3u) != 0 ||
              (reinterpret_cast<uintptr_t>(v_scale) & 3u) != 0))
    return FA_ERR_INVALID_ARG;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_INVALID_ARG;
  const size_t need = fa_decode_workspace_bytes(B, Sq, Hq, D, (int)max_len, kv_chunk);   // D = the tile width
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return FA_ERR_WORKSPACE;
  const int64_t max_chunks = n_chunks_for(max_len, kv_chunk);
  const int64_t n_slots = max_chunks + 1;
  const int64_t rows = (int64_t)Sq * (Hq / Hkv);
  // the split kernel counts tiles (at most one per 32 keys plus one per
  // chunk, per block of 32 rows and KV head) in 32-bit integers
  if ((int64_t)B * Hkv * ((rows + 31) / 32) * ((max_len + 31) / 32 + max_chunks) > INT32_MAX)
    return FA_ERR_INVALID_ARG;
  if ((int64_t)B * Hq * Sq > kMaxGrid) return FA_ERR_INVALID_ARG;   // one combine workgroup per row

  const int64_t prow = (int64_t)B * Hq * Sq;
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align256((size_t)(prow * n_slots * D) * sizeof(float)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (max_chunks > 0) {
    SplitDesc sd{q, kcache, vcache, block_table, seq_lens, o_part, lse_part, qs, ks, vs,
                 B, Sq, Hq, Hkv, D, num_pages, page_shift, max_pages_per_seq, kv_chunk,
                 (int)n_slots, causal, window, Dk, Dv, scale, md.softcap, md.max_bias, md.mask, md.mask_sb,
                 md.mask_ss, kv8, k_scale, v_scale};
    const int s = to_status(launch_split(sd, st));
    if (s != FA_OK) return s;
  }
  CombineDesc cd{o_part, lse_part, nullptr, seq_lens, (int)max_len, kv_chunk, (int)n_slots, o, lse, os, md.sinks,
                 B, Sq, Hq, D, Dv};
  return to_status(launch_combine(cd, st));
}

}  // namespace

extern "C" {

int fa_decode_paged_strided(const void* q, const int64_t* q_stride,
                            const void* kcache, const int64_t* k_stride,
                            const void* vcache, const int64_t* v_stride,
                            const int32_t* block_table, const int32_t* seq_lens,
                            void* o, const int64_t* o_stride, float* lse,
                            int B, int Sq, int Hq, int Hkv, int Dk, int Dv,
                            int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                            int causal, int window, float scale, const fa_score_mods* mods,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, q_stride, kcache, k_stride, vcache, v_stride, nullptr, nullptr, false, block_table,
                     seq_lens, o, o_stride, lse, B, Sq, Hq, Hkv, Dk, Dv, num_pages, page_size,
                     max_pages_per_seq, kv_chunk, causal, window, scale, mods, workspace, workspace_bytes,
                     stream);
}

int fa_decode_paged_fp8(const void* q, const int64_t* q_stride,
                        const void* kcache, const int64_t* k_stride,
                        const void* vcache, const int64_t* v_stride,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        void* o, const int64_t* o_stride, float* lse,
                        int B, int Sq, int Hq, int Hkv, int D,
                        int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                        int causal, int window, float scale, const fa_score_mods* mods,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, q_stride, kcache, k_stride, vcache, v_stride, k_scale, v_scale, true, block_table,
                     seq_lens, o, o_stride, lse, B, Sq, Hq, Hkv, D, D, num_pages, page_size,
                     max_pages_per_seq, kv_chunk, causal, window, scale, mods, workspace, workspace_bytes,
                     stream);
}

int fa_decode_paged(const void* q, const void* kcache, const void* vcache,
                    const int32_t* block_table, const int32_t* seq_lens,
                    void* o, float* lse,
                    int B, int Sq, int Hq, int Hkv, int D,
                    int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                    int causal, int window, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return fa_decode_paged_strided(q, nullptr, kcache, nullptr, vcache, nullptr, block_table, seq_lens,
                                 o, nullptr, lse, B, Sq, Hq, Hkv, D, D, num_pages, page_size,
                                 max_pages_per_seq, kv_chunk, causal, window, scale, nullptr, workspace,
                                 workspace_bytes, stream);
}

int fa_combine_lse(const float* o_part, const float* lse_part, const int32_t* n_chunks,
                   int max_chunks, void* o, float* lse,
                   int B, int Sq, int Hq, int D, void* stream) {
  if (B < 0 || Sq < 0 || Hq <= 0 || max_chunks < 0) return FA_ERR_INVALID_ARG;
  if (!tile_dim_ok(D)) return FA_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) return FA_OK;
  if (!o || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (max_chunks > 0 && (!o_part || !lse_part || !aligned16(o_part))) return FA_ERR_INVALID_ARG;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * Hq * Sq > kMaxGrid) return FA_ERR_INVALID_ARG;
  const Strides od{(int64_t)Sq * Hq * D, (int64_t)Hq * D, D};
  CombineDesc cd{o_part, lse_part, n_chunks, nullptr, 0, 0, max_chunks, o, lse, od, nullptr, B, Sq, Hq, D, D};
  return to_status(launch_combine(cd, static_cast<hipStream_t>(stream)));
}

int fa_kv_append(void* kcache, const int64_t* k_stride, void* vcache, const int64_t* v_stride,
                 const int32_t* block_table, const int32_t* seq_lens,
                 const void* knew, const int64_t* knew_stride, const void* vnew, const int64_t* vnew_stride,
                 int B, int Snew, int Hkv, int Dk, int Dv, int num_pages, int page_size,
                 int max_pages_per_seq, void* stream) {
  if (B < 0 || Snew < 0 || Hkv <= 0 || max_pages_per_seq < 0) return FA_ERR_INVALID_ARG;
  if (!dims_ok(Dk, Dv)) return FA_ERR_UNSUPPORTED;
  const int page_shift = log2_exact(page_size);
  if (page_shift < 0 || page_shift > 16) return FA_ERR_UNSUPPORTED;
  const int64_t max_len = (int64_t)max_pages_per_seq << page_shift;
  if (max_len > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (block_table != nullptr && num_pages <= 0) return FA_ERR_INVALID_ARG;
  Strides kcs, vcs, kns, vns;
  auto cache_dense = [&](int64_t d) {
    return block_table != nullptr ? Strides{(int64_t)page_size * Hkv * d, (int64_t)Hkv * d, d}
                                  : Strides{max_len * Hkv * d, (int64_t)Hkv * d, d};
  };
  auto new_dense = [&](int64_t d) { return Strides{(int64_t)Snew * Hkv * d, (int64_t)Hkv * d, d}; };
  if (!get_strides(k_stride, cache_dense(Dk), false, kcs) || !get_strides(v_stride, cache_dense(Dv), false, vcs) ||
      !get_strides(knew_stride, new_dense(Dk), false, kns) || !get_strides(vnew_stride, new_dense(Dv), false, vns))
    return FA_ERR_INVALID_ARG;
  if (B == 0 || Snew == 0 || max_len == 0) return FA_OK;
  if (!kcache || !vcache || !knew || !vnew || !seq_lens) return FA_ERR_INVALID_ARG;
  if (!aligned16(kcache) || !aligned16(vcache) || !aligned16(knew) || !aligned16(vnew))
    return FA_ERR_INVALID_ARG;
  AppendDesc d{kcache, vcache, knew, vnew, block_table, seq_lens, kcs, vcs, kns, vns,
               B, Snew, Hkv, Dk, Dv, num_pages, page_shift, max_pages_per_seq};
  return to_status(launch_append(d, static_cast<hipStream_t>(stream)));
}

int fa_kv_append_fp8(void* kcache, const int64_t* k_stride, void* vcache, const int64_t* v_stride,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_table, const int32_t* seq_lens,
                     const void* knew, const int64_t* knew_stride, const void* vnew, const int64_t* vnew_stride,
                     int B, int Snew, int Hkv, int D, int num_pages, int page_size, int max_pages_per_seq,
                     void* stream) {
  if (B < 0 || Snew < 0 || Hkv <= 0 || max_pages_per_seq < 0) return FA_ERR_INVALID_ARG;
  if (!head_dim_ok(D) || D % 16 != 0) return FA_ERR_UNSUPPORTED;
  const int page_shift = log2_exact(page_size);
  if (page_shift < 0 || page_shift > 16) return FA_ERR_UNSUPPORTED;
  const int64_t max_len = (int64_t)max_pages_per_seq << page_shift;
  if (max_len > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (block_table != nullptr && num_pages <= 0) return FA_ERR_INVALID_ARG;
  Strides kcs, vcs, kns, vns;
  const Strides cd = block_table != nullptr ? Strides{(int64_t)page_size * Hkv * D, (int64_t)Hkv * D, D}
                                            : Strides{max_len * Hkv * D, (int64_t)Hkv * D, D};
  const Strides nd{(int64_t)Snew * Hkv * D, (int64_t)Hkv * D, D};
  if (!get_strides(k_stride, cd, false, kcs, 16) || !get_strides(v_stride, cd, false, vcs, 16) ||
      !get_strides(knew_stride, nd, false, kns) || !get_strides(vnew_stride, nd, false, vns))
    return FA_ERR_INVALID_ARG;
  if (B == 0 || Snew == 0 || max_len == 0) return FA_OK;
  if (!kcache || !vcache || !knew || !vnew || !seq_lens || !k_scale || !v_scale) return FA_ERR_INVALID_ARG;
  if (!aligned16(kcache) || !aligned16(vcache) || !aligned16(knew) || !aligned16(vnew) ||
      (reinterpret_cast<uintptr_t>(k_scale) & 3u) != 0 || (reinterpret_cast<uintptr_t>(v_scale) & 3u) != 0)
    return FA_ERR_INVALID_ARG;
  AppendFp8Desc d{kcache, vcache, knew, vnew, k_scale, v_scale, block_table, seq_lens, kcs, vcs, kns, vns,
                  B, Snew, Hkv, D, num_pages, page_shift, max_pages_per_seq};
  return to_status(launch_append_fp8(d, static_cast<hipStream_t>(stream)));
}

int fa_paged_gather(const void* cache, const int32_t* block_table, const int32_t* seq_lens,
                    void* out, int B, int Hkv, int D, int num_pages, int page_size,
                    int max_pages_per_seq, void* stream) {
  if (B < 0 || Hkv <= 0 || max_pages_per_seq < 0) return FA_ERR_INVALID_ARG;
  if (!head_dim_ok(D)) return FA_ERR_UNSUPPORTED;
  const int page_shift = log2_exact(page_size);
  if (page_shift < 0 || page_shift > 16) return FA_ERR_UNSUPPORTED;
  if (((int64_t)max_pages_per_seq << page_shift) > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (B == 0 || max_pages_per_seq == 0) return FA_OK;
  if (!cache || !block_table || !seq_lens || !out || num_pages <= 0) return FA_ERR_INVALID_ARG;
  if (!aligned16(cache) || !aligned16(out)) return FA_ERR_INVALID_ARG;
  GatherDesc d{cache, block_table, seq_lens, out, B, Hkv, D, num_pages, page_shift, max_pages_per_seq};
  return to_status(launch_gather(d, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode / verify without allocation: the split partials go to a static
// device array of FA_NOALLOC_SCRATCH_BYTES that each GPU holds for the life
// of the process, instead of a caller workspace.

namespace {

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on each device: the array's name is a host-side
// stand-in, so the address is looked up once per device (with that device
// current) and kept. Devices past the table are looked up on every call.
constexpr int kScratchDevs = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevs] = {};

int scratch_address(int dev, void** out) {
  if (dev >= 0 && dev < kScratchDevs) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] != nullptr) {
      *out = g_scratch_ptr[dev];
      return FA_OK;
    }
  }
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_LAUNCH;
  if (e != hipSuccess || ptr == nullptr) return FA_ERR_LAUNCH;
  if (dev >= 0 && dev < kScratchDevs) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    g_scratch_ptr[dev] = ptr;
  }
  *out = ptr;
  return FA_OK;
}

}  // namespace

extern "C" int fa_decode_paged_noalloc(const void* q, const int64_t* q_stride,
                                       const void* kcache, const int64_t* k_stride,
                                       const void* vcache, const int64_t* v_stride,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       void* o, const int64_t* o_stride, float* lse,
                                       int B, int Sq, int Hq, int Hkv, int Dk, int Dv,
                                       int num_pages, int page_size, int max_pages_per_seq, int kv_chunk,
                                       int causal, int window, float scale, const fa_score_mods* mods,
                                       void* stream) {
  // size check first: the partials of this call must fit the static array
  if (B >= 0 && Sq >= 0 && Hq > 0 && max_pages_per_seq >= 0 && dims_ok(Dk, Dv)) {
    const int ps = log2_exact(page_size);
    const int64_t max_len = ps >= 0 ? ((int64_t)max_pages_per_seq << ps) : 0;
    if (ps >= 0 && ps <= 16 && max_len <= INT32_MAX && kv_chunk > 0 && kv_chunk % 32 == 0) {
      const size_t need = fa_decode_workspace_bytes(B, Sq, Hq, Dk > Dv ? Dk : Dv, (int)max_len, kv_chunk);
      if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    }
  }
  // the array of the stream's device (a stream belongs to one device)
  int dev = 0;
  if (stream != nullptr) {
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return FA_ERR_INVALID_ARG;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return FA_ERR_LAUNCH;
  }
  void* ws = nullptr;
  const int st = scratch_address(dev, &ws);
  if (st != FA_OK) return st;
  return decode_impl(q, q_stride, kcache, k_stride, vcache, v_stride, nullptr, nullptr, false, block_table,
                     seq_lens, o, o_stride, lse, B, Sq, Hq, Hkv, Dk, Dv, num_pages, page_size,
                     max_pages_per_seq, kv_chunk, causal, window, scale, mods, ws,
                     (size_t)FA_NOALLOC_SCRATCH_BYTES, stream);
}
