// Internal launchers behind the C ABI. Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace gqafa {

// Element strides of a [B, S, H, D] tensor (or a paged cache [pages, slots,
// H, D]): outer (batch or page), token (or slot), head; D is unit-stride.
struct Strides {
  int64_t outer, token, head;
};

struct PrefillDesc {
  const void* q; const void* k; const void* v; void* o; float* lse;
  Strides qs, ks, vs, os;
  int B, Hq, Hkv, Sq, Skv, D, causal, window;   // D: the tile width (64, 128, 256 or 512)
  int dk, dv;                         // key / value head dims, multiples of 8, <= D
  float scale;
  float softcap, max_bias;            // 0 = off
  const float* sinks;                 // device [Hq] or null
  const void* mask;                   // device bf16 additive mask or null
  int64_t mask_sb, mask_ss;           // its sequence and query-row strides (keys unit-stride)
};

struct SplitDesc {
  const void* q; const void* kcache; const void* vcache;
  const int32_t* table; const int32_t* seq_lens;
  float* o_part; float* lse_part;   // [B, Hq, Sq, n_slots(, D)]: chunks + 1 slots per row
  Strides qs, ks, vs;
  int B, Sq, Hq, Hkv, D, num_pages, page_shift, max_pages, kv_chunk, n_slots, causal, window;
  int dk, dv;                         // key / value head dims, multiples of 8, <= D
  float scale;
  float softcap, max_bias;            // 0 = off (sinks are the combine's)
  const void* mask;                   // device bf16 additive mask (token positions) or null
  int64_t mask_sb, mask_ss;
  bool kv8;                           // fp8 (OCP e4m3) caches, D = 128
  const float* k_scale;               // kv8: device [Hkv] dequantisation scales
  const float* v_scale;
};

struct CombineDesc {
  const float* o_part; const float* lse_part;
  const int32_t* n_chunks;   // device [B] or null: partials to merge per sequence
  const int32_t* seq_lens;   // used when n_chunks is null: ceil(len / kv_chunk) + 1 slots (0 if len = 0),
                             // len = seq_lens[b] clamped to [0, max_len]
  int max_len;               // keys a sequence can hold (the cache's capacity)
  int kv_chunk, n_slots;     // n_slots: slots per row in memory
  void* o; float* lse;
  Strides os;                // o [B, Sq, Hq, D]
  const float* sinks;        // device [Hq] logits joining each row's denominator, or null
  int B, Sq, Hq, D;          // D: width of a partial (64, 128, 256 or 512)
  int dv;                    // columns of O written (a multiple of 8, <= D)
};

struct AppendDesc {
  void* kcache; void* vcache; const void* knew; const void* vnew;
  const int32_t* table; const int32_t* seq_lens;
  Strides kcs, vcs, kns, vns;
  int B, Snew, Hkv, dk, dv, num_pages, page_shift, max_pages;   // dk, dv: multiples of 8
};

struct AppendFp8Desc {
  void* kcache; void* vcache; const void* knew; const void* vnew;   // caches: one byte per element
  const float* k_scale; const float* v_scale;                         // device [Hkv]
  const int32_t* table; const int32_t* seq_lens;
  Strides kcs, vcs, kns, vns;
  int B, Snew, Hkv, D, num_pages, page_shift, max_pages;
};

struct GatherDesc {
  const void* cache; const int32_t* table; const int32_t* seq_lens; void* out;
  int B, Hkv, D, num_pages, page_shift, max_pages;
};

// Workgroups of a kernel the GPU holds at once: CUs x resident workgroups per
// CU. Measured on MI355X, a CU holds at most 144 KiB of LDS across
// workgroups of 32 KiB or less (the occupancy query allows 160), so the
// count is the smaller of the two. The device is the stream's (the current
// one for the null stream). The answer is kept per device (the library's
// only process state besides the no-allocation scratch array: a pure
// function of the kernel and the device; used by the split kernels and the
// persistent prefill kernels); devices past the table are
// queried on every call.
inline constexpr int kResidentDevs = 64;
template <typename Kernel>
inline int resident_workgroups(Kernel kernel, int threads, std::atomic<int>* cache, hipStream_t stream) {
  int dev = 0;
  const bool known = (stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) == hipSuccess;
  const bool keep = known && dev >= 0 && dev < kResidentDevs;
  if (keep) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int occ = 0, cus = 0;
  hipFuncAttributes attr{};
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess) occ = 1;
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel)) == hipSuccess &&
      attr.sharedSizeBytes > 0)
    occ = std::min<int>(occ, (int)(147456 / attr.sharedSizeBytes));
  if (!known || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
  const int n = std::max(occ, 1) * std::max(cus, 1);
  if (keep) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Each returns hipSuccess or the launch error.
hipError_t launch_prefill(const PrefillDesc& d, hipStream_t stream);
hipError_t launch_split(const SplitDesc& d, hipStream_t stream);
hipError_t launch_combine(const CombineDesc& d, hipStream_t stream);
hipError_t launch_gather(const GatherDesc& d, hipStream_t stream);
hipError_t launch_append(const AppendDesc& d, hipStream_t stream);
// split kernels of one tile width each (fa_split_d*.hip)
hipError_t launch_split_d64(const SplitDesc& d, hipStream_t stream);
hipError_t launch_split_d128(const SplitDesc& d, hipStream_t stream);
hipError_t launch_split_d256(const SplitDesc& d, hipStream_t stream);
hipError_t launch_split_d512(const SplitDesc& d, hipStream_t stream);
hipError_t launch_append_fp8(const AppendFp8Desc& d, hipStream_t stream);

}  // namespace gqafa
