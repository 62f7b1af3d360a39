// Internal launchers behind the C ABI. Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqafa {

struct PrefillDesc {
  const void* q; const void* k; const void* v; void* o; float* lse;
  int B, Hq, Hkv, Sq, Skv, D, causal, window;
  float scale;
};

struct SplitDesc {
  const void* q; const void* kcache; const void* vcache;
  const int32_t* table; const int32_t* seq_lens;
  float* o_part; float* lse_part;
  int B, Sq, Hq, Hkv, D, num_pages, page_shift, max_pages, kv_chunk, max_chunks, causal, window;
  float scale;
};

struct CombineDesc {
  const float* o_part; const float* lse_part;
  const int32_t* n_chunks;   // device [B] or null
  const int32_t* seq_lens;   // used when n_chunks is null and kv_chunk > 0
  int kv_chunk, max_chunks;
  void* o; float* lse;
  int B, Sq, Hq, D;
};

struct GatherDesc {
  const void* cache; const int32_t* table; const int32_t* seq_lens; void* out;
  int B, Hkv, D, num_pages, page_shift, max_pages;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_prefill(const PrefillDesc& d, hipStream_t stream);
hipError_t launch_split(const SplitDesc& d, hipStream_t stream);
hipError_t launch_combine(const CombineDesc& d, hipStream_t stream);
hipError_t launch_gather(const GatherDesc& d, hipStream_t stream);

}  // namespace gqafa
