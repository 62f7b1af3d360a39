// Split-KV dispatch by head dim, the LSE combine kernel and the paged-gather
// test hook (which applies the split kernel's page address rule, clamp_page
// and paged_row of fa_device.h, to every token).
//
// Split-KV (fa_split.h): a persistent grid streams all K/V tiles in equal
// contiguous ranges and writes one fp32 partial output per range and block
// of rows, normalised by its own row sum, plus the row LSEs; the combine
// kernel merges the partials of a row by their LSE (beellama.cpp PR 149: a combine kernel runs after the split blocks
// when the KV range is split into parallel blocks, on the same stream, and
// every partial must publish its (max, rowsum)).
#include <algorithm>

#include "fa_attn_kernel.h"
#include "fa_launch.h"

namespace gqafa {

namespace {

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  const int32_t* n_chunks;
  const int32_t* seq_lens;
  int max_len;
  int kv_chunk, n_slots;
  uint16_t* o;
  float* lse;
  int64_t o_sb, o_ss, o_sh;     // element strides of o (sequence, row, head)
  const float* sinks;           // per query head logit joining the denominator, or null
  int dv;                       // columns of O written
  int B, Sq, Hq;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) x = fmaxf(x, __shfl_xor(x, s, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) x += __shfl_xor(x, s, 64);
  return x;
}

// One wave (one workgroup) per output row (sequence b, query head h, query
// row i). The row's slots are taken in blocks of 256 (four LSEs per lane);
// the non-empty ones (finite LSE) of a block are listed in LDS by ballot and
// lane-prefix count, and their partial outputs are fetched CPI x BATCH at a
// time: with D/4 16-byte slices per partial, the lanes cover (partial, slice)
// pairs, CPI = 64 / (D/4) partials per step (D <= 256) or SPL = (D/4) / 64
// slices of one partial per lane (D = 512). Rows of at most 256 slots (the
// common case) read their LSEs once; longer rows read them once for the max
// and again per block.
template <int D>
__global__ void __launch_bounds__(64) combine_kernel(const CombineArgs c) {
  constexpr int SL = D / 4;                       // float4 slices per partial
  constexpr int CPI = SL >= 64 ? 1 : 64 / SL;     // partials per step
  constexpr int SPL = SL >= 64 ? SL / 64 : 1;     // slices per lane
  constexpr int BATCH = 16 / SPL;                  // steps whose loads are in flight together
  __shared__ int s_slot[256];
  __shared__ float s_lse[256];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int i = (int)(row % c.Sq);
  const int64_t t = row / c.Sq;
  const int h = (int)(t % c.Hq);
  const int b = (int)(t / c.Hq);

  const float* lp = c.lse_part + row * c.n_slots;
  const float* op = c.o_part + row * c.n_slots * D;
  // The first block of LSEs is loaded before the row's slot count is known
  // (every slot below n_slots lies in the buffer; those past the count are
  // dropped below), so the two loads take one memory round trip.
  float lv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = lane + 64 * r;
    lv[r] = k < c.n_slots ? lp[k] : -INFINITY;
  }
  int n = c.n_slots;
  if (c.n_chunks != nullptr) {
    n = c.n_chunks[b];
  } else if (c.seq_lens != nullptr) {
    // the split kernel clamps lengths into the cache the same way
    const int len = min(max(c.seq_lens[b], 0), c.max_len);
    n = len > 0 ? (int)(((int64_t)len + c.kv_chunk - 1) / c.kv_chunk) + 1 : 0;
  }
  n = max(0, min(n, c.n_slots));
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (lane + 64 * r >= n) lv[r] = -INFINITY;

  auto load_block = [&](int b0, float (&lv)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = b0 + lane + 64 * r;
      lv[r] = k < n ? lp[k] : -INFINITY;
    }
  };
  float m = fmaxf(fmaxf(lv[0], lv[1]), fmaxf(lv[2], lv[3]));
  for (int b0 = 256; b0 < n; b0 += 256) {
    float lw[4];
    load_block(b0, lw);
    m = fmaxf(m, fmaxf(fmaxf(lw[0], lw[1]), fmaxf(lw[2], lw[3])));
  }
  m = wave_max(m);
  // a sink logit is one more partial with O = 0
  const float sink = c.sinks != nullptr ? c.sinks[h] : -INFINITY;
  m = fmaxf(m, sink);

  const int co = CPI > 1 ? lane / SL : 0;         // partial offset of this lane in a step
  const int sl = CPI > 1 ? lane % SL : lane;      // first slice of this lane
  f32x4 acc[SPL];
#pragma unroll
  for (int v = 0; v < SPL; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lse_out = -INFINITY;
  if (m != -INFINITY) {
    float tot = 0.f;
    for (int b0 = 0; b0 < n; b0 += 256) {
      if (b0 > 0) load_block(b0, lv);
      // list the block's non-empty slots (empty ones: weight 0, O never read)
      int nv = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = lv[r] != -INFINITY;
        const uint64_t mask = __builtin_amdgcn_ballot_w64(ok);
        const int pos = nv + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (ok) {
          s_slot[pos] = b0 + lane + 64 * r;
          s_lse[pos] = lv[r];
          tot += fast_exp2((lv[r] - m) * kLog2e);
        }
        nv += __builtin_popcountll(mask);
      }
      __syncthreads();
      for (int k0 = 0; k0 < nv; k0 += CPI * BATCH) {
        f32x4 x[BATCH][SPL];
        float e[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int j = k0 + CPI * u + co;
          const bool ok = j < nv;
          const int slot = ok ? s_slot[j] : 0;
          e[u] = ok ? fast_exp2((s_lse[j] - m) * kLog2e) : 0.f;
#pragma unroll
          for (int v = 0; v < SPL; ++v)
            x[u][v] = ok ? *reinterpret_cast<const f32x4*>(op + (int64_t)slot * D + 4 * (sl + 64 * v))
                         : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
#pragma unroll
          for (int v = 0; v < SPL; ++v) acc[v] += e[u] * x[u][v];
      }
      __syncthreads();                            // the list is rewritten by the next block
    }
    tot = wave_sum(tot);
    if (sink != -INFINITY) tot += fast_exp2((sink - m) * kLog2e);
    const float inv = 1.0f / tot;
    lse_out = m + fast_log2(tot) * kLn2;
#pragma unroll
    for (int v = 0; v < SPL; ++v) acc[v] *= inv;
    // add the CPI lane groups that hold the same slice
#pragma unroll
    for (int sft = 32; sft >= SL && CPI > 1; sft >>= 1)
#pragma unroll
      for (int v = 0; v < SPL; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[v][e] += __shfl_xor(acc[v][e], sft, 64);
  }
  if (co == 0) {
    uint16_t* dst = c.o + (int64_t)b * c.o_sb + (int64_t)i * c.o_ss + (int64_t)h * c.o_sh;
#pragma unroll
    for (int v = 0; v < SPL; ++v) {
      u32x2 val = {pack_bf16(acc[v][0], acc[v][1]), pack_bf16(acc[v][2], acc[v][3])};
      if (4 * (sl + 64 * v) < c.dv) *reinterpret_cast<u32x2*>(dst + 4 * (sl + 64 * v)) = val;
    }
  }
  if (c.lse != nullptr && lane == 0) c.lse[((int64_t)b * c.Hq + h) * c.Sq + i] = lse_out;
}

template <int D>
hipError_t run_combine(const CombineDesc& d, hipStream_t stream) {
  CombineArgs c{d.o_part, d.lse_part, d.n_chunks, d.seq_lens, d.max_len, d.kv_chunk, d.n_slots,
                static_cast<uint16_t*>(d.o), d.lse, d.os.outer, d.os.token, d.os.head, d.sinks,
                d.dv, d.B, d.Sq, d.Hq};
  const int64_t rows = (int64_t)d.B * d.Hq * d.Sq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)rows), dim3(64), 0, stream, c);
  return hipGetLastError();
}

struct GatherArgs {
  const uint16_t* cache;
  const int32_t* table;
  const int32_t* seq_lens;
  uint16_t* out;
  int B, Hkv, D, num_pages, page_shift, max_pages;
};

// One thread per 16-byte chunk of the dense output; grid-stride. Slots at or
// past a sequence's length are written as zero.
__global__ void __launch_bounds__(256) gather_kernel(const GatherArgs a) {
  const int64_t slots = (int64_t)a.max_pages << a.page_shift;
  const int chunks = a.D / 8;
  const int64_t total = (int64_t)a.B * slots * a.Hkv * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int ch = (int)(idx % chunks);
    int64_t rest = idx / chunks;
    const int g = (int)(rest % a.Hkv);
    rest /= a.Hkv;
    const int t = (int)(rest % slots);
    const int b = (int)(rest / slots);
    int64_t len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > slots ? slots : len);
    // the split kernel's address rule: clamped page, then slot
    const int64_t off = t < len ? paged_row(clamp_page(a.table[(int64_t)b * a.max_pages + (t >> a.page_shift)],
                                                       a.num_pages),
                                            t & ((1 << a.page_shift) - 1),
                                            ((int64_t)a.Hkv * a.D) << a.page_shift, (int64_t)a.Hkv * a.D) +
                                      (int64_t)g * a.D
                                : -1;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (off >= 0) w = *reinterpret_cast<const u32x4*>(a.cache + off + 8 * ch);
    *reinterpret_cast<u32x4*>(a.out + (((int64_t)b * slots + t) * a.Hkv + g) * a.D + 8 * ch) = w;
  }
}

}  // namespace

hipError_t launch_split(const SplitDesc& d, hipStream_t stream) {
  switch (d.D) {
    case 64: return launch_split_d64(d, stream);
    case 128: return launch_split_d128(d, stream);
    case 256: return launch_split_d256(d, stream);
    case 512: return launch_split_d512(d, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const CombineDesc& d, hipStream_t stream) {
  switch (d.D) {
    case 64: return run_combine<64>(d, stream);
    case 128: return run_combine<128>(d, stream);
    case 256: return run_combine<256>(d, stream);
    case 512: return run_combine<512>(d, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gather(const GatherDesc& d, hipStream_t stream) {
  GatherArgs a{static_cast<const uint16_t*>(d.cache), d.table, d.seq_lens,
               static_cast<uint16_t*>(d.out), d.B, d.Hkv, d.D, d.num_pages, d.page_shift, d.max_pages};
  const int64_t slots = (int64_t)d.max_pages << d.page_shift;
  const int64_t total = (int64_t)d.B * slots * d.Hkv * (d.D / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gqafa
