// Split-KV decode / speculative-verify launcher, the LSE combine kernel and
// the paged-gather test hook.
//
// Split-KV: each workgroup takes one (sequence, KV head, block of rows,
// chunk of kv_chunk keys) and writes an fp32 partial output normalised by its
// own row sum plus the row LSE; the combine kernel merges the chunks of a row
// by their LSE (beellama.cpp PR 149: a combine kernel runs after the split
// blocks when the KV range is split into parallel blocks, on the same stream,
// and every partial must publish its (max, rowsum)).
#include <algorithm>

#include "fa_attn_kernel.h"
#include "fa_launch.h"

namespace gqafa {

namespace {

// Split-kernel tile shape by head dim and row waves (32 rows each). Head dim
// 256 splits D over two waves per 32 rows, head dim 512 over four.
template <int D, int NWR> struct SplitCfg {
  static constexpr int DS = D >= 512 ? 4 : (D >= 256 ? 2 : 1);
  static constexpr int NW = NWR * DS;
  static constexpr int BN = (NWR == 4 && D <= 128) ? 64 : 32;
  static constexpr int WPE = D <= 128 ? 2 : 1;
  // tile buffers per operand (measured on MI355X: one row wave streams best
  // with two, a two-wave block with three; larger head dims are LDS-bound)
  static constexpr int NBUF = D == 512 ? 2 : (D == 256 ? 3 : ((NWR == 1 || BN * D >= 8192) ? 2 : 3));
  // several chunks per workgroup
  static constexpr bool MULTI = true;
};

template <int D, int NWR>
hipError_t run_split(const SplitDesc& d, hipStream_t stream) {
  using C = SplitCfg<D, NWR>;
  constexpr int NW = C::NW;
  constexpr int BM = NWR * 32;
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(d.q);
  a.k = static_cast<const uint16_t*>(d.kcache);
  a.v = static_cast<const uint16_t*>(d.vcache);
  a.o_part = d.o_part;
  a.lse_part = d.lse_part;
  a.seq_lens = d.seq_lens;
  a.table = d.table;
  a.page_shift = d.page_shift;
  a.max_pages = d.max_pages;
  a.num_pages = d.num_pages;
  a.slots = (int64_t)d.max_pages << d.page_shift;
  a.B = d.B; a.Sq = d.Sq; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.Hq / d.Hkv;
  a.causal = d.causal; a.window = d.window;
  a.sl2 = d.scale * kLog2e;
  const int64_t rows = (int64_t)d.Sq * a.G;
  a.n_rb = (int)((rows + BM - 1) / BM);
  a.chunk = d.kv_chunk;
  a.max_chunks = d.max_chunks;
  // Very large grids of short chunks merge several consecutive chunks into
  // one workgroup, whose copy stream then runs across chunk boundaries (one
  // partial per chunk is still written); chunks must be whole tiles for this.
  // Up to 16384 chunk slots, one chunk per workgroup streams best.
  const int64_t slots = (int64_t)d.B * d.Hkv * a.n_rb * d.max_chunks;
  int cpw = 1;
  if (C::MULTI && d.kv_chunk % C::BN == 0 && slots > 16384)
    cpw = (int)std::min<int64_t>(d.max_chunks, (slots + 16383) / 16384);
  a.cpw = cpw;
  a.n_cg = (d.max_chunks + cpw - 1) / cpw;
  const int64_t grid = (int64_t)d.B * d.Hkv * a.n_rb * a.n_cg;
  if (grid == 0) return hipSuccess;
  if (d.table != nullptr)
    hipLaunchKernelGGL((attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::MULTI, C::WPE>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::MULTI, C::WPE>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t run_split_d(const SplitDesc& d, hipStream_t stream) {
  const int64_t rows = (int64_t)d.Sq * (d.Hq / d.Hkv);
  if constexpr (D >= 512) {
    return run_split<D, 1>(d, stream);      // LDS holds one 32-row block at D = 512
  } else if constexpr (D >= 256) {
    if (rows <= 32) return run_split<D, 1>(d, stream);
    return run_split<D, 2>(d, stream);
  } else {
    if (rows <= 32) return run_split<D, 1>(d, stream);
    if (rows <= 64) return run_split<D, 2>(d, stream);
    return run_split<D, 4>(d, stream);
  }
}

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  const int32_t* n_chunks;
  const int32_t* seq_lens;
  int kv_chunk, max_chunks;
  uint16_t* o;
  float* lse;
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
// row i), in two memory round trips: every LSE of the row at once (lane k
// holds chunks k and k + 64, ...), then every partial slice the lane needs.
// The lanes cover (chunk, 16-byte slice of D) pairs: with D/4 slices per
// chunk, CPI = 64 / (D/4) chunks per step (D <= 256), or SPL = (D/4) / 64
// slices of one chunk per lane (D = 512). A chunk's weight comes from the
// lane holding its LSE by a lane shuffle.
template <int D>
__global__ void __launch_bounds__(64) combine_kernel(const CombineArgs c) {
  constexpr int SL = D / 4;                       // float4 slices per chunk
  constexpr int CPI = SL >= 64 ? 1 : 64 / SL;     // chunks per step
  constexpr int SPL = SL >= 64 ? SL / 64 : 1;     // slices per lane
  constexpr int MAXL = 4;                          // LSEs held per lane: up to 256 chunks at once
  constexpr int BATCH = 8;                         // partial loads in flight per lane
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int i = (int)(row % c.Sq);
  const int64_t t = row / c.Sq;
  const int h = (int)(t % c.Hq);
  const int b = (int)(t / c.Hq);

  int n = c.max_chunks;
  if (c.n_chunks != nullptr) {
    n = c.n_chunks[b];
  } else if (c.seq_lens != nullptr) {
    const int len = max(c.seq_lens[b], 0);
    n = (int)(((int64_t)len + c.kv_chunk - 1) / c.kv_chunk);
  }
  n = max(0, min(n, c.max_chunks));

  const float* lp = c.lse_part + row * c.max_chunks;
  float lv[MAXL];
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < MAXL; ++r) {
    const int k = lane + 64 * r;
    lv[r] = k < n ? lp[k] : -INFINITY;
    m = fmaxf(m, lv[r]);
  }
  for (int k = lane + 64 * MAXL; k < n; k += 64) m = fmaxf(m, lp[k]);   // rows with > 256 chunks
  m = wave_max(m);

  const int co = CPI > 1 ? lane / SL : 0;         // chunk offset of this lane in a step
  const int sl = CPI > 1 ? lane % SL : lane;      // first slice of this lane
  f32x4 acc[SPL];
#pragma unroll
  for (int v = 0; v < SPL; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lse_out = -INFINITY;
  if (m != -INFINITY) {
    float tot = 0.f;
#pragma unroll
    for (int r = 0; r < MAXL; ++r) tot += fast_exp2((lv[r] - m) * kLog2e);
    for (int k = lane + 64 * MAXL; k < n; k += 64) tot += fast_exp2((lp[k] - m) * kLog2e);
    tot = wave_sum(tot);
    const float inv = 1.0f / tot;
    lse_out = m + fast_log2(tot) * kLn2;
    const float* op = c.o_part + row * c.max_chunks * D;
    for (int k0 = 0; k0 < n; k0 += CPI * BATCH) {
      f32x4 x[BATCH][SPL];
      float lk[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int k = k0 + CPI * u + co;
        // the LSE of chunk k sits in lane k % 64, register k / 64 (< 256 chunks)
        // (k / 64 is the same for the whole wave: 64 is a multiple of CPI)
        float src = lv[0];
#pragma unroll
        for (int r = 1; r < MAXL; ++r)
          if (((k0 + CPI * u) >> 6) == r) src = lv[r];
        const float from_lane = __shfl(src, k & 63, 64);
        lk[u] = k < n ? (k < 64 * MAXL ? from_lane : lp[k]) : -INFINITY;
#pragma unroll
        for (int v = 0; v < SPL; ++v)
          x[u][v] = (k < n && lk[u] != -INFINITY)
                        ? *reinterpret_cast<const f32x4*>(op + (int64_t)k * D + 4 * (sl + 64 * v))
                        : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        // empty chunk (LSE -inf): weight 0 and its contents are never read
        const float w = lk[u] == -INFINITY ? 0.f : fast_exp2((lk[u] - m) * kLog2e) * inv;
#pragma unroll
        for (int v = 0; v < SPL; ++v) acc[v] += w * x[u][v];
      }
    }
    // add the CPI lane groups that hold the same slice
#pragma unroll
    for (int sft = 32; sft >= SL && CPI > 1; sft >>= 1)
#pragma unroll
      for (int v = 0; v < SPL; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[v][e] += __shfl_xor(acc[v][e], sft, 64);
  }
  if (co == 0) {
    uint16_t* dst = c.o + (((int64_t)b * c.Sq + i) * c.Hq + h) * D;
#pragma unroll
    for (int v = 0; v < SPL; ++v) {
      u32x2 val = {pack_bf16(acc[v][0], acc[v][1]), pack_bf16(acc[v][2], acc[v][3])};
      *reinterpret_cast<u32x2*>(dst + 4 * (sl + 64 * v)) = val;
    }
  }
  if (c.lse != nullptr && lane == 0) c.lse[((int64_t)b * c.Hq + h) * c.Sq + i] = lse_out;
}

template <int D>
hipError_t run_combine(const CombineDesc& d, hipStream_t stream) {
  CombineArgs c{d.o_part, d.lse_part, d.n_chunks, d.seq_lens, d.kv_chunk, d.max_chunks,
                static_cast<uint16_t*>(d.o), d.lse, d.B, d.Sq, d.Hq};
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

// One thread per 16-byte chunk of the dense output; grid-stride.
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
    KvAddr kv;
    kv.table = a.table;
    kv.page_shift = a.page_shift;
    kv.max_pages = a.max_pages;
    kv.num_pages = a.num_pages;
    kv.slots = slots;
    kv.row_stride = (int64_t)a.Hkv * a.D;
    kv.head_off = (int64_t)g * a.D;
    int64_t len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > slots ? slots : len);
    const int64_t off = t < len ? kv.row(b, t) : -1;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (off >= 0) w = *reinterpret_cast<const u32x4*>(a.cache + off + 8 * ch);
    *reinterpret_cast<u32x4*>(a.out + (((int64_t)b * slots + t) * a.Hkv + g) * a.D + 8 * ch) = w;
  }
}

}  // namespace

hipError_t launch_split(const SplitDesc& d, hipStream_t stream) {
  switch (d.D) {
    case 64: return run_split_d<64>(d, stream);
    case 128: return run_split_d<128>(d, stream);
    case 256: return run_split_d<256>(d, stream);
    case 512: return run_split_d<512>(d, stream);
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
