// Split-KV decode / speculative-verify launcher, the LSE combine kernel and
// the paged-gather test hook.
//
// Split-KV: a persistent grid, one workgroup per slot the GPU holds at once,
// streams all K/V tiles in equal contiguous ranges (whole tiles of chunks of
// kv_chunk keys) and writes one fp32 partial output per range and block of
// rows, normalised by its own row sum, plus the row LSEs; the combine kernel
// merges the partials of a row by their LSE (beellama.cpp PR 149: a combine kernel runs after the split blocks
// when the KV range is split into parallel blocks, on the same stream, and
// every partial must publish its (max, rowsum)).
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
  static constexpr int BN = 32;
  // waves per SIMD the registers are sized for: one-wave workgroups (four
  // per CU, held by LDS) run one wave per SIMD; two- and four-wave ones two
  static constexpr int WPE = (D <= 128 && NW > 1) ? 2 : 1;
  // with a mask (its values stay in registers through a step) or head dims
  // below D, the two- and four-wave D = 128 kernels need more than half the
  // register file
  static constexpr int WPE_MASK = (D == 128 && NW >= 2) ? 1 : WPE;
  // tile buffers per operand: two keep 3/4 of the ring in flight; larger
  // head dims are LDS-bound
  static constexpr int NBUF = 2;
  // fp8 tiles are half the bytes. One-wave workgroups keep two buffers: 18
  // KiB of LDS lets a CU hold eight of them, two waves per SIMD, with as many
  // bytes in flight as four bf16 workgroups (the one-wave kernel is bound by
  // the latency of its own step, so a second wave per SIMD is what pays).
  // Wider workgroups are held by registers at two waves per SIMD and take
  // deeper rings instead (three for the paged two-wave kernel, which holds
  // no more within its register budget).
  static constexpr int NBUF8 = NW == 1 ? 2 : 4;
  static constexpr int NBUF8P = NW == 1 ? 2 : (NW == 2 ? 3 : 4);
  static constexpr int WPE8 = 2;
};

// Workgroups of a kernel the GPU holds at once: CUs x resident workgroups per
// CU. Measured on MI355X, a CU holds at most 144 KiB of LDS across
// workgroups of 32 KiB or less (the occupancy query allows 160), so the
// count is the smaller of the two.
template <typename Kernel>
int resident_workgroups(Kernel kernel, int threads, int* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (cache[dev] > 0) return cache[dev];
  int occ = 0, cus = 0;
  hipFuncAttributes attr{};
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess) occ = 1;
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel)) == hipSuccess &&
      attr.sharedSizeBytes > 0)
    occ = std::min<int>(occ, (int)(147456 / attr.sharedSizeBytes));
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
  cache[dev] = std::max(occ, 1) * std::max(cus, 1);
  return cache[dev];
}

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
  a.q_sb = d.qs.outer; a.q_ss = d.qs.token; a.q_sh = d.qs.head;
  a.k_sb = d.ks.outer; a.k_ss = d.ks.token; a.k_sh = d.ks.head;
  a.v_sb = d.vs.outer; a.v_ss = d.vs.token; a.v_sh = d.vs.head;
  a.B = d.B; a.Sq = d.Sq; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.Hq / d.Hkv;
  a.causal = d.causal; a.window = d.window;
  a.sl2 = d.scale * kLog2e;
  a.dk = d.dk;
  a.dv = d.dv;
  a.k_scale = d.k_scale;
  a.v_scale = d.v_scale;
  set_mods(a, d.scale, d.softcap, d.max_bias, nullptr, d.Hq, d.mask, d.mask_sb, d.mask_ss);
  const int64_t rows = (int64_t)d.Sq * a.G;
  a.n_rb = (int)((rows + BM - 1) / BM);
  a.chunk = d.kv_chunk;
  a.n_slots = d.n_slots;
  // kernel level: 0 plain, 1 softcap / ALiBi, 2 with a mask; with head dims
  // below D, 3 (no score transform) or 4 (transform and mask). Sinks are
  // added by the combine.
  const bool xform = d.softcap > 0.f || d.max_bias > 0.f;
  const int level = (d.dk < D || d.dv < D) ? (xform || d.mask != nullptr ? 4 : 3)
                    : d.mask != nullptr ? 2 : (xform ? 1 : 0);
  using K = decltype(&attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE, 0>);
  static const K kernels[2][5] = {
      {attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::WPE, 0>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::WPE, 1>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::WPE_MASK, 2>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::WPE_MASK, 3>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::WPE_MASK, 4>},
      {attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE, 0>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE, 1>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE_MASK, 2>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE_MASK, 3>,
       attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE_MASK, 4>}};
  const int paged = d.table != nullptr ? 1 : 0;
  K k = kernels[paged][level];
  int* cache_row;
  // the grid is what the chosen kernel holds resident
  static int cache[2][5][16];
  cache_row = cache[paged][level];
  if constexpr (D == 128) {
    if (d.kv8) {
      // fp8 caches: plain, or score transform and mask (softcap / ALiBi alone
      // run with a null mask)
      static const K kernels8[2][2] = {
          {attn_kernel<D, NW, C::BN, C::DS, C::NBUF8, false, true, C::WPE8, 0, true>,
           attn_kernel<D, NW, C::BN, C::DS, C::NBUF8, false, true, C::WPE_MASK, 2, true>},
          {attn_kernel<D, NW, C::BN, C::DS, C::NBUF8P, true, true, C::WPE8, 0, true>,
           attn_kernel<D, NW, C::BN, C::DS, C::NBUF8P, true, true, C::WPE_MASK, 2, true>}};
      static int cache8[2][2][16];
      const int l8 = level == 0 ? 0 : 1;
      k = kernels8[paged][l8];
      cache_row = cache8[paged][l8];
    }
  }
  const int resident = resident_workgroups(k, NW * 64, cache_row);
  // whole sets of Hkv workgroups, one per KV head
  const int grid = std::max(resident / d.Hkv, 1) * d.Hkv;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(NW * 64), 0, stream, a);
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

  int n = c.n_slots;
  if (c.n_chunks != nullptr) {
    n = c.n_chunks[b];
  } else if (c.seq_lens != nullptr) {
    const int len = max(c.seq_lens[b], 0);
    n = len > 0 ? (int)(((int64_t)len + c.kv_chunk - 1) / c.kv_chunk) + 1 : 0;
  }
  n = max(0, min(n, c.n_slots));

  const float* lp = c.lse_part + row * c.n_slots;
  const float* op = c.o_part + row * c.n_slots * D;
  auto load_block = [&](int b0, float (&lv)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = b0 + lane + 64 * r;
      lv[r] = k < n ? lp[k] : -INFINITY;
    }
  };
  float lv[4];
  load_block(0, lv);
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
  CombineArgs c{d.o_part, d.lse_part, d.n_chunks, d.seq_lens, d.kv_chunk, d.n_slots,
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
