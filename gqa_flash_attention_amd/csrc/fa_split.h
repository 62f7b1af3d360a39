// Split-KV decode / speculative-verify launcher: a persistent grid, one
// workgroup per slot the GPU holds at once, streams all K/V tiles in equal
// contiguous ranges (whole tiles of chunks of kv_chunk keys) and writes one
// fp32 partial output per range and block of rows, normalised by its own row
// sum, plus the row LSEs (merged by the combine kernel in fa_decode.hip).
// Included by one source per head dim (fa_split_d*.hip), so that the many
// kernel instantiations compile in parallel.
#pragma once

#include <algorithm>
#include <atomic>

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
  static constexpr int NBUF8 = (NW == 1 || D > 128) ? 2 : 4;
  static constexpr int NBUF8P = (NW == 1 || D > 128) ? 2 : (NW == 2 ? 3 : 4);
  // Above head dim 128 the fp8 kernels split D over the waves of 32 rows as
  // the bf16 ones do, with the half-size tiles in a two-buffer ring (two
  // workgroups per CU at 256, one at 512 by LDS).
  static constexpr int WPE8 = 2;
  static constexpr int WPE8_MASK = D == 128 ? WPE_MASK : 2;
  // keys per fp8 tile: the one-wave head-dim-128 kernel takes 64 (the bytes
  // of a 32-key bf16 tile) at one wave per SIMD, so it runs the bf16
  // kernel's step count per byte
  static constexpr int BN8 = (D == 128 && NW == 1) ? 64 : 32;
  static constexpr int WPE8_1 = (D == 128 && NW == 1) ? 1 : WPE8;
  static constexpr int WPE8M_1 = (D == 128 && NW == 1) ? 1 : WPE8_MASK;
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
  std::atomic<int>* cache_row;
  // the grid is what the chosen kernel holds resident
  static std::atomic<int> cache[2][5][kResidentDevs];
  cache_row = cache[paged][level];
  if constexpr (D == 512) {
    if (d.dk > D) {
      // 576-wide keys: plain, or score transform and mask
      static const K kernelsx[2][2] = {
          {attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::WPE, 0, false, true>,
           attn_kernel<D, NW, C::BN, C::DS, C::NBUF, false, true, C::WPE, 2, false, true>},
          {attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE, 0, false, true>,
           attn_kernel<D, NW, C::BN, C::DS, C::NBUF, true, true, C::WPE, 2, false, true>}};
      static std::atomic<int> cachex[2][2][kResidentDevs];
      const int lx = level == 0 ? 0 : 1;
      k = kernelsx[paged][lx];
      cache_row = cachex[paged][lx];
    }
  }
  if constexpr (D >= 128) {
    if (d.kv8) {
      // fp8 caches: plain, or score transform and mask (softcap / ALiBi alone
      // run with a null mask)
      static const K kernels8[2][2] = {
          {attn_kernel<D, NW, C::BN8, C::DS, C::NBUF8, false, true, C::WPE8_1, 0, true>,
           attn_kernel<D, NW, C::BN8, C::DS, C::NBUF8, false, true, C::WPE8M_1, 2, true>},
          {attn_kernel<D, NW, C::BN8, C::DS, C::NBUF8P, true, true, C::WPE8_1, 0, true>,
           attn_kernel<D, NW, C::BN8, C::DS, C::NBUF8P, true, true, C::WPE8M_1, 2, true>}};
      static std::atomic<int> cache8[2][2][kResidentDevs];
      const int l8 = level == 0 ? 0 : 1;
      k = kernels8[paged][l8];
      cache_row = cache8[paged][l8];
    }
  }
  const int resident = resident_workgroups(k, NW * 64, cache_row, stream);
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

}  // namespace

}  // namespace gqafa
