// Prefill launcher: one workgroup per (sequence, KV head, block of rows).
#include "fa_attn_kernel.h"
#include "fa_launch.h"

namespace gqafa {

namespace {

// Tile shape per head dim: waves per workgroup, keys per tile, D split (two
// waves per 32 rows) and the waves per SIMD the register budget is sized for.
// Head dim 256 runs one full-D wave per SIMD (Q fed to the MFMAs from AGPRs):
// measured on MI355X 7 % faster than a D split over two waves per 32 rows
// at two waves per SIMD, which exponentiated every tile twice and exchanged
// partial scores through LDS. Head dim 512 keeps the split: one full-D
// wave's O alone would fill the register file.
template <int D> struct PrefillCfg;
template <> struct PrefillCfg<64>  { static constexpr int NW = 4, BN = 64, DS = 1, WPE = 2; };
template <> struct PrefillCfg<128> { static constexpr int NW = 4, BN = 64, DS = 1, WPE = 2; };
template <> struct PrefillCfg<256> { static constexpr int NW = 4, BN = 32, DS = 1, WPE = 1; };
template <> struct PrefillCfg<512> { static constexpr int NW = 4, BN = 32, DS = 2, WPE = 1; };

template <int D>
hipError_t run(const PrefillDesc& d, hipStream_t stream) {
  using C = PrefillCfg<D>;
  constexpr int BM = C::NW * 32 / C::DS;
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(d.q);
  a.k = static_cast<const uint16_t*>(d.k);
  a.v = static_cast<const uint16_t*>(d.v);
  a.o = static_cast<uint16_t*>(d.o);
  a.lse = d.lse;
  a.q_sb = d.qs.outer; a.q_ss = d.qs.token; a.q_sh = d.qs.head;
  a.o_sb = d.os.outer; a.o_ss = d.os.token; a.o_sh = d.os.head;
  a.k_sb = d.ks.outer; a.k_ss = d.ks.token; a.k_sh = d.ks.head;
  a.v_sb = d.vs.outer; a.v_ss = d.vs.token; a.v_sh = d.vs.head;
  a.B = d.B; a.Sq = d.Sq; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.Hq / d.Hkv;
  a.skv = d.Skv;
  a.causal = d.causal; a.window = d.window;
  a.sl2 = d.scale * kLog2e;
  a.dk = d.dk;
  a.dv = d.dv;
  set_mods(a, d.scale, d.softcap, d.max_bias, d.sinks, d.Hq, d.mask, d.mask_sb, d.mask_ss);
  const int64_t rows = (int64_t)d.Sq * a.G;
  a.n_rb = (int)((rows + BM - 1) / BM);
  const int64_t grid = (int64_t)d.B * d.Hkv * a.n_rb;
  if (grid == 0) return hipSuccess;
  // kernel level: 0 plain (sinks are read in the epilogue of every level),
  // 1 softcap / ALiBi, 2 with a mask; with head dims below D, 3 (no score
  // transform) or 4 (transform and mask)
  const bool xform = d.softcap > 0.f || d.max_bias > 0.f;
  if constexpr (D == 512) {
    if (d.dk > D) {
      // 576-wide keys (the 512 tile plus 64 extra key columns): plain, or
      // with the score transform and mask (softcap / ALiBi alone run with a
      // null mask)
      if (xform || d.mask != nullptr)
        hipLaunchKernelGGL((attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 2, false, true>),
                           dim3((unsigned)grid), dim3(C::NW * 64), 0, stream, a);
      else
        hipLaunchKernelGGL((attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 0, false, true>),
                           dim3((unsigned)grid), dim3(C::NW * 64), 0, stream, a);
      return hipGetLastError();
    }
  }
  const int level = (d.dk < D || d.dv < D) ? (xform || d.mask != nullptr ? 4 : 3)
                    : d.mask != nullptr ? 2 : (xform ? 1 : 0);
  if constexpr (D == 128) {
    if (level == 0) {
      // eight waves in two ping-pong groups, 256 rows per workgroup
      constexpr int kWaves = 8;
      a.n_rb = (int)((rows + kWaves * 32 - 1) / (kWaves * 32));
      const int64_t grid_pp = (int64_t)d.B * d.Hkv * a.n_rb;
      hipLaunchKernelGGL((attn_kernel<D, kWaves, 64, 1, 3, false, false, 2, 0>), dim3((unsigned)grid_pp),
                         dim3(kWaves * 64), 0, stream, a);
      return hipGetLastError();
    }
  }
  using K = decltype(&attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 0>);
  static const K kernels[5] = {
      &attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 0>,
      &attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 1>,
      &attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 2>,
      &attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 3>,
      &attn_kernel<D, C::NW, C::BN, C::DS, 2, false, false, C::WPE, 4>};
  const K kern = kernels[level];
  int64_t g_launch = grid;
  if constexpr (D == 256) {
    // persistent kernels: as many workgroups as the GPU holds at once, each
    // taking several blocks of rows
    static std::atomic<int> cache[5][kResidentDevs];
    g_launch = std::min<int64_t>(grid, resident_workgroups(kern, C::NW * 64, cache[level], stream));
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)g_launch), dim3(C::NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillDesc& d, hipStream_t stream) {
  switch (d.D) {
    case 64: return run<64>(d, stream);
    case 128: return run<128>(d, stream);
    case 256: return run<256>(d, stream);
    case 512: return run<512>(d, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqafa
