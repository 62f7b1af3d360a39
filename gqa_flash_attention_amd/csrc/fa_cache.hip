// KV-cache append: writes the newest K/V rows of each sequence into a paged
// (or contiguous) cache through the block table -- the step that precedes a
// decode or verify call over the same cache. All operands are read and
// written by stride (ATOM PR 2938, Summary: only the innermost dimension
// needs unit stride), so K and V may share one allocation.
#include <algorithm>

#include "fa_device.h"
#include "fa_launch.h"

namespace gqafa {

namespace {

struct AppendArgs {
  uint16_t* kc;
  uint16_t* vc;
  const uint16_t* kn;
  const uint16_t* vn;
  const int32_t* table;       // [B, max_pages] or null (contiguous cache)
  const int32_t* seq_lens;    // [B]: tokens in the cache including the new rows
  int64_t kc_sb, kc_ss, kc_sh, vc_sb, vc_ss, vc_sh;   // cache strides (page or sequence, slot, head)
  int64_t kn_sb, kn_ss, kn_sh, vn_sb, vn_ss, vn_sh;   // new rows [B, Snew, Hkv, D]
  int B, Snew, Hkv, dk, dv, num_pages, page_shift, max_pages;
};

// One thread per 16-byte chunk of the new rows (the wider of the K and V
// rows); grid-stride. New row i of sequence b lands at token seq_lens[b] -
// Snew + i. Rows whose token would be negative (a sequence shorter than
// Snew) and rows whose block-table entry is outside [0, num_pages) are not
// written.
__global__ void __launch_bounds__(256) append_kernel(const AppendArgs a) {
  const int chunks = max(a.dk, a.dv) / 8;
  const int64_t total = (int64_t)a.B * a.Snew * a.Hkv * chunks;
  const int64_t cap = (int64_t)a.max_pages << a.page_shift;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int ch = (int)(idx % chunks);
    int64_t rest = idx / chunks;
    const int g = (int)(rest % a.Hkv);
    rest /= a.Hkv;
    const int i = (int)(rest % a.Snew);
    const int b = (int)(rest / a.Snew);
    int64_t len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > cap ? cap : len);
    const int64_t t = len - a.Snew + i;
    if (t < 0) continue;
    int64_t krow, vrow;
    if (a.table != nullptr) {
      const int page = a.table[(int64_t)b * a.max_pages + (t >> a.page_shift)];
      if (page < 0 || page >= a.num_pages) continue;
      const int64_t slot = t & ((1 << a.page_shift) - 1);
      krow = (int64_t)page * a.kc_sb + slot * a.kc_ss;
      vrow = (int64_t)page * a.vc_sb + slot * a.vc_ss;
    } else {
      krow = (int64_t)b * a.kc_sb + t * a.kc_ss;
      vrow = (int64_t)b * a.vc_sb + t * a.vc_ss;
    }
    const int64_t e = 8 * ch;
    if (e < a.dk) {
      const u32x4 kw = *reinterpret_cast<const u32x4*>(a.kn + (int64_t)b * a.kn_sb + (int64_t)i * a.kn_ss +
                                                       (int64_t)g * a.kn_sh + e);
      *reinterpret_cast<u32x4*>(a.kc + krow + (int64_t)g * a.kc_sh + e) = kw;
    }
    if (e < a.dv) {
      const u32x4 vw = *reinterpret_cast<const u32x4*>(a.vn + (int64_t)b * a.vn_sb + (int64_t)i * a.vn_ss +
                                                       (int64_t)g * a.vn_sh + e);
      *reinterpret_cast<u32x4*>(a.vc + vrow + (int64_t)g * a.vc_sh + e) = vw;
    }
  }
}

// OCP e4m3 code of an fp32 value: nearest, ties to even, saturating at
// +-448, NaN -> 0x7f, sign kept (bit manipulation on the fp32 encoding).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0x7fu;                    // NaN
  if (mag >= 0x43e00000u) return sign | 0x7eu;            // |x| >= 448 (and inf)
  if (mag >= 0x3c800000u) {                               // |x| >= 2^-6: normal
    // round the 23-bit mantissa to 3 bits (to nearest, ties to even); a carry
    // moves into the exponent, and nothing below 448 rounds past 448
    const uint32_t r = (mag + 0x7ffffu + ((mag >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));                      // exponent bias 127 -> 7
  }
  // subnormal: |x| = m 2^-9 with m rounded to an integer in 0 .. 8 (8 is the
  // smallest normal, code 0x08)
  const float m = __builtin_rintf(__uint_as_float(mag) * 512.0f);
  return sign | (uint32_t)m;
}

struct AppendFp8Args {
  uint8_t* kc;
  uint8_t* vc;
  const uint16_t* kn;
  const uint16_t* vn;
  const float* ksc;
  const float* vsc;
  const int32_t* table;
  const int32_t* seq_lens;
  int64_t kc_sb, kc_ss, kc_sh, vc_sb, vc_ss, vc_sh;   // cache strides in bytes (= elements)
  int64_t kn_sb, kn_ss, kn_sh, vn_sb, vn_ss, vn_sh;   // new rows [B, Snew, Hkv, D] (bf16 elements)
  int B, Snew, Hkv, D, num_pages, page_shift, max_pages;
};

// One thread per 8 elements of the new rows; grid-stride. Each value is
// divided by its KV head's scale (fp32, rounded to nearest) and encoded;
// rows are placed as in append_kernel.
__global__ void __launch_bounds__(256) append_fp8_kernel(const AppendFp8Args a) {
  const int chunks = a.D / 8;
  const int64_t total = (int64_t)a.B * a.Snew * a.Hkv * chunks;
  const int64_t cap = (int64_t)a.max_pages << a.page_shift;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int ch = (int)(idx % chunks);
    int64_t rest = idx / chunks;
    const int g = (int)(rest % a.Hkv);
    rest /= a.Hkv;
    const int i = (int)(rest % a.Snew);
    const int b = (int)(rest / a.Snew);
    int64_t len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > cap ? cap : len);
    const int64_t t = len - a.Snew + i;
    if (t < 0) continue;
    int64_t krow, vrow;
    if (a.table != nullptr) {
      const int page = a.table[(int64_t)b * a.max_pages + (t >> a.page_shift)];
      if (page < 0 || page >= a.num_pages) continue;
      const int64_t slot = t & ((1 << a.page_shift) - 1);
      krow = (int64_t)page * a.kc_sb + slot * a.kc_ss;
      vrow = (int64_t)page * a.vc_sb + slot * a.vc_ss;
    } else {
      krow = (int64_t)b * a.kc_sb + t * a.kc_ss;
      vrow = (int64_t)b * a.vc_sb + t * a.vc_ss;
    }
    const int64_t e = 8 * ch;
    const float ks = a.ksc[g], vs = a.vsc[g];
    const u32x4 kw = *reinterpret_cast<const u32x4*>(a.kn + (int64_t)b * a.kn_sb + (int64_t)i * a.kn_ss +
                                                     (int64_t)g * a.kn_sh + e);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(a.vn + (int64_t)b * a.vn_sb + (int64_t)i * a.vn_ss +
                                                     (int64_t)g * a.vn_sh + e);
    u32x2 kq = {0u, 0u}, vq = {0u, 0u};
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const uint32_t kb16 = (kw[x >> 1] >> (16 * (x & 1))) & 0xffffu;
      const uint32_t vb16 = (vw[x >> 1] >> (16 * (x & 1))) & 0xffffu;
      const uint32_t kc8 = e4m3_code(__fdiv_rn(__uint_as_float(kb16 << 16), ks));
      const uint32_t vc8 = e4m3_code(__fdiv_rn(__uint_as_float(vb16 << 16), vs));
      kq[x >> 2] |= kc8 << (8 * (x & 3));
      vq[x >> 2] |= vc8 << (8 * (x & 3));
    }
    *reinterpret_cast<u32x2*>(a.kc + krow + (int64_t)g * a.kc_sh + e) = kq;
    *reinterpret_cast<u32x2*>(a.vc + vrow + (int64_t)g * a.vc_sh + e) = vq;
  }
}

}  // namespace

hipError_t launch_append_fp8(const AppendFp8Desc& d, hipStream_t stream) {
  AppendFp8Args a{static_cast<uint8_t*>(d.kcache), static_cast<uint8_t*>(d.vcache),
                  static_cast<const uint16_t*>(d.knew), static_cast<const uint16_t*>(d.vnew),
                  d.k_scale, d.v_scale, d.table, d.seq_lens,
                  d.kcs.outer, d.kcs.token, d.kcs.head, d.vcs.outer, d.vcs.token, d.vcs.head,
                  d.kns.outer, d.kns.token, d.kns.head, d.vns.outer, d.vns.token, d.vns.head,
                  d.B, d.Snew, d.Hkv, d.D, d.num_pages, d.page_shift, d.max_pages};
  const int64_t total = (int64_t)d.B * d.Snew * d.Hkv * (d.D / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(append_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendDesc& d, hipStream_t stream) {
  AppendArgs a{static_cast<uint16_t*>(d.kcache), static_cast<uint16_t*>(d.vcache),
               static_cast<const uint16_t*>(d.knew), static_cast<const uint16_t*>(d.vnew),
               d.table, d.seq_lens,
               d.kcs.outer, d.kcs.token, d.kcs.head, d.vcs.outer, d.vcs.token, d.vcs.head,
               d.kns.outer, d.kns.token, d.kns.head, d.vns.outer, d.vns.token, d.vns.head,
               d.B, d.Snew, d.Hkv, d.dk, d.dv, d.num_pages, d.page_shift, d.max_pages};
  const int64_t total = (int64_t)d.B * d.Snew * d.Hkv * (std::max(d.dk, d.dv) / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gqafa
