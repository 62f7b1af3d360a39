// Device helpers for the gfx950 (CDNA4) attention kernels: MFMA operand
// types, lane exchanges, bf16 packing, LDS reads and copies, and the paged
// KV-cache address rule shared by the split-KV kernel and the paged-gather
// test hook.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqafa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The online softmax moves its reference max only when a row's max grows by
// more than this many powers of two (P then stays below 2^8).
constexpr float kRescaleLog2 = 8.0f;
// the same bound on a sum of weights (2^kRescaleLog2)
constexpr float kRescaleSum = 256.0f;

// D[32x32] += A[32x16] * B[16x32], bf16 inputs, fp32 accumulators. Lane l
// supplies row (l % 32) of A and column (l % 32) of B, eight consecutive K
// slots each; the lane halves (l / 32) hold the two halves of the 16 K slots.
// Both operands use the same K-slot assignment, so the contraction is the
// plain sum over the 16 K positions whatever order the unit walks them in.
// The result layout: acc[4 * r + e] of lane l is D[8 r + 4 (l / 32) + e][l % 32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Reductions over the two lanes 32 apart (l and l ^ 32), via
// v_permlane32_swap. With x in both operands, the swap leaves lanes 0-31 with
// (own, partner) and lanes 32-63 with (partner, own) in its two results, so
// the max and the sum of the two results are the pair's max and sum in every
// lane; the sum is formed in the same order (lower lane first) in both
// halves, so the pair holds bit-identical values.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 values -> packed bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Low or high 16-bit halves of two words, packed (x half in the low 16 bits).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4). The LDS
// destination `lds_seg` must be the same for the whole wave: lane L's 16 bytes
// land at lds_seg + 16 L bytes. STREAM sets the non-temporal hint (nt): data
// read once (a decode step's KV cache) streams past the caches; measured on
// MI355X, it is what lets these copies approach HBM bandwidth (without it a
// pure copy stream stalls near 4.7 TB/s).
template <bool STREAM>
__device__ __forceinline__ void dma16(const uint16_t* gsrc, uint16_t* lds_seg) {
  constexpr int kNonTemporal = 2;
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_seg, 16, 0,
                                   STREAM ? kNonTemporal : 0);
}

// The same copy through a buffer resource: 16 bytes from base + voffset
// (this lane's byte offset) into this lane's 16 bytes of the LDS segment.
// After a copy in the global (flat-encoded) form the compiler treats every
// LDS read as possibly out of order and makes each use wait for all of
// them (lgkmcnt 0); after the buffer form its LDS waits stay graded, so
// operand reads issued ahead of their MFMAs stay in flight. Range checking
// is off (the copies stay in range by construction); descriptor word 3 is
// the gfx9-family default.
template <bool STREAM>
__device__ __forceinline__ void dma16_buf(const void* base, uint32_t voffset, uint16_t* lds_seg) {
  constexpr int kNonTemporal = 2;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_seg, 16,
                                           voffset, 0, 0, STREAM ? kNonTemporal : 0);
}

// The same with a uniform byte offset (soffset) added to every lane's: the
// row part of a copy's source offset, kept on the scalar unit.
template <bool STREAM>
__device__ __forceinline__ void dma16_buf_s(const void* base, uint32_t voffset, uint32_t soffset,
                                            uint16_t* lds_seg) {
  constexpr int kNonTemporal = 2;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_seg, 16,
                                           voffset, soffset, 0, STREAM ? kNonTemporal : 0);
}

// Scheduling hints (sched_group_barrier masks: 0x2 VALU, 0x8 MFMA, 0x100
// DS read). One pipeline step: N1 MFMAs that each consume R1 LDS reads and
// may hide V1 VALU instructions, then N2 MFMAs consuming R2 reads each. The
// reads run AHEAD reads in front of their MFMAs.
template <int N, int R, int AHEAD, int V, int I>
__device__ __forceinline__ void sched_phase() {
  if constexpr (I < N) {
    constexpr int total = N * R;
    constexpr int lo = I * R + AHEAD < total ? I * R + AHEAD : total;
    constexpr int hi = (I + 1) * R + AHEAD < total ? (I + 1) * R + AHEAD : total;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (hi > lo) __builtin_amdgcn_sched_group_barrier(0x100, hi - lo, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    sched_phase<N, R, AHEAD, V, I + 1>();
  }
}
// As sched_phase, with one vector memory instruction (a tile copy) placed
// after MFMA number C1 and one after MFMA number C2.
template <int N, int R, int AHEAD, int C1, int C2, int I>
__device__ __forceinline__ void sched_phase_copies() {
  if constexpr (I < N) {
    constexpr int total = N * R;
    constexpr int lo = I * R + AHEAD < total ? I * R + AHEAD : total;
    constexpr int hi = (I + 1) * R + AHEAD < total ? (I + 1) * R + AHEAD : total;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (hi > lo) __builtin_amdgcn_sched_group_barrier(0x100, hi - lo, 0);
    if constexpr (I == C1 || I == C2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    sched_phase_copies<N, R, AHEAD, C1, C2, I + 1>();
  }
}
// One continuous operand-read stream over both phases of a step: N1 MFMAs
// that consume R1 LDS reads each (hiding V1 VALU instructions each), then
// N2 MFMAs consuming R2 reads each, with the reads AHEAD in front of their
// MFMAs across the phase boundary (the second phase's first reads go out
// beside the first phase's last MFMAs instead of after them), and one
// vector memory instruction after MFMAs C1 and C2. The caller issues the
// first AHEAD reads.
template <int N1, int R1, int N2, int R2, int AHEAD, int V1, int C1, int C2, int I>
__device__ __forceinline__ void sched_cont() {
  if constexpr (I < N1 + N2) {
    constexpr int total = N1 * R1 + N2 * R2;
    constexpr int used = I < N1 ? (I + 1) * R1 : N1 * R1 + (I + 1 - N1) * R2;
    constexpr int used_prev = I == 0 ? 0 : (I - 1 < N1 ? I * R1 : N1 * R1 + (I - N1) * R2);
    constexpr int lo = used_prev + AHEAD < total ? used_prev + AHEAD : total;
    constexpr int hi = used + AHEAD < total ? used + AHEAD : total;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (hi > lo) __builtin_amdgcn_sched_group_barrier(0x100, hi - lo, 0);
    if constexpr (I < N1 && V1 > 0) __builtin_amdgcn_sched_group_barrier(0x002, V1, 0);
    if constexpr (I == C1 || I == C2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    sched_cont<N1, R1, N2, R2, AHEAD, V1, C1, C2, I + 1>();
  }
}
template <int N1, int R1, int N2, int R2, int AHEAD, int V1>
__device__ __forceinline__ void sched_step() {
  constexpr int a1 = AHEAD < N1 * R1 ? AHEAD : N1 * R1;
  __builtin_amdgcn_sched_group_barrier(0x100, a1, 0);
  sched_phase<N1, R1, a1, V1, 0>();
  constexpr int a2 = AHEAD < N2 * R2 ? AHEAD : N2 * R2;
  __builtin_amdgcn_sched_group_barrier(0x100, a2, 0);
  sched_phase<N2, R2, a2, 0, 0>();
}

// Wait until at most N of this wave's global loads (including global -> LDS
// copies, which complete in issue order) are outstanding: s_waitcnt vmcnt(N).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt is six bits");
  constexpr int imm = (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Wait until every LDS (and scalar-memory) access of this wave has completed:
// s_waitcnt lgkmcnt(0), leaving vmcnt and expcnt at their maxima.
__device__ __forceinline__ void wait_lgkm0() {
  constexpr int imm = 15 | (7 << 4) | (0 << 8) | (3 << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Workgroup barrier for handing LDS over between the waves of these kernels:
// the wave's own LDS reads and writes are complete (lgkmcnt 0), the compiler
// moves no memory access across it, and every wave arrives. It does not wait
// for global loads, stores or global -> LDS copies: the waves never read
// each other's global writes, and each barrier that hands over a copied tile
// follows an explicit wait for that tile's copies. A fenced barrier
// (__syncthreads, or a release fence on LDS) would wait for every copy in
// flight, since copies into LDS count as LDS writes.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// Holds a value in VGPRs at this point of the program: the value must be
// computed before it, and code after it sees the pinned copy. With it, pure
// arithmetic (exponentials, MFMAs) cannot be moved across the barrier that
// follows by the compiler, which orders only memory accesses around one.
template <typename T>
__device__ __forceinline__ void pin_vgpr(T& x) {
  asm volatile("" : "+v"(x));
}

// Transposing LDS read of four 16-bit values (ds_read_b64_tr_b16). Within
// each group of 16 lanes, lane i receives element i % 4 of the 8-byte rows
// addressed by lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 (in that
// order).
__device__ __forceinline__ u32x2 read_tr16(const uint16_t* lds) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lds);
  return __builtin_bit_cast(u32x2, v);
}

// Transposing LDS read of eight 8-bit values (ds_read_b64_tr_b8). Within
// each group of 16 lanes, lane i receives byte i % 8 of the 8-byte rows
// addressed by lanes i / 8, i / 8 + 2, ..., i / 8 + 14 (in that order) of the
// group (measured on gfx950).
__device__ __forceinline__ u32x2 read_tr8(const unsigned char* lds) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)lds);
  return __builtin_bit_cast(u32x2, v);
}

// Eight OCP e4m3 (fp8) values, byte k of w = element k, as eight bf16 in the
// same order: gfx950's v_cvt_scalef32_pk_bf16_fp8 widens two codes of one
// half of a dword straight to a bf16 pair (value times the scale, here 1;
// every e4m3 value is exact in bf16), four instructions per eight values
// where widening to fp32 and packing took eight. A GPU test decodes every
// finite code through both the K and the V path.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[h], 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[h], 1.0f, true);
    r[2 * h] = __builtin_bit_cast(uint32_t, lo);
    r[2 * h + 1] = __builtin_bit_cast(uint32_t, hi);
  }
  return r;
}

// Paged KV caches [num_pages, page_size, Hkv, D]: the address rule of the
// split-KV kernel, shared with the paged-gather hook (fa_paged_gather), so
// that the hook's byte-exact test pins the decode path's own arithmetic.
// A block-table entry outside [0, num_pages) is clamped into range (every
// load stays inside the cache; a sequence with such an entry covering its
// tokens gets unspecified output).
__device__ __forceinline__ int clamp_page(int page, int num_pages) { return min(max(page, 0), num_pages - 1); }

// Element offset of slot `slot` of (clamped) page `page`, given the page and
// token strides of the cache (head offset not included). 64-bit arithmetic.
__device__ __forceinline__ int64_t paged_row(int page, int slot, int64_t page_stride, int64_t token_stride) {
  return (int64_t)page * page_stride + (int64_t)slot * token_stride;
}

}  // namespace gqafa
