// Device helpers shared by the attention kernels: buffer descriptors, direct
// buffer->LDS loads with hand-counted waits, wavefront reductions (DPP and
// cross-half swaps), bf16 packing, and the window-row prefix sum.
#pragma once

#include "internal.h"

#include "pkv.h"

namespace pkv {
namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

#ifndef PKV_VALU_NBUF
#define PKV_VALU_NBUF 2  // LDS ring depth (chunks) per wave, VALU row tile
#endif
#ifndef PKV_VALU_Q8_NBUF
#define PKV_VALU_Q8_NBUF 2  // LDS ring depth (chunks) per wave, VALU row tile over a Q8 cache
#endif
#ifndef PKV_VALU_Q4_NBUF
#define PKV_VALU_Q4_NBUF 4  // LDS ring depth (chunks) per wave, VALU row tile over a Q4 cache
#endif
#ifndef PKV_MFMA_NBUF
#define PKV_MFMA_NBUF 2  // LDS ring depth (chunks) per wave, MFMA row tile
#endif
#ifndef PKV_VALU_WAVES
#define PKV_VALU_WAVES 4  // waves per workgroup, VALU row tile
#endif
#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4  // waves per workgroup, MFMA row tile
#endif
#ifndef PKV_PREFILL_NBUF
#define PKV_PREFILL_NBUF 8  // K/V chunks in the ring shared by a prefill workgroup
#endif
#ifndef PKV_SHARED_WG
#define PKV_SHARED_WG kNumCu  // workgroups the shared-prefix kernel aims for
#endif
#ifndef PKV_SHARED_ROW_TILE
#define PKV_SHARED_ROW_TILE 1  // shared-prefix keys of few-row batches on the decode / verify row tile
#endif
#ifndef PKV_FORCE_PPS
#define PKV_FORCE_PPS 0  // pages per split; 0 = planned per shape
#endif

constexpr u32 PKV_EFLAG_PAGE_BIT = 1u, PKV_EFLAG_QLEN_BIT = 2u, PKV_EFLAG_ROWS_BIT = 4u;
constexpr int kNumCu = 256;           // MI355X compute units
#ifndef PKV_VALU_MAX_ROWS
#define PKV_VALU_MAX_ROWS 4
#endif
constexpr int kValuMaxRows = PKV_VALU_MAX_ROWS;  // q rows per (sequence, KV head) on the VALU tile
constexpr int kLdsPerCu = 160 * 1024;  // gfx950 LDS per CU
constexpr float kNegInf = -__builtin_inff();
// Quantized caches: what a token's staged K/V values must be multiplied by,
// besides its scale, to give the cached values (Q4 stages 16 x code; the
// factor is exact while the scale is at least 2^-122).
template <int QB>
constexpr float kStageFactor = QB == 4 ? 0.0625f : 1.f;

__device__ __forceinline__ u32 uniform(u32 x) { return __builtin_amdgcn_readfirstlane(x); }

// Raw buffer descriptor: 48-bit base, stride 0, num_records bytes. Reads at
// offsets >= num_records return zero and never fault.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, u32 bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r.x = uniform(static_cast<u32>(a));
  r.y = uniform(static_cast<u32>(a >> 32));
  r.z = uniform(bytes);
  r.w = 0x00020000u;
  return r;
}

// One 16-byte-per-lane load from the buffer straight into LDS: lane i's 16
// bytes land at lds_addr + 16 * i. The s_nop covers the wait states a VALU
// write of an operand SGPR needs before a VMEM read; m0 holds the LDS address
// (declared clobbered, so the compiler keeps nothing of its own in m0 across).
__device__ __forceinline__ void dma16(u32x4 rsrc, u32 voff, u32 lds_addr) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory", "m0");
}

// One 4-byte-per-lane load straight into LDS: lane i's word lands at
// lds_addr + 4 * i.
__device__ __forceinline__ void dma4(u32x4 rsrc, u32 voff, u32 lds_addr) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max / sum over the 16 lanes of a DPP row; every lane gets the result.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) {
  const int lane = threadIdx.x & 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __float_as_int(x)));
}

// Reductions across the two 32-lane halves in one VALU instruction, without
// an LDS round trip: v_permlane32_swap exchanges the upper 32 lanes of its
// first operand with the lower 32 of its second, so with x in both every lane
// holds {x of this lane, x of lane ^ 32} (lane layout checked on the GPU).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Split partials cross XCDs (each XCD has its own L2). Agent-scope relaxed
// atomic stores/loads are write-through / coherent by themselves, so the
// partials need no L2-wide write-back or invalidate.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf16lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(u32 w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float dot2(u32 a, u32 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

__device__ __forceinline__ u32 pack_bf16(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(u32, v);
}

// Signed byte B of w as a float: one sign-extending SDWA convert (left to
// itself the compiler sometimes shifts and bit-extracts every byte first).
template <int B>
__device__ __forceinline__ float sbyte_f32(u32 w) {
  static_assert(B >= 0 && B < 4, "byte index");
  float r;
  if constexpr (B == 0)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w));
  else if constexpr (B == 1)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
  else if constexpr (B == 2)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
  else
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}

// The four signed bytes of w as two bf16 pairs (bytes 0, 1 and 2, 3); exact
// for bytes in [-128, 127].
__device__ __forceinline__ void sbytes_bf16(u32 w, u32& lo, u32& hi) {
  lo = pack_bf16(sbyte_f32<0>(w), sbyte_f32<1>(w));
  hi = pack_bf16(sbyte_f32<2>(w), sbyte_f32<3>(w));
}

__device__ __forceinline__ u32 lds_addr_of(const void* p) {
  return static_cast<u32>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Window-row bookkeeping of sequence b, by one wave over q_lens[0..B): the
// first row of b (the sum of q_lens[0..b)), the sum over the whole batch,
// and whether a length before b is negative (then b's first row means
// nothing and b is skipped; that sequence's own item flags it).
struct RowPrefix {
  int start, total;
  bool bad_before;
};
__device__ __forceinline__ RowPrefix row_prefix(const int32_t* q_lens, int b, int B) {
  const int lane = threadIdx.x & 63;
  int pre = 0, tot = 0, neg = 0;
  for (int i = lane; i < B; i += 64) {
    const int v = q_lens[i];
    tot += v;
    if (i < b) {
      pre += v;
      neg |= v < 0;
    }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    pre += __builtin_amdgcn_ds_bpermute(((lane ^ m) << 2), pre);
    tot += __builtin_amdgcn_ds_bpermute(((lane ^ m) << 2), tot);
    neg |= __builtin_amdgcn_ds_bpermute(((lane ^ m) << 2), neg);
  }
  return {(int)__builtin_amdgcn_readfirstlane(pre), (int)__builtin_amdgcn_readfirstlane(tot),
          __builtin_amdgcn_readfirstlane(neg) != 0};
}

constexpr int kSc1 = 16;  // cache-policy bit: coherent across XCDs (write-through / miss)

// s_waitcnt immediate for vmcnt(0) alone (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 at their maxima)
constexpr int kVmcnt0 = 0x0F70;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, u32 bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Wait until at most `ahead` (0..MAXA) chunks of N load ops each are pending.
template <int N, int MAXA>
__device__ __forceinline__ void wait_ahead(int ahead) {
  static_assert(MAXA <= 5 && MAXA * N < 64, "vmcnt range");
  if constexpr (MAXA >= 5) {
    if (ahead >= 5) { wait_vmcnt<5 * N>(); return; }
  }
  if constexpr (MAXA >= 4) {
    if (ahead >= 4) { wait_vmcnt<4 * N>(); return; }
  }
  if constexpr (MAXA >= 3) {
    if (ahead >= 3) { wait_vmcnt<3 * N>(); return; }
  }
  if constexpr (MAXA >= 2) {
    if (ahead >= 2) { wait_vmcnt<2 * N>(); return; }
  }
  if (ahead >= 1) wait_vmcnt<N>();
  else wait_vmcnt<0>();
}

// Geometry of a K (or V) chunk of TC tokens in LDS.
template <int D, int TC>
struct TileGeom {
  static constexpr int NC = D / 8;                 // 16-byte chunks per token row
  static constexpr int RB = D * 2;                 // bytes per token row
  static constexpr int NI = TC * NC / 64;          // 1 KiB load instructions per tile
  static constexpr int TILE = TC * RB;             // bytes of one K (or V) chunk
  static_assert(TC * NC % 64 == 0, "chunk must fill whole load instructions");
};

}  // namespace
}  // namespace pkv
