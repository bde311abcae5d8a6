// Paged K/V attention for gfx950: one split-K kernel that serves decode
// (q_len = 1) and speculative verification (q_len = k + 1, causal inside the
// window), with the cross-split log-sum-exp merge done by the last workgroup
// of each (sequence, KV head).
//
// Sources: ExLlamaV2 "Dynamic Generator" page, "Continuous Batching" (256-token
// pages reached through a per-sequence block table; indices need not be
// contiguous) and "Deduplication" (pages shared between sequences); Hugging
// Face "Assisted Generation" page, "How Assisted Generation works" (one pass
// scores every position of the draft window). The pages give no kernel
// design; everything below is this library's own.
//
// Work item = (sequence b, KV head g, split s of `pps` pages). A workgroup of
// kWaves waves takes one item; its waves interleave the split's token chunks,
// each wave with a private ring of LDS buffers filled by direct
// buffer->LDS loads (no VGPR staging) and its own online-softmax state. The
// waves merge in LDS; a single-split sequence writes `out` directly, otherwise
// the workgroup writes its partial (m, l, acc) and the last one to finish
// merges all splits of (b, g) in a fixed order, so results are deterministic.
//
// Row tiles. The q rows that share KV head g are the window rows times the
// head group (rows = q_len * Hq/Hkv):
//  * rows <= 12: VALU tile. Scores: one lane per (row group, token), bf16
//    pairs through v_dot2_f32_bf16 against a token row read from the
//    XOR-swizzled LDS tile; row maxima by DPP within 16-lane rows. P.V: one
//    lane per (token group, 8-dim chunk) in fp32 FMA, P read back from LDS.
//  * rows >= 13: MFMA tile (v_mfma_f32_32x32x16_bf16), rows padded to 32 or
//    64. S^T = K . Q^T puts one q row in each lane column, so the softmax
//    state and the rescale of O^T are per lane; O^T += V^T . P^T takes P from
//    registers (rounded to bf16) and V^T by 16-bit LDS reads.
//
// LDS tile layout: token t, 16-byte chunk c of its D-dim row sits at slot
// t * NC + (c ^ (t % NC)) (NC = D / 8), so a wave reading one token row per
// lane hits distinct banks; the swizzle is applied on the global side of the
// direct loads, which stay fully coalesced per 1 KiB instruction.

#include "internal.h"

namespace pkv {
namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef PKV_VALU_NBUF
#define PKV_VALU_NBUF 2  // LDS ring depth (chunks) per wave, VALU row tile
#endif
#ifndef PKV_MFMA_NBUF
#define PKV_MFMA_NBUF 2  // LDS ring depth (chunks) per wave, MFMA row tile
#endif
#ifndef PKV_FORCE_PPS
#define PKV_FORCE_PPS 0  // pages per split; 0 = planned per shape
#endif

constexpr int kWaves = 4;
constexpr int kNumCu = 256;           // MI355X compute units
constexpr int kLdsPerCu = 160 * 1024;  // gfx950 LDS per CU
constexpr int kThreads = kWaves * 64;
constexpr float kNegInf = -__builtin_inff();

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
// write of an operand SGPR needs before a VMEM read; m0 holds the LDS address.
__device__ __forceinline__ void dma16(u32x4 rsrc, u32 voff, u32 lds_addr) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory");
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

__device__ __forceinline__ u32 lds_addr_of(const void* p) {
  return static_cast<u32>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Sum of q_lens[0..b) by one wave.
__device__ __forceinline__ int wave_prefix(const int32_t* q_lens, int b) {
  const int lane = threadIdx.x & 63;
  int s = 0;
  for (int i = lane; i < b; i += 64) s += q_lens[i];
  for (int m = 32; m >= 1; m >>= 1) s += __builtin_amdgcn_ds_bpermute(((lane ^ m) << 2), s);
  return s;
}

// ----------------------------------------------------------------- row tiles

// Geometry shared by both row tiles.
template <int D, int TC>
struct TileGeom {
  static constexpr int NC = D / 8;                 // 16-byte chunks per token row
  static constexpr int RB = D * 2;                 // bytes per token row
  static constexpr int NI = TC * NC / 64;          // 1 KiB load instructions per tile
  static constexpr int TILE = TC * RB;             // bytes of one K (or V) chunk
  static_assert(TC * NC % 64 == 0, "chunk must fill whole load instructions");
};

// VALU row tile: rows = 4 * RPL (RPL q rows per lane in the score phase).
template <int D, int RPL>
struct ValuTile {
  static constexpr int TC = 16;
  static constexpr int NC = D / 8;
  static constexpr int TG = 64 / NC;  // token groups in the P.V phase
  static constexpr int RP = 4 * RPL;  // padded rows
  static constexpr int STEPS = TC / TG;
  static constexpr int PBUF = TC * RP * 4;  // P staging bytes per wave

  u32 q[RPL][D / 2];
  float m[RPL], l[RPL];
  int lim[RPL];
  float acc[RP][8];

  __device__ __forceinline__ void init(const uint16_t* qbase, int Hq, int group, int g, int rows,
                                       int q_start, int seq_len, int q_len) {
    const int lane = threadIdx.x & 63;
    const int rg = lane >> 4;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const int r = rg + 4 * j;
      m[j] = kNegInf;
      l[j] = 0.f;
      if (r < rows) {
        const int w = r / group, h = g * group + r % group;
        lim[j] = seq_len - q_len + w;
        const u32x4* src = reinterpret_cast<const u32x4*>(qbase + ((size_t)(q_start + w) * Hq + h) * D);
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
          u32x4 v = src[c];
          q[j][4 * c + 0] = v.x;
          q[j][4 * c + 1] = v.y;
          q[j][4 * c + 2] = v.z;
          q[j][4 * c + 3] = v.w;
        }
      } else {
        lim[j] = -1;
#pragma unroll
        for (int c = 0; c < D / 2; ++c) q[j][c] = 0u;
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  // One chunk of TC tokens starting at absolute token tok0; nv of them are
  // inside the sequence. kt / vt: LDS tiles; pb: this wave's P staging.
  __device__ __forceinline__ void step(const char* kt, const char* vt, float* pb, int tok0, int nv,
                                       float scale_log2) {
    const int lane = threadIdx.x & 63;
    const int rg = lane >> 4, t = lane & 15;
    const u32x4* kl = reinterpret_cast<const u32x4*>(kt);
    // the whole token row first, so the LDS reads overlap each other
    u32x4 kv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) kv[c] = kl[t * NC + (c ^ (t & (NC - 1)))];
    float s[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) s[j] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int j = 0; j < RPL; ++j) {
        s[j] = dot2(q[j][4 * c + 0], kv[c].x, s[j]);
        s[j] = dot2(q[j][4 * c + 1], kv[c].y, s[j]);
        s[j] = dot2(q[j][4 * c + 2], kv[c].z, s[j]);
        s[j] = dot2(q[j][4 * c + 3], kv[c].w, s[j]);
      }
    }
    const int tok = tok0 + t;
    float alpha[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const float x = (tok <= lim[j] && t < nv) ? s[j] * scale_log2 : kNegInf;
      const float mn = fmaxf(m[j], row16_max(x));
      const float mu = (mn == kNegInf) ? 0.f : mn;
      alpha[j] = exp2f_fast(m[j] - mu);
      const float p = exp2f_fast(x - mu);
      l[j] = l[j] * alpha[j] + p;
      m[j] = mn;
      pb[t * RP + rg + 4 * j] = p;
    }
    // rescale the accumulators of every row by its alpha
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[j]), g4 * 16));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g4 + 4 * j][e] *= a;
      }
    }
    // P.V
    const int tg = lane / NC, dc = lane % NC;
    const u32x4* vl = reinterpret_cast<const u32x4*>(vt);
    const f32x4* pl = reinterpret_cast<const f32x4*>(pb);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int tt = st * TG + tg;
      u32x4 vv = vl[tt * NC + (dc ^ (tt & (NC - 1)))];
      if (tt >= nv) vv = u32x4{0u, 0u, 0u, 0u};
      float v8[8] = {bf16lo(vv.x), bf16hi(vv.x), bf16lo(vv.y), bf16hi(vv.y),
                     bf16lo(vv.z), bf16hi(vv.z), bf16lo(vv.w), bf16hi(vv.w)};
#pragma unroll
      for (int r4 = 0; r4 < RP / 4; ++r4) {
        const f32x4 pp = pl[tt * (RP / 4) + r4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[4 * r4 + 0][e] = __builtin_fmaf(pp.x, v8[e], acc[4 * r4 + 0][e]);
          acc[4 * r4 + 1][e] = __builtin_fmaf(pp.y, v8[e], acc[4 * r4 + 1][e]);
          acc[4 * r4 + 2][e] = __builtin_fmaf(pp.z, v8[e], acc[4 * r4 + 2][e]);
          acc[4 * r4 + 3][e] = __builtin_fmaf(pp.w, v8[e], acc[4 * r4 + 3][e]);
        }
      }
    }
  }

  // Write this wave's (m, l, acc) for rows < RP into the merge area.
  __device__ __forceinline__ void spill(float* rm, float* rl, float* racc) {
    const int lane = threadIdx.x & 63;
    const int rg = lane >> 4, t = lane & 15;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const float ls = row16_sum(l[j]);
      if (t == 0) {
        rm[rg + 4 * j] = m[j];
        rl[rg + 4 * j] = ls;
      }
    }
    // sum the token groups (lanes dc, dc + NC, ...)
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int msk = NC; msk < 64; msk <<= 1) acc[r][e] += shfl_xor(acc[r][e], msk);
    if (lane < NC) {
#pragma unroll
      for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) racc[r * D + lane * 8 + e] = acc[r][e];
    }
  }
};

// MFMA row tile: rows padded to 32 * NRB.
template <int D, int NRB>
struct MfmaTile {
  static constexpr int TC = 32;
  static constexpr int NC = D / 8;
  static constexpr int KK = D / 16;  // k-steps of the score product
  static constexpr int MB = D / 32;  // 32-dim blocks of the output
  static constexpr int RP = 32 * NRB;
  static constexpr int PBUF = 0;

  u32x4 qb[NRB][KK];
  float m[NRB], l[NRB];
  int lim[NRB];
  f32x16 acc[NRB][MB];

  __device__ __forceinline__ void init(const uint16_t* qbase, int Hq, int group, int g, int rows,
                                       int q_start, int seq_len, int q_len) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + row;
      m[rb] = kNegInf;
      l[rb] = 0.f;
      if (r < rows) {
        const int w = r / group, h = g * group + r % group;
        lim[rb] = seq_len - q_len + w;
        const uint16_t* src = qbase + ((size_t)(q_start + w) * Hq + h) * D + half * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qb[rb][kk] = *reinterpret_cast<const u32x4*>(src + kk * 16);
      } else {
        lim[rb] = -1;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qb[rb][kk] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb][mb][i] = 0.f;
    }
  }

  __device__ __forceinline__ void step(const char* kt, const char* vt, float*, int tok0, int nv,
                                       float scale_log2) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 31, half = lane >> 5;
    const u32x4* kl = reinterpret_cast<const u32x4*>(kt);
    f32x16 S[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[rb][i] = 0.f;
    // S^T[token][q row] = sum_d K[token][d] * Q[q row][d]
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int c = 2 * kk + half;
      const u32x4 a = kl[row * NC + (c ^ (row & (NC - 1)))];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        S[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, qb[rb][kk]), S[rb], 0, 0,
                                                        0);
    }
    // this lane holds tokens 8*(i/4) + 4*half + i%4 of q row `row`
    u32x4 pb[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float x[16];
      float cm = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tt = 8 * (i >> 2) + 4 * half + (i & 3);
        x[i] = (tok0 + tt <= lim[rb] && tt < nv) ? S[rb][i] * scale_log2 : kNegInf;
        cm = fmaxf(cm, x[i]);
      }
      cm = fmaxf(cm, shfl_xor(cm, 32));
      const float mn = fmaxf(m[rb], cm);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float alpha = exp2f_fast(m[rb] - mu);
      float ps = 0.f;
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = exp2f_fast(x[i] - mu);
        ps += p[i];
      }
      l[rb] = l[rb] * alpha + ps;
      m[rb] = mn;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[rb][mb] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pb[rb][ks].x = pack_bf16(p[8 * ks + 0], p[8 * ks + 1]);
        pb[rb][ks].y = pack_bf16(p[8 * ks + 2], p[8 * ks + 3]);
        pb[rb][ks].z = pack_bf16(p[8 * ks + 4], p[8 * ks + 5]);
        pb[rb][ks].w = pack_bf16(p[8 * ks + 6], p[8 * ks + 7]);
      }
    }
    // O^T[d][q row] += sum_token V[token][d] * P[q row][token]; k index j of
    // lane half h at k-step ks is token 16*ks + 8*(j/4) + 4*h + j%4.
    const uint16_t* vl = reinterpret_cast<const uint16_t*>(vt);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int d = mb * 32 + row;
      const int dch = d >> 3, dw = d & 7;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32 w4[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u32 lohi[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int j = 2 * jj + z;
            const int tt = 16 * ks + 8 * (j >> 2) + 4 * half + (j & 3);
            u32 v = vl[(tt * NC + (dch ^ (tt & (NC - 1)))) * 8 + dw];
            lohi[z] = (tt < nv) ? v : 0u;
          }
          w4[jj] = lohi[0] | (lohi[1] << 16);
        }
        const u32x4 a = {w4[0], w4[1], w4[2], w4[3]};
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                __builtin_bit_cast(bf16x8, pb[rb][ks]),
                                                                acc[rb][mb], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void spill(float* rm, float* rl, float* racc) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + row;
      const float ls = l[rb] + shfl_xor(l[rb], 32);
      if (half == 0) {
        rm[r] = m[rb];
        rl[r] = ls;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          racc[r * D + d] = acc[rb][mb][i];
        }
    }
  }
};

// ------------------------------------------------------------------- kernel

template <int D, class Tile, int NBUF>
struct KernelCfg {
  static constexpr int TC = Tile::TC;
  using G = TileGeom<D, TC>;
  static constexpr int RING = NBUF * 2 * G::TILE;        // per wave: K and V tiles
  static constexpr int STAGE = kWaves * (RING + Tile::PBUF);
  static constexpr int MERGE = kWaves * Tile::RP * (D + 2) * 4;
  static constexpr int SMEM = STAGE > MERGE ? STAGE : MERGE;
  static constexpr int MAX_PPS = 64;
};

template <int D, class Tile, int NBUF>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(AttnParams p) {
  using C = KernelCfg<D, Tile, NBUF>;
  using G = typename C::G;
  constexpr int TC = C::TC;
  constexpr int NI = G::NI;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_pages[C::MAX_PPS];
  __shared__ int s_last;

  // XCD-aware item order: consecutive logical items (the same split and KV
  // head over consecutive sequences, which share prefix pages under dedup)
  // land on the same XCD and its L2.
  const int per_xcd = (p.num_items + kNumXcd - 1) / kNumXcd;
  const int item = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
  if (item >= p.num_items) return;
  const int b = item % p.B;
  const int rest = item / p.B;
  const int g = rest % p.Hkv;
  const int s = rest / p.Hkv;

  const int seq_len = p.seq_lens[b];
  const int q_len = p.q_lens[b];
  if (q_len <= 0) return;
  const int n_pages = (seq_len + kPage - 1) / kPage;
  const int n_splits = (n_pages + p.pps - 1) / p.pps;
  if (q_len > p.max_q_len || q_len > seq_len || n_pages > p.W) {
    if (s == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, 2u);
    return;
  }
  if (s >= n_splits) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q_start = __builtin_amdgcn_readfirstlane(wave_prefix(p.q_lens, b));
  if (q_start + q_len > p.total_q) {
    if (s == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, 4u);
    return;
  }

  const int page0 = s * p.pps;
  const int npg = min(p.pps, n_pages - page0);
  if (threadIdx.x < npg) {
    int pg = p.block_table[(size_t)b * p.W + page0 + threadIdx.x];
    if (pg < 0 || pg >= p.P) {
      atomicOr(p.err, 1u);
      pg = -1;
    }
    s_pages[threadIdx.x] = pg;
  }
  __syncthreads();

  const int tok_begin = page0 * kPage;
  const int tok_end = min(seq_len, (page0 + npg) * kPage);
  const int n_chunks = (tok_end - tok_begin + TC - 1) / TC;
  const int my_chunks = n_chunks > wave ? (n_chunks - wave + kWaves - 1) / kWaves : 0;

  char* ring = smem + wave * C::RING;
  float* pbuf = reinterpret_cast<float*>(smem + kWaves * C::RING + wave * Tile::PBUF);
  const u32 ring_lds = lds_addr_of(ring);

  // per-lane byte offsets of the direct loads (the chunk base goes into the
  // descriptor, so they are the same for every chunk)
  u32 voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = i * 64 + lane;
    const int t = slot / G::NC, pos = slot % G::NC;
    voff[i] = t * G::RB + ((pos ^ (t & (G::NC - 1))) * 16);
  }

  const size_t head_stride = (size_t)kPage * D;  // elements per (page, head) tile
  auto issue = [&](int k) {
    const int c = wave + k * kWaves;
    const int t0 = tok_begin + c * TC;
    const int jp = t0 / kPage - page0;
    const int in_page = t0 % kPage;
    const int phys = __builtin_amdgcn_readfirstlane(s_pages[jp]);
    const int page_valid = min(kPage, seq_len - (page0 + jp) * kPage);
    int nvt = min(TC, page_valid - in_page);
    if (phys < 0) nvt = 0;
    const size_t off = ((size_t)(phys < 0 ? 0 : phys) * p.Hkv + g) * head_stride + (size_t)in_page * D;
    const u32 bytes = nvt > 0 ? (u32)(nvt * G::RB) : 0u;
    const u32x4 rk = make_rsrc(p.k_pool + off, bytes);
    const u32x4 rv = make_rsrc(p.v_pool + off, bytes);
    const u32 base = uniform(ring_lds + (k % NBUF) * 2 * G::TILE);
    wait_lgkm0();
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(rk, voff[i], base + i * 1024);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(rv, voff[i], base + G::TILE + i * 1024);
  };

  // rows of this sequence: window rows times the head group (<= Tile::RP)
  Tile tile;
  tile.init(p.q, p.Hq, p.group, g, q_len * p.group, q_start, seq_len, q_len);
  // Retire every compiler-visible load now (q rows, table entries): the
  // waitcnt pass then has nothing outstanding to wait for inside the loop,
  // where its waits would also drain the direct-to-LDS prefetches.
  __builtin_amdgcn_s_waitcnt(0);

#pragma unroll
  for (int k = 0; k < NBUF - 1; ++k)
    if (k < my_chunks) issue(k);

  for (int k = 0; k < my_chunks; ++k) {
    if (k + NBUF - 1 < my_chunks) issue(k + NBUF - 1);
    const int ahead = min(NBUF - 1, my_chunks - 1 - k);
    if constexpr (NBUF >= 4) {
      if (ahead >= 3) wait_vmcnt<3 * 2 * NI>();
      else if (ahead == 2) wait_vmcnt<2 * 2 * NI>();
      else if (ahead == 1) wait_vmcnt<2 * NI>();
      else wait_vmcnt<0>();
    } else if constexpr (NBUF == 3) {
      if (ahead >= 2) wait_vmcnt<2 * 2 * NI>();
      else if (ahead == 1) wait_vmcnt<2 * NI>();
      else wait_vmcnt<0>();
    } else {
      if (ahead >= 1) wait_vmcnt<2 * NI>();
      else wait_vmcnt<0>();
    }
    const int c = wave + k * kWaves;
    const int t0 = tok_begin + c * TC;
    const char* kt = ring + (k % NBUF) * 2 * G::TILE;
    tile.step(kt, kt + G::TILE, pbuf, t0, min(TC, tok_end - t0), p.scale_log2);
  }

  // ---- merge the waves in LDS
  __syncthreads();
  constexpr int RP = Tile::RP;
  float* red_m = reinterpret_cast<float*>(smem);
  float* red_l = red_m + kWaves * RP;
  float* red_acc = red_l + kWaves * RP;
  tile.spill(red_m + wave * RP, red_l + wave * RP, red_acc + (size_t)wave * RP * D);
  __syncthreads();

  const int rows = min(p.rows_max, RP);
  const int it = (b * p.Hkv + g) * p.max_splits + s;
  for (int e = threadIdx.x; e < rows * D; e += kThreads) {
    const int r = e / D, d = e % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w * RP + r]);
    float L = 0.f, A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = red_m[w * RP + r];
        const float wt = (mw == kNegInf) ? 0.f : exp2f_fast(mw - M);
        L += wt * red_l[w * RP + r];
        A += wt * red_acc[((size_t)w * RP + r) * D + d];
      }
    }
    const int wpos = r / p.group;
    if (wpos >= q_len) continue;
    if (n_splits == 1) {
      const int h = g * p.group + r % p.group;
      p.out[((size_t)(q_start + wpos) * p.Hq + h) * D + d] = A / L;
    } else {
      st_coherent(&p.part_acc[((size_t)it * p.rows_max + r) * D + d], A);
      if (d == 0) {
        st_coherent(&p.part_ml[((size_t)it * p.rows_max + r) * 2 + 0], M);
        st_coherent(&p.part_ml[((size_t)it * p.rows_max + r) * 2 + 1], L);
      }
    }
  }
  if (n_splits == 1) return;

  // ---- last workgroup of (b, g) merges every split in split order. Every
  // thread's partial stores are acknowledged (vmcnt 0) before the barrier,
  // so they are visible device-wide before thread 0 bumps the counter.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const u32 prev = __hip_atomic_fetch_add(p.counters + (b * p.Hkv + g), 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (u32)(n_splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  const int it0 = (b * p.Hkv + g) * p.max_splits;
  const int qrows = min(rows, q_len * p.group);
  for (int e = threadIdx.x; e < qrows * D; e += kThreads) {
    const int r = e / D, d = e % D;
    float M = kNegInf;
    for (int sp = 0; sp < n_splits; ++sp)
      M = fmaxf(M, ld_coherent(&p.part_ml[((size_t)(it0 + sp) * p.rows_max + r) * 2]));
    float L = 0.f, A = 0.f;
    for (int sp = 0; sp < n_splits; ++sp) {
      const size_t base = (size_t)(it0 + sp) * p.rows_max + r;
      const float ms = ld_coherent(&p.part_ml[base * 2]);
      const float wt = (ms == kNegInf) ? 0.f : exp2f_fast(ms - M);
      L += wt * ld_coherent(&p.part_ml[base * 2 + 1]);
      A += wt * ld_coherent(&p.part_acc[base * D + d]);
    }
    const int wpos = r / p.group, h = g * p.group + r % p.group;
    p.out[((size_t)(q_start + wpos) * p.Hq + h) * D + d] = A / L;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(p.counters + (b * p.Hkv + g), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, class Tile, int NBUF>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  const int per_xcd = (p.num_items + kNumXcd - 1) / kNumXcd;
  const int grid = per_xcd * kNumXcd;
  hipLaunchKernelGGL((attn_split_kernel<D, Tile, NBUF>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, const AttnPlan& plan, hipStream_t stream) {
  if (!plan.mfma) {
    const int rpl = (plan.rows + 3) / 4;
    switch (rpl) {
      case 1: return launch_one<D, ValuTile<D, 1>, PKV_VALU_NBUF>(p, stream);
      case 2: return launch_one<D, ValuTile<D, 2>, PKV_VALU_NBUF>(p, stream);
      default: return launch_one<D, ValuTile<D, 3>, PKV_VALU_NBUF>(p, stream);
    }
  }
  if (plan.rows <= 32) return launch_one<D, MfmaTile<D, 1>, PKV_MFMA_NBUF>(p, stream);
  return launch_one<D, MfmaTile<D, 2>, PKV_MFMA_NBUF>(p, stream);
}

}  // namespace

AttnPlan attn_plan(int B, int Hkv, int W, int max_q_len, int group) {
  AttnPlan pl;
  pl.rows = max_q_len * group;
  pl.mfma = pl.rows > 12;
  // Workgroups resident per CU, from the LDS each variant claims.
  int smem;
  if (pl.mfma)
    smem = pl.rows <= 32 ? KernelCfg<128, MfmaTile<128, 1>, PKV_MFMA_NBUF>::SMEM
                         : KernelCfg<128, MfmaTile<128, 2>, PKV_MFMA_NBUF>::SMEM;
  else
    smem = KernelCfg<128, ValuTile<128, 3>, PKV_VALU_NBUF>::SMEM;
  int per_cu = kLdsPerCu / smem;
  if (per_cu < 1) per_cu = 1;
  // Pages per split: as few splits as keep one round of workgroups on every
  // CU. Each extra split costs a partial write and read plus a merge; an
  // idle CU costs more. The table width bounds every sequence's pages.
  const long tiles = (long)B * Hkv * W;
  const long slots = (long)kNumCu * per_cu;
  long pps = (tiles + slots - 1) / slots;
  if (PKV_FORCE_PPS > 0) pps = PKV_FORCE_PPS;
  if (pps < 1) pps = 1;
  if (pps > W) pps = W;
  if (pps > 64) pps = 64;  // the kernel stages at most 64 table entries per split
  pl.pps = (int)pps;
  pl.max_splits = (W + pl.pps - 1) / pl.pps;
  return pl;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

AttnWorkspace attn_workspace(int B, int Hkv, int W, int max_q_len, int group, int D) {
  const AttnPlan pl = attn_plan(B, Hkv, W, max_q_len, group);
  AttnWorkspace ws;
  const size_t items = (size_t)B * Hkv * pl.max_splits;
  ws.err_off = 0;
  ws.counters_off = 256;
  ws.ml_off = align_up(ws.counters_off + (size_t)B * Hkv * 4, 256);
  ws.acc_off = align_up(ws.ml_off + items * pl.rows * 2 * 4, 256);
  ws.total = align_up(ws.acc_off + items * pl.rows * (size_t)D * 4, 256);
  return ws;
}

hipError_t launch_attn(const AttnParams& p, const AttnPlan& plan, hipStream_t stream) {
  if (p.num_items == 0) return hipSuccess;
  if (p.D == 64) return launch_d<64>(p, plan, stream);
  return launch_d<128>(p, plan, stream);
}

}  // namespace pkv
