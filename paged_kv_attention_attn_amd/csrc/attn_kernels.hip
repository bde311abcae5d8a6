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
//  * rows <= 4 (decode with a head group of up to 4): VALU tile. Scores: one
//    lane per (row group, token), bf16 pairs through v_dot2_f32_bf16 against
//    a token row read from the XOR-swizzled LDS tile; row maxima by DPP
//    within 16-lane rows. P.V: one lane per (token group, 8-dim chunk) in
//    fp32 FMA, P read back from LDS.
//  * rows >= 5: MFMA tile (v_mfma_f32_32x32x16_bf16), rows padded to 32 or
//    64. S^T = K . Q^T puts one q row in each lane column, so the softmax
//    state and the rescale of O^T are per lane; O^T += V^T . P^T takes P from
//    registers (rounded to bf16) and V^T by 16-bit LDS reads.
//
// LDS tile layout: token t, 16-byte chunk c of its D-dim row sits at slot
// t * NC + (c ^ (t % NC)) (NC = D / 8), so a wave reading one token row per
// lane hits distinct banks; the swizzle is applied on the global side of the
// direct loads, which stay fully coalesced per 1 KiB instruction.

#include "device.h"

#include <type_traits>

namespace pkv {
namespace {

// ----------------------------------------------------------------- row tiles

// VALU row tile: rows = 4 * RPL (RPL q rows per lane in the score phase);
// launched with RPL = 1, where it beats the matrix cores (8 and 12 rows run
// faster on the MFMA tile).
template <int D, int RPL>
struct ValuTile {
  static constexpr int TC = 16;
  static constexpr int NC = D / 8;
  static constexpr int TG = 64 / NC;  // token groups in the P.V phase
  static constexpr int RP = 4 * RPL;  // padded rows
  static constexpr int STEPS = TC / TG;
  static constexpr int PBUF = TC * RP * 4;  // P staging bytes per wave
  static constexpr int MS = D;              // row stride (floats) of the waves' merge area
  static constexpr bool kVDirect = true;    // quantized caches: V converted straight from its codes
  static constexpr float kSplitWeight = 1.f / 8.f;  // the MFMA tile's two-term threshold
  static constexpr float kLazyLog2 = 8.f;           // reference-max slack, as on the long-window tile

  u32 q[RPL][D / 2];
  float m[RPL], l[RPL];
  float mu[RPL];  // m, or 0 while m is -inf (the exponent's offset)
  int lim[RPL];
  float acc[RP][8];
  u32x4 kv[NC];      // this lane's token row of the current K chunk
  u32x4 vv[STEPS];   // this lane's V pieces of the current chunk

  __device__ __forceinline__ void init(int group, int rows, int seq_len, int q_len) {
    const int rg = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const int r = rg + 4 * j;
      m[j] = kNegInf;
      mu[j] = 0.f;
      l[j] = 0.f;
      lim[j] = r < rows ? seq_len - q_len + r / group : -1;
    }
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  // q rows from the swizzled LDS copy (rows past the window are zero there)
  __device__ __forceinline__ void load_q(const char* qlds) {
    const int rg = (threadIdx.x & 63) >> 4;
    const u32x4* ql = reinterpret_cast<const u32x4*>(qlds);
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const int r = rg + 4 * j;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 v = ql[r * NC + (c ^ (r & (NC - 1)))];
        q[j][4 * c + 0] = v.x;
        q[j][4 * c + 1] = v.y;
        q[j][4 * c + 2] = v.z;
        q[j][4 * c + 3] = v.w;
      }
    }
  }

  // One chunk of TC tokens starting at absolute token tok0; nv of them are
  // inside the sequence. kt / vt: LDS tiles; pb: this wave's P staging.
  // Copy one chunk's operands out of its LDS slot (so the slot can be
  // refilled while this chunk is computed): this lane's token row of K and
  // its 8-dim pieces of V (rows past the sequence zeroed).
  __device__ __forceinline__ void fetch(const char* kt, const char* vt, int nv) {
    const int lane = threadIdx.x & 63;
    const int t = lane & 15;
    const u32x4* kl = reinterpret_cast<const u32x4*>(kt);
#pragma unroll
    for (int c = 0; c < NC; ++c) kv[c] = kl[t * NC + (c ^ (t & (NC - 1)))];
    const int tg = lane / NC, dc = lane % NC;
    const u32x4* vl = reinterpret_cast<const u32x4*>(vt);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int tt = st * TG + tg;
      vv[st] = vl[tt * NC + (dc ^ (tt & (NC - 1)))];
      if (tt >= nv) vv[st] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Quantized caches: this lane's K row from the slot's staged bf16 K tile
  // (as fetch), and its V pieces converted straight from the slot's codes
  // (vc: token-major, D * QB / 8 bytes per token; each V code is read and
  // converted once, by the lane whose P.V piece it is): Q8, one
  // sign-extending byte convert per code; Q4, 16 * code per byte as in
  // q_decode_slot. The converts pair the two tokens of each P.V step per dim
  // (vv[2 sp] holds dims 0..3 as (tA, tB) bf16 pairs, vv[2 sp + 1] dims
  // 4..7), the layout compute() would otherwise build with shifts and masks.
  // Tokens past the sequence end need no mask: their codes and scales were
  // loaded as zeros, so their weights P * V scale are zero and their V
  // values finite (a zero Q4 byte stages as 16 * -8).
  template <int QB>
  __device__ __forceinline__ void fetch_q(const char* kt, const char* vc) {
    const int lane = threadIdx.x & 63;
    const int t = lane & 15;
    const u32x4* kl = reinterpret_cast<const u32x4*>(kt);
#pragma unroll
    for (int c = 0; c < NC; ++c) kv[c] = kl[t * NC + (c ^ (t & (NC - 1)))];
    const int tg = lane / NC, dc = lane % NC;
    constexpr int TB = D * QB / 8;  // code bytes per token
    static_assert(STEPS % 2 == 0, "token pairs");
#pragma unroll
    for (int sp = 0; sp < STEPS / 2; ++sp) {
      const int tA = 2 * sp * TG + tg, tB = tA + TG;
      float a[8], b[8];
      if constexpr (QB == 8) {
        const u32x2 wa = *reinterpret_cast<const u32x2*>(vc + tA * TB + dc * 8);
        const u32x2 wb = *reinterpret_cast<const u32x2*>(vc + tB * TB + dc * 8);
        a[0] = sbyte_f32<0>(wa.x), a[1] = sbyte_f32<1>(wa.x), a[2] = sbyte_f32<2>(wa.x), a[3] = sbyte_f32<3>(wa.x);
        a[4] = sbyte_f32<0>(wa.y), a[5] = sbyte_f32<1>(wa.y), a[6] = sbyte_f32<2>(wa.y), a[7] = sbyte_f32<3>(wa.y);
        b[0] = sbyte_f32<0>(wb.x), b[1] = sbyte_f32<1>(wb.x), b[2] = sbyte_f32<2>(wb.x), b[3] = sbyte_f32<3>(wb.x);
        b[4] = sbyte_f32<0>(wb.y), b[5] = sbyte_f32<1>(wb.y), b[6] = sbyte_f32<2>(wb.y), b[7] = sbyte_f32<3>(wb.y);
      } else {
        const u32 wa = *reinterpret_cast<const u32*>(vc + tA * TB + dc * 4);
        const u32 wb = *reinterpret_cast<const u32*>(vc + tB * TB + dc * 4);
        // dim 2i in the low nibble of byte i
        const u32 la = ((wa << 4) & 0xF0F0F0F0u) ^ 0x80808080u, ha = (wa & 0xF0F0F0F0u) ^ 0x80808080u;
        const u32 lb = ((wb << 4) & 0xF0F0F0F0u) ^ 0x80808080u, hb = (wb & 0xF0F0F0F0u) ^ 0x80808080u;
        a[0] = sbyte_f32<0>(la), a[1] = sbyte_f32<0>(ha), a[2] = sbyte_f32<1>(la), a[3] = sbyte_f32<1>(ha);
        a[4] = sbyte_f32<2>(la), a[5] = sbyte_f32<2>(ha), a[6] = sbyte_f32<3>(la), a[7] = sbyte_f32<3>(ha);
        b[0] = sbyte_f32<0>(lb), b[1] = sbyte_f32<0>(hb), b[2] = sbyte_f32<1>(lb), b[3] = sbyte_f32<1>(hb);
        b[4] = sbyte_f32<2>(lb), b[5] = sbyte_f32<2>(hb), b[6] = sbyte_f32<3>(lb), b[7] = sbyte_f32<3>(hb);
      }
      vv[2 * sp] = u32x4{pack_bf16(a[0], b[0]), pack_bf16(a[1], b[1]), pack_bf16(a[2], b[2]), pack_bf16(a[3], b[3])};
      vv[2 * sp + 1] =
          u32x4{pack_bf16(a[4], b[4]), pack_bf16(a[5], b[5]), pack_bf16(a[6], b[6]), pack_bf16(a[7], b[7])};
    }
  }

  // One chunk of TC tokens starting at absolute token tok0 (nv of them
  // inside the sequence), from the operands fetch() copied. Quantized caches
  // (QB != 0): the staged operands are codes, and qsc holds the chunk's K
  // scales (words 0..) and V scales (words 64..): token t's score is scaled
  // by its K scale, its weight P by its V scale (the row sum keeps plain P).
  // (MAYMASK is accepted for the kernel's sake; this tile always masks)
  template <int QB = 0, bool MAYMASK = true>
  __device__ __forceinline__ void compute(float* pb, int tok0, int nv, float scale_log2, const float* qsc) {
    const int lane = threadIdx.x & 63;
    const int rg = lane >> 4, t = lane & 15;
    float ksl = scale_log2, vsc = 1.f;
    if constexpr (QB != 0) {
      ksl = qsc[t] * (scale_log2 * kStageFactor<QB>);
      vsc = qsc[64 + t] * kStageFactor<QB>;
    }
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
    // Lazy rescale: a row keeps its reference max m while the chunk's scores
    // stay below m + kLazyLog2, so P = 2^(x - m) may reach 2^kLazyLog2 and the
    // weights' ratios are unchanged; only a row that outgrows it moves m and
    // rescales its sum and accumulators (rare after the first chunks, and
    // then the whole wave skips the accumulator pass). m is uniform over a
    // row's 16 lanes, so a lane's own score decides whether its row grows;
    // the row maximum is taken only then.
    float x[RPL];
    bool grow = false;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      x[j] = (tok <= lim[j] && t < nv) ? s[j] * ksl : kNegInf;
      grow |= x[j] > m[j] + kLazyLog2;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
      float alpha[RPL];
#pragma unroll
      for (int j = 0; j < RPL; ++j) {
        const float cm = row16_max(x[j]);
        const bool g = cm > m[j] + kLazyLog2;
        alpha[j] = g ? exp2f_fast(m[j] - cm) : 1.f;  // 0 while m is -inf
        m[j] = g ? cm : m[j];
        mu[j] = (m[j] == kNegInf) ? 0.f : m[j];
        l[j] *= alpha[j];
      }
#pragma unroll
      for (int j = 0; j < RPL; ++j) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[j]), g4 * 16));
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g4 + 4 * j][e] *= a;
        }
      }
    }
    bool heavy = false;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const float p = exp2f_fast(x[j] - mu[j]);
      l[j] += p;
      pb[t * RP + rg + 4 * j] = QB != 0 ? p * vsc : p;
      // a key of this chunk weighing more than kSplitWeight of its row's sum
      // so far (the row's 16 lanes): its bf16 P would not average out
      heavy |= p > kSplitWeight * row16_sum(l[j]);
    }
    const bool split = __builtin_amdgcn_ballot_w64(heavy) != 0;
    // P.V on bf16 pairs: tokens tA = 2*sp*TG + tg and tB = tA + TG are
    // interleaved per dim, P is rounded to bf16 (as on the MFMA path), and
    // one v_dot2 per (row, dim) takes both tokens. On chunks with a heavy
    // key P enters as two bf16 terms (the rounding remainder in a second
    // v_dot2), about 16 significant bits.
    const int tg = lane / NC;
    const f32x4* pl = reinterpret_cast<const f32x4*>(pb);
    static_assert(STEPS % 2 == 0, "token pairs");
#pragma unroll
    for (int sp = 0; sp < STEPS / 2; ++sp) {
      const int tA = 2 * sp * TG + tg, tB = tA + TG;
      const u32x4 wa = vv[2 * sp], wb = vv[2 * sp + 1];
      u32 vp[8];  // (V[tA][d], V[tB][d]) for the lane's 8 dims
      if constexpr (QB != 0) {  // fetch_q converted them in this order
        vp[0] = wa.x, vp[1] = wa.y, vp[2] = wa.z, vp[3] = wa.w;
        vp[4] = wb.x, vp[5] = wb.y, vp[6] = wb.z, vp[7] = wb.w;
      } else {
        const u32 va4[4] = {wa.x, wa.y, wa.z, wa.w}, vb4[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          vp[2 * k] = (va4[k] & 0xFFFFu) | (vb4[k] << 16);
          vp[2 * k + 1] = (va4[k] >> 16) | (vb4[k] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int r4 = 0; r4 < RP / 4; ++r4) {
        const f32x4 pa = pl[tA * (RP / 4) + r4], pc = pl[tB * (RP / 4) + r4];
        const u32 pp[4] = {pack_bf16(pa.x, pc.x), pack_bf16(pa.y, pc.y), pack_bf16(pa.z, pc.z),
                           pack_bf16(pa.w, pc.w)};
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[4 * r4 + rr][e] = dot2(pp[rr], vp[e], acc[4 * r4 + rr][e]);
        if (split) {
          const float pf[4][2] = {{pa.x, pc.x}, {pa.y, pc.y}, {pa.z, pc.z}, {pa.w, pc.w}};
          u32 pq[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            pq[rr] = pack_bf16(pf[rr][0] - bf16lo(pp[rr]), pf[rr][1] - bf16hi(pp[rr]));
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[4 * r4 + rr][e] = dot2(pq[rr], vp[e], acc[4 * r4 + rr][e]);
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
        for (int msk = NC; msk < 64; msk <<= 1)
          acc[r][e] = msk == 32 ? sum_xor32(acc[r][e]) : acc[r][e] + shfl_xor(acc[r][e], msk);
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
  // row stride (floats) of the waves' merge area: one row per lane, so a
  // stride of D would put every lane of a store on the same bank; 4 more
  // floats move each row by four banks
  static constexpr int MS = D + 4;
  static constexpr bool kVDirect = false;  // quantized caches: V staged as bf16 like K

  u32x4 qb[NRB][KK];
  float m[NRB], l[NRB];
  int lim[NRB];
  f32x16 acc[NRB][MB];
  u32x4 ka[KK];      // K operand of the current chunk
  u32x4 va[MB][2];   // V^T operands of the current chunk

  __device__ __forceinline__ void init(int group, int rows, int seq_len, int q_len) {
    const int row = threadIdx.x & 31;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + row;
      m[rb] = kNegInf;
      l[rb] = 0.f;
      lim[rb] = r < rows ? seq_len - q_len + r / group : -1;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb][mb][i] = 0.f;
    }
  }

  // Rows row0 .. row0 + 32 * NRB of a longer row set, where row r is window
  // token r / group and rows outside [r_lo, r_hi) are padding: row r sees
  // keys 0 .. lim_base + r / group.
  __device__ __forceinline__ void init_rows(int row0, int group, int lim_base, int r_lo, int r_hi) {
    const int row = threadIdx.x & 31;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = row0 + rb * 32 + row;
      m[rb] = kNegInf;
      l[rb] = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) lacc[rb][i] = 0.f;
      lim[rb] = (r >= r_lo && r < r_hi) ? lim_base + r / group : -1;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb][mb][i] = 0.f;
    }
  }

  __device__ __forceinline__ void load_q(const char* qlds) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 31, half = lane >> 5;
    const u32x4* ql = reinterpret_cast<const u32x4*>(qlds);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + row;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int c = 2 * kk + half;
        qb[rb][kk] = ql[r * NC + (c ^ (r & (NC - 1)))];
      }
    }
  }

  // Copy one chunk's MFMA operands out of its LDS slot: the K rows as the
  // A operand of S^T, and V^T as the A operand of O^T, where k index j of
  // lane half h at k-step ks is token 16*ks + 8*(j/4) + 4*h + j%4 (matching
  // where P sits in the S^T result).
  //
  // V^T comes from transposing LDS reads (ds_read_b64_tr_b16). Within each
  // 16-lane group, source lane j names 4 consecutive bf16 of one tile row and
  // destination lane i receives element i%4 of source lanes i/4, i/4 + 4,
  // i/4 + 8 and i/4 + 12. With source lane j at token t0 + j/4 and dims
  // d0 + 4*(j%4) .. + 3, lane i gets tokens t0 .. t0 + 3 of dim d0 + i. Rows
  // past the sequence end were zero-filled by the chunk load, so no mask.
  __device__ __forceinline__ void fetch_k(const char* kt) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 31, half = lane >> 5;
    const u32x4* kl = reinterpret_cast<const u32x4*>(kt);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int c = 2 * kk + half;
      ka[kk] = kl[row * NC + (c ^ (row & (NC - 1)))];
    }
  }

  __device__ __forceinline__ void fetch_v(const char* vt) {
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int tq = (lane & 15) >> 2;                         // token within the 4-token group
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // dims within the 32-dim block
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int d = mb * 32 + dsub;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x2 w[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int t = 16 * ks + 8 * hh + 4 * half + tq;
          const char* src = vt + (t * NC + ((d >> 3) ^ (t & (NC - 1)))) * 16 + (d & 7) * 2;
          w[hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src));
        }
        va[mb][ks] = u32x4{w[0].x, w[0].y, w[1].x, w[1].y};
      }
    }
  }

  __device__ __forceinline__ void fetch(const char* kt, const char* vt, int) {
    fetch_k(kt);
    fetch_v(vt);
  }

  // Quantized caches (QB != 0): as the VALU tile's compute, with the K scale
  // on each score and the V scale on each weight of P.V (rows' sums keep
  // plain P).
  // MAYMASK false: every chunk is whole and seen in full by every row (the
  // shared-prefix rows), so no mask code at all
  template <int QB = 0, bool MAYMASK = true>
  __device__ __forceinline__ void compute(float*, int tok0, int nv, float scale_log2, const float* qsc) {
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    f32x16 S[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[rb][i] = 0.f;
    // S^T[token][q row] = sum_d K[token][d] * Q[q row][d], row block by row
    // block, so the first block's softmax can run beside the next block's
    // products
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        S[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[kk]),
                                                        __builtin_bit_cast(bf16x8, qb[rb][kk]), S[rb], 0, 0,
                                                        0);
    // this lane holds tokens 8*(i/4) + 4*half + i%4 of q row `row`
    u32x4 pb[NRB][2];
    float p[NRB][16];
    float x[NRB][16], cm[NRB];
    // a row sees the chunk's tokens 0 .. thr[rb]; the mask is skipped when
    // every row of the wave sees the whole chunk (padding rows, lim < 0,
    // hold scores of a zero q row and are never read)
    int thr[NRB];
    bool partial = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      thr[rb] = min(lim[rb] - tok0, nv - 1);
      partial |= lim[rb] >= 0 && thr[rb] < TC - 1;
    }
    const bool masked = MAYMASK && __builtin_amdgcn_ballot_w64(partial) != 0;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tt = 8 * (i >> 2) + 4 * half + (i & 3);
        const float ksl = QB != 0 ? qsc[tt] * (scale_log2 * kStageFactor<QB>) : scale_log2;
        x[rb][i] = S[rb][i] * ksl;
      }
    if (masked) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tt = 8 * (i >> 2) + 4 * half + (i & 3);
          if (tt > thr[rb]) x[rb][i] = kNegInf;
        }
    }
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      cm[rb] = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) cm[rb] = fmaxf(cm[rb], x[rb][i]);
      cm[rb] = max_xor32(cm[rb]);
      grow |= cm[rb] > m[rb] + kLazyLog2;
    }
    // Lazy rescale: a row keeps its reference max m while the chunk stays
    // below m + kLazyLog2, so P = 2^(x - m) may reach 2^kLazyLog2 and the
    // softmax ratio is unchanged; only a row that outgrows it moves m and
    // rescales its sum and O^T (rare after the first chunk).
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // O^T stays in the accumulation registers: read, multiply and write
      // back each element in place (a plain multiply would make the compiler
      // keep a VALU-side copy of O^T across the chunk loop). The s_nop runs
      // cover the matrix-core result latency before the first read and the
      // write-to-operand latency after the last write.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const bool gr = cm[rb] > m[rb] + kLazyLog2;
        const float alpha = gr ? exp2f_fast(m[rb] - cm[rb]) : 1.f;
        m[rb] = gr ? cm[rb] : m[rb];
        l[rb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float v = acc[rb][mb][i], t;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(v), "=&v"(t)
                : "v"(alpha));
            acc[rb][mb][i] = v;
          }
      }
      asm volatile("s_nop 3" ::: "memory");
    }
    bool heavy = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mu = (m[rb] == kNegInf) ? 0.f : m[rb];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[rb][i] = exp2f_fast(x[rb][i] - mu);
        ps += p[rb][i];
      }
      l[rb] += ps;
      // a key of this chunk weighing more than kSplitWeight of its row's sum
      // so far (both halves of the row): its bf16 P would not average out
      // (evaluated without a branch: exp2 of -inf is 0)
      heavy |= (cm[rb] != kNegInf) & (exp2f_fast(cm[rb] - mu) > kSplitWeight * sum_xor32(l[rb]));
      if constexpr (QB != 0) {  // P.V weights carry the V scales
#pragma unroll
        for (int i = 0; i < 16; ++i) p[rb][i] *= qsc[64 + 8 * (i >> 2) + 4 * half + (i & 3)] * kStageFactor<QB>;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pb[rb][ks].x = pack_bf16(p[rb][8 * ks + 0], p[rb][8 * ks + 1]);
        pb[rb][ks].y = pack_bf16(p[rb][8 * ks + 2], p[rb][8 * ks + 3]);
        pb[rb][ks].z = pack_bf16(p[rb][8 * ks + 4], p[rb][8 * ks + 5]);
        pb[rb][ks].w = pack_bf16(p[rb][8 * ks + 6], p[rb][8 * ks + 7]);
      }
    }
    // O^T[d][q row] += sum_token V[token][d] * P[q row][token]
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          acc[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mb][ks]),
                                                                __builtin_bit_cast(bf16x8, pb[rb][ks]),
                                                                acc[rb][mb], 0, 0, 0);
    // rows dominated by a few keys: P enters as two bf16 terms (the rounding
    // remainder in a second pass), about 16 significant bits
    if (__builtin_amdgcn_ballot_w64(heavy)) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32 lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32 h = pb[rb][ks][e];
            lo[e] = pack_bf16(p[rb][8 * ks + 2 * e] - bf16lo(h), p[rb][8 * ks + 2 * e + 1] - bf16hi(h));
          }
          pb[rb][ks] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mb][ks]),
                                                                  __builtin_bit_cast(bf16x8, pb[rb][ks]),
                                                                  acc[rb][mb], 0, 0, 0);
    }
  }

  // Long-window variant of compute (query tiles that see thousands of keys),
  // in steps the caller can interleave across chunks:
  //  * qk(): S^T on matrix cores; scores(): S^T scaled (and masked unless
  //    MASK is false, for chunks every row of the wave sees in full) into xs,
  //    and the chunk's row maxima into cmax. Lazy rescale: a row keeps its reference
  //    max m while the chunk stays below m + kLazyLog2, so P = 2^(x - m) may
  //    reach 2^kLazyLog2 and the softmax ratio is unchanged; scores() returns
  //    whether some row of the wave outgrew that;
  //  * rescale(): moves those rows' m and rescales their l and O^T;
  //  * probs(): P, packed to bf16; pv(): O^T += V^T . P^T and the row sums.
  //    SPLIT_P: P enters as two bf16 terms (its rounding and the remainder),
  //    about 16 significant bits instead of 8, for rows that see so few keys
  //    that nothing averages the rounding out.
  static constexpr float kLazyLog2 = 8.f;
  float xs[NRB][16], cmax[NRB];
  // Row sums on the matrix cores: an all-ones block in place of V^T, so each
  // row's sum is taken over the same bf16 P that multiplies V and the output
  // is an exact weighted mean of the rounded weights (every element of
  // lacc[rb] holds the sum of the lane's row).
  f32x16 lacc[NRB];

  // S^T of the current K operand for every row block.
  __device__ __forceinline__ void qk(f32x16* S) const {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[rb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        S[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[kk]),
                                                        __builtin_bit_cast(bf16x8, qb[rb][kk]), S[rb], 0, 0,
                                                        0);
    }
  }

  template <bool MASK>
  __device__ __forceinline__ bool scores(const f32x16* S, int tok0, int nv, float scale_log2) {
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float cm = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tt = 8 * (i >> 2) + 4 * half + (i & 3);
        if constexpr (MASK)
          xs[rb][i] = (tok0 + tt <= lim[rb] && tt < nv) ? S[rb][i] : kNegInf;
        else
          xs[rb][i] = S[rb][i];
        // one read out of the accumulation registers serves the max here and
        // the exponentials of the next step
        asm volatile("" : "+v"(xs[rb][i]));
        cm = fmaxf(cm, xs[rb][i]);
      }
      // scale_log2 > 0 here, so scaling commutes with the max
      cmax[rb] = max_xor32(cm) * scale_log2;
      grow |= cmax[rb] > m[rb] + kLazyLog2;
    }
    return __builtin_amdgcn_ballot_w64(grow) != 0;
  }

  // O^T lives in the accumulation registers; the rescale multiplies it in
  // place there (read, multiply, write back per element), so the compiler
  // never needs a VALU-side copy of it in the chunk loop. The s_nop runs
  // cover the matrix-core result latency before the first read and the
  // write-to-operand latency after the last write.
  __device__ __forceinline__ void rescale() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const bool g = cmax[rb] > m[rb] + kLazyLog2;
      const float alpha = g ? exp2f_fast(m[rb] - cmax[rb]) : 1.f;
      m[rb] = g ? cmax[rb] : m[rb];
      {
        // every element of lacc[rb] holds the row sum and only element 0 is
        // read, so only it is rescaled (the others are never used)
        float x = lacc[rb][0], t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(x), "=&v"(t)
            : "v"(alpha));
        lacc[rb][0] = x;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = acc[rb][mb][i], t;
          asm volatile(
              "v_accvgpr_read_b32 %1, %0\n\t"
              "v_mul_f32 %1, %1, %2\n\t"
              "v_accvgpr_write_b32 %0, %1"
              : "+a"(x), "=&v"(t)
              : "v"(alpha));
          acc[rb][mb][i] = x;
        }
    }
    asm volatile("s_nop 3" ::: "memory");
  }

  // Whether the current chunk needs P in two bf16 terms: some row of the
  // wave has a key whose weight, against the row sum so far, exceeds
  // kSplitWeight. A key's final weight can only be lower than that, so with a
  // single bf16 P no key weighs more than kSplitWeight when rounded.
  static constexpr float kSplitWeight = 1.f / 8.f;
  __device__ __forceinline__ bool needs_split() const {
    bool any = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mu = (m[rb] == kNegInf) ? 0.f : m[rb];
      float ls;  // the row sum, read straight out of its accumulation register
      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(ls) : "a"(lacc[rb][0]));
      any |= exp2f_fast(cmax[rb] - mu) > kSplitWeight * ls;
    }
    return __builtin_amdgcn_ballot_w64(any) != 0;
  }

  // P of the current scores, packed to bf16 operand pairs (and the rounding
  // remainders under SPLIT_P).
  u32x4 pb[NRB][2], pl[NRB][2];
  template <bool SPLIT_P>
  __device__ __forceinline__ void probs(float scale_log2) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mu = (m[rb] == kNegInf) ? 0.f : m[rb];
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = exp2f_fast(__builtin_fmaf(xs[rb][i], scale_log2, -mu));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32 h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = pack_bf16(p[8 * ks + 2 * e], p[8 * ks + 2 * e + 1]);
        pb[rb][ks] = u32x4{h[0], h[1], h[2], h[3]};
        if constexpr (SPLIT_P) {
          u32 lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lo[e] = pack_bf16(p[8 * ks + 2 * e] - bf16lo(h[e]), p[8 * ks + 2 * e + 1] - bf16hi(h[e]));
          pl[rb][ks] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        }
      }
    }
  }

  // O^T += V^T . P^T and the row sums, from probs() and the current V operand.
  template <bool SPLIT_P>
  __device__ __forceinline__ void pv() {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          acc[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mb][ks]),
                                                                __builtin_bit_cast(bf16x8, pb[rb][ks]),
                                                                acc[rb][mb], 0, 0, 0);
          if constexpr (SPLIT_P)
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mb][ks]),
                                                                  __builtin_bit_cast(bf16x8, pl[rb][ks]),
                                                                  acc[rb][mb], 0, 0, 0);
        }
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        lacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ones),
                                                           __builtin_bit_cast(bf16x8, pb[rb][ks]), lacc[rb], 0, 0,
                                                           0);
        if constexpr (SPLIT_P)
          lacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ones),
                                                             __builtin_bit_cast(bf16x8, pl[rb][ks]), lacc[rb], 0,
                                                             0, 0);
      }
  }

  __device__ __forceinline__ void spill(float* rm, float* rl, float* racc) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + row;
      const float ls = sum_xor32(l[rb]);
      if (half == 0) {
        rm[r] = m[rb];
        rl[r] = ls;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = mb * 32 + 8 * j + 4 * half;
          *reinterpret_cast<f32x4*>(racc + r * MS + d) =
              f32x4{acc[rb][mb][4 * j], acc[rb][mb][4 * j + 1], acc[rb][mb][4 * j + 2], acc[rb][mb][4 * j + 3]};
        }
    }
  }
};

// ------------------------------------------------------------------- kernel

// Quantized caches (QBITS = 8: int8 codes; 4: two 4-bit codes per byte): a
// ring slot holds a chunk's K and V codes (TC x D x QBITS / 8 bytes each,
// token-major as in the pool, in whole 1 KiB load areas) and their per-token
// scales (a 256-byte area each, filled by one 4-byte load per lane); the wave
// decodes the slot's codes into a bf16 K/V pair in the layout of a bf16
// slot, its staging area (followed by the scales), which the row tiles read
// as they read a bf16 slot, applying the scales to scores and weights.
template <int D, class Tile, int NBUF, int WAVES, int QBITS = 0>
struct KernelCfg {
  static constexpr int W = WAVES;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int TC = Tile::TC;
  using G = TileGeom<D, TC>;
  static constexpr int QTILE = TC * D * QBITS / 8;          // code bytes of one K (or V) chunk
  static constexpr int QAREA = (QTILE + 1023) / 1024 * 1024;  // its load area (tail read as zeros)
  static constexpr int NCI = QAREA / 1024;               // 1 KiB code loads per K (or V) chunk
  static constexpr int SLOT = QBITS ? 2 * QAREA + 512 : 2 * G::TILE;
  static constexpr int OPS = QBITS ? 2 * NCI + 2 : 2 * G::NI;  // load instructions per chunk
  // staging: the bf16 K tile (and V tile unless the row tile converts V
  // straight from its codes), then the chunk's scales
  static constexpr bool VDIRECT = QBITS != 0 && Tile::kVDirect;
  static constexpr int STG_TILES = VDIRECT ? 1 : 2;
  static constexpr int RING = NBUF * SLOT + (QBITS ? STG_TILES * G::TILE + 512 : 0);  // per wave (+ staging)
  static constexpr int QB = (Tile::RP * D * 2 + 1023) / 1024 * 1024;  // whole 1 KiB loads
  static constexpr int NQI = QB / 1024;                  // q load instructions per workgroup
  static constexpr int STAGE = WAVES * (RING + Tile::PBUF) + QB;
  static constexpr int MERGE = WAVES * Tile::RP * (Tile::MS + 2) * 4;
  static constexpr int SMEM = STAGE > MERGE ? STAGE : MERGE;
  static constexpr int MAX_PPS = 64;
};

// Decode one quantized ring slot (see KernelCfg) into bf16 K and V tiles at
// stg, in the swizzled layout of a bf16 slot, and copy its per-token scales
// after them (K scales at word 0, V scales at word 64). A cached value is
// code * scale exactly; the staged tiles hold only the codes, exact in bf16,
// and the row tiles apply a token's K scale to its score and its V scale to
// its weight P. Q8: a code is one sign-extending byte convert. Q4: each
// nibble n = code + 8 is moved to the top of its byte and the byte's sign bit
// flipped, which leaves 16 * code as a signed byte (n >= 8: 16n - 128; n < 8:
// 16n + 128 - 256), so it too is one byte convert; the row tiles fold the
// 1/16 into the scales. Each lane takes 16-code pieces (one token, 16 dims:
// 16 bytes at QB = 8, 8 bytes of nibbles at QB = 4, dim 2i in the low nibble
// of byte i). Tokens past the sequence end have zero codes and zero scales
// (the chunk load zero-fills them): their scores and weights are zero.
template <int D, int TC, int QB, int QAREA, int TILES = 2>
__device__ __forceinline__ void q_decode_slot(const char* slot, char* stg) {
  constexpr int NC = D / 8;          // 16-byte bf16 chunks per token
  constexpr int PPT = D / 16;        // 16-code pieces per token
  constexpr int NP = TC * PPT / 64;  // pieces per lane per tile
  constexpr int PB = 16 * QB / 8;    // bytes per piece
  static_assert(TC * PPT % 64 == 0, "pieces must fill the wave");
  const int lane = threadIdx.x & 63;
  const float* sc = reinterpret_cast<const float*>(slot + 2 * QAREA);
  float* ss = reinterpret_cast<float*>(stg + TILES * TC * D * 2);
  ss[lane] = sc[lane];
  ss[64 + lane] = sc[64 + lane];
#pragma unroll
  for (int kv = 0; kv < TILES; ++kv) {
    const char* src = slot + kv * QAREA;
    u32x4* dst = reinterpret_cast<u32x4*>(stg + kv * TC * D * 2);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pc = i * 64 + lane;
      const int t = pc / PPT, h = pc % PPT;
      u32 o[8];
      if constexpr (QB == 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src + pc * PB);
        const u32 ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) sbytes_bf16(ws[j], o[2 * j], o[2 * j + 1]);
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(src + pc * PB);
        const u32 ws[2] = {w.x, w.y};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // even dims (low nibbles) and odd dims (high nibbles), 16 * code per byte
          const u32 lo = ((ws[j] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
          const u32 hi = (ws[j] & 0xF0F0F0F0u) ^ 0x80808080u;
          o[4 * j + 0] = pack_bf16(sbyte_f32<0>(lo), sbyte_f32<0>(hi));
          o[4 * j + 1] = pack_bf16(sbyte_f32<1>(lo), sbyte_f32<1>(hi));
          o[4 * j + 2] = pack_bf16(sbyte_f32<2>(lo), sbyte_f32<2>(hi));
          o[4 * j + 3] = pack_bf16(sbyte_f32<3>(lo), sbyte_f32<3>(hi));
        }
      }
      dst[t * NC + ((2 * h) ^ (t & (NC - 1)))] = u32x4{o[0], o[1], o[2], o[3]};
      dst[t * NC + ((2 * h + 1) ^ (t & (NC - 1)))] = u32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

// SHR: the shared-prefix call's shared keys on few rows (decode and verify
// batches). Work item = (KV head g, tile of RP stacked batch rows, split s of
// the shared pages), KV head fastest so that every item of one head lands on
// one XCD when Hkv is a multiple of 8. Rows are the batch's window rows times
// the head group, stacked (row R: window row R / group, q head g * group +
// R % group); every row sees every shared key, so nothing is masked. The
// split's table entries are sequence 0's; the grid checks that every table
// starts with them and that every window lies past them. Each item leaves
// its rows' partial (m, l, acc) in part_ml / part_acc, laid out
// [Hkv][splits][total_q * group], for the tails to merge. pps = shared pages
// per split, max_splits = the splits, page_offset = the shared pages.
template <int D, class Tile, int NBUF, int WAVES, int QB = 0, bool SHR = false>
__global__ __launch_bounds__(WAVES * 64) void attn_split_kernel(
    // leading scalars: what the first loads need, preloaded into SGPRs at
    // wave launch instead of read from the argument buffer
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_lens, int num_items, int B, int Hkv, int pps, int W, AttnParams p) {
  using C = KernelCfg<D, Tile, NBUF, WAVES, QB>;
  constexpr int kWaves = WAVES;
  constexpr int kThreads = WAVES * 64;
  using G = typename C::G;
  constexpr int TC = C::TC;
  constexpr int NI = G::NI;
  constexpr int NC = G::NC;
  constexpr int RP = Tile::RP;
  static_assert(NBUF >= 1 && NBUF <= 6, "ring depth");
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_pages[C::MAX_PPS];
  __shared__ int s_last;

  // XCD-aware item order. The dispatcher deals workgroup i to XCD i % 8; XCD
  // x takes the (KV head, split) pairs j = x, x + 8, ... (j = g + Hkv * s) in
  // turn, each pair's sequences consecutively. So the sequences of one pair,
  // which share prefix pages under dedup, read them through one L2; every XCD
  // gets the same mix of early splits (work for every sequence) and late ones
  // (only long sequences have them); and a ragged batch's empty items come
  // last in each XCD's queue.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  int b, g, s, seq_len, q_len, q_start, n_splits, page0, npg, rows;
  int rt = 0;  // SHR: row tile
  if constexpr (SHR) {
    const int rows_all = p.total_q * p.group;
    const int row_tiles = (rows_all + RP - 1) / RP;
    g = blockIdx.x % Hkv;
    rt = (blockIdx.x / Hkv) % row_tiles;
    s = blockIdx.x / Hkv / row_tiles;
    b = 0;
    const int shared_pages = p.page_offset;
    seq_len = shared_pages * kPage;
    // the contract, one (sequence, shared entry) pair per thread of the grid
    for (long e = (long)blockIdx.x * kThreads + threadIdx.x; e < (long)B * shared_pages;
         e += (long)gridDim.x * kThreads) {
      const int bb = (int)(e / shared_pages), jj = (int)(e % shared_pages);
      if (block_table[(size_t)bb * W + jj] != block_table[jj]) atomicOr(p.err, PKV_EFLAG_PAGE_BIT);
      if (jj == 0 && q_lens[bb] > 0 && seq_lens[bb] - q_lens[bb] < seq_len) atomicOr(p.err, PKV_EFLAG_QLEN_BIT);
    }
    q_len = 0;
    q_start = 0;
    n_splits = p.max_splits;
    page0 = s * pps;
    if (s >= n_splits || page0 >= shared_pages) return;
    npg = min(pps, shared_pages - page0);
    if ((int)threadIdx.x < npg) {
      int tbl = block_table[page0 + threadIdx.x];
      if (tbl < 0 || tbl >= p.P) {
        atomicOr(p.err, PKV_EFLAG_PAGE_BIT);
        tbl = -1;
      }
      s_pages[threadIdx.x] = tbl;
    }
    rows = min(RP, rows_all - rt * RP);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
  } else {
    const int pairs = num_items / B;
    const int xcd = blockIdx.x % kNumXcd, k = blockIdx.x / kNumXcd;
    b = k % B;
    const int j = xcd + kNumXcd * (k / B);
    if (j >= pairs) return;
    g = j % Hkv;
    s = j / Hkv;

    // independent loads first, so their latencies overlap: the sequence's
    // lengths, the split's table entries and the window-row prefix sum
    // p.page_offset leading table entries (and their tokens) are skipped: a
    // shared prefix attended to elsewhere; 0 otherwise
    const int po = p.page_offset;
    page0 = s * pps;
    int tbl = -1;
    if ((int)threadIdx.x < pps && page0 + (int)threadIdx.x < W - po)
      tbl = block_table[(size_t)b * W + po + page0 + threadIdx.x];
    seq_len = seq_lens[b] - po * kPage;
    q_len = q_lens[b];
    const RowPrefix rp = row_prefix(q_lens, b, B);
    q_start = rp.start;
    // the batch's row count against total_q, once per launch (item 0 always exists)
    if (blockIdx.x == 0 && threadIdx.x == 0 && rp.total != p.total_q) atomicOr(p.err, PKV_EFLAG_ROWS_BIT);
    if (q_len < 0) {
      if (s == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, PKV_EFLAG_QLEN_BIT);
      return;
    }
    if (q_len == 0 || rp.bad_before) return;
    const int n_pages = (seq_len + kPage - 1) / kPage;
    n_splits = (n_pages + pps - 1) / pps;
    if (q_len > p.max_q_len || q_len > seq_len || n_pages > W - po) {
      if (s == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, PKV_EFLAG_QLEN_BIT);
      return;
    }
    if (s >= n_splits) return;
    if (q_start + q_len > p.total_q) {
      if (s == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, PKV_EFLAG_ROWS_BIT);
      return;
    }
    npg = min(pps, n_pages - page0);
    if ((int)threadIdx.x < npg) {
      if (tbl < 0 || tbl >= p.P) {
        atomicOr(p.err, PKV_EFLAG_PAGE_BIT);
        tbl = -1;
      }
      s_pages[threadIdx.x] = tbl;
    }
    // Every load the compiler issued itself has landed by now (the table
    // entries were just used). A wait it can see says so: otherwise, before it
    // reuses the registers those loads targeted, it inserts vmcnt(0), which also
    // counts the direct q and K/V loads below and would hold the first K/V
    // chunk back until the q rows landed.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    rows = q_len * p.group;  // <= RP by the plan
    __syncthreads();
  }

  const int tok_begin = page0 * kPage;
  const int tok_end = min(seq_len, (page0 + npg) * kPage);
  const int n_chunks = (tok_end - tok_begin + TC - 1) / TC;
  const int my_chunks = n_chunks > wave ? (n_chunks - wave + kWaves - 1) / kWaves : 0;

  char* ring = smem + wave * C::RING;
  float* pbuf = reinterpret_cast<float*>(smem + kWaves * C::RING + wave * Tile::PBUF);
  char* qlds = smem + kWaves * (C::RING + Tile::PBUF);
  const u32 ring_lds = lds_addr_of(ring);

  // ---- q rows of (b, g) into LDS, XOR-swizzled like the K tiles; rows past
  // the window read out of range and land as zeros. The waves share the work.
  {
    const u32 q_bytes = (u32)p.total_q * p.Hq * D * 2;
    const u32x4 rq = make_rsrc(p.q, q_bytes);
    const u32 qbase = lds_addr_of(qlds);
    for (int i = wave; i < C::NQI; i += kWaves) {
      const int slot = i * 64 + lane;
      const int r = slot / NC, pos = slot % NC;
      u32 off = q_bytes;  // out of range: zero
      if (r < rows) {
        const int c = pos ^ (r & (NC - 1));
        const int R = SHR ? rt * RP + r : r;  // SHR: the stacked batch row
        off = (u32)(((q_start + R / p.group) * p.Hq + g * p.group + R % p.group) * D) * 2u + c * 16;
      }
      dma16(rq, off, uniform(qbase + i * 1024));
    }
  }

  // per-lane byte offsets of the K/V direct loads (the chunk base goes into
  // the descriptor, so they are the same for every chunk)
  u32 voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = i * 64 + lane;
    const int t = slot / NC, pos = slot % NC;
    voff[i] = t * G::RB + ((pos ^ (t & (NC - 1))) * 16);
  }

  auto issue = [&](int k) {
    const int c = wave + k * kWaves;
    const int t0 = tok_begin + c * TC;
    const int jp = t0 / kPage - page0;
    const int in_page = t0 % kPage;
    const int phys = __builtin_amdgcn_readfirstlane(s_pages[jp]);
    const int page_valid = min(kPage, seq_len - (page0 + jp) * kPage);
    int nvt = min(TC, page_valid - in_page);
    if (phys < 0) nvt = 0;
    const size_t tok = ((size_t)(phys < 0 ? 0 : phys) * Hkv + g) * kPage + in_page;  // token index in the pool
    const u32 base = uniform(ring_lds + (k % NBUF) * C::SLOT);
    if constexpr (QB != 0) {
      // codes: byte i of the chunk lands at byte i of its area (no swizzle);
      // scales: lane i's word at word i of the scale area
      constexpr int TB = D * QB / 8;  // code bytes per token
      const u32 cbytes = nvt > 0 ? (u32)(nvt * TB) : 0u;
      const u32 sbytes = nvt > 0 ? (u32)(nvt * 4) : 0u;
      const auto* kc = reinterpret_cast<const char*>(p.k_pool) + tok * TB;
      const auto* vc = reinterpret_cast<const char*>(p.v_pool) + tok * TB;
      const u32x4 rk = make_rsrc(kc, cbytes), rv = make_rsrc(vc, cbytes);
      const u32x4 rks = make_rsrc(p.k_scales + tok, sbytes), rvs = make_rsrc(p.v_scales + tok, sbytes);
      wait_lgkm0();
#pragma unroll
      for (int i = 0; i < C::NCI; ++i) dma16(rk, (u32)(i * 64 + lane) * 16u, base + i * 1024);
#pragma unroll
      for (int i = 0; i < C::NCI; ++i) dma16(rv, (u32)(i * 64 + lane) * 16u, base + C::QAREA + i * 1024);
      dma4(rks, (u32)lane * 4u, base + 2 * C::QAREA);
      dma4(rvs, (u32)lane * 4u, base + 2 * C::QAREA + 256);
    } else {
      const size_t off = tok * D;
      const u32 bytes = nvt > 0 ? (u32)(nvt * G::RB) : 0u;
      const u32x4 rk = make_rsrc(p.k_pool + off, bytes);
      const u32x4 rv = make_rsrc(p.v_pool + off, bytes);
      wait_lgkm0();
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(rk, voff[i], base + i * 1024);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(rv, voff[i], base + G::TILE + i * 1024);
    }
  };

  Tile tile;
  if constexpr (SHR)
    tile.init(1, rows, 1 << 30, 0);  // every shared key visible to every row
  else
    tile.init(p.group, rows, seq_len, q_len);
  // fill the whole ring
  const int pro = min(NBUF, my_chunks);
#pragma unroll
  for (int k = 0; k < NBUF; ++k)
    if (k < my_chunks) issue(k);
  // this wave's q loads were issued before its prologue chunks: once at most
  // `pro` chunks remain in flight they have landed; the barrier covers the
  // other waves' share
  wait_ahead<C::OPS, NBUF>(pro);
  asm volatile("s_barrier" ::: "memory");
  tile.load_q(qlds);

  for (int k = 0; k < my_chunks; ++k) {
    // chunk k has landed once at most the chunks issued after it are pending
    wait_ahead<C::OPS, NBUF - 1>(min(NBUF - 1, my_chunks - 1 - k));
    const int c = wave + k * kWaves;
    const int t0 = tok_begin + c * TC;
    const int nv = min(TC, tok_end - t0);
    const char* kt = ring + (k % NBUF) * C::SLOT;
    const float* qsc = nullptr;  // quantized: the chunk's staged K and V scales
    if constexpr (QB != 0) {
      char* stg = ring + NBUF * C::SLOT;
      q_decode_slot<D, TC, QB, C::QAREA, C::STG_TILES>(kt, stg);
      qsc = reinterpret_cast<const float*>(stg + C::STG_TILES * G::TILE);
      if constexpr (C::VDIRECT)
        tile.template fetch_q<QB>(stg, kt + C::QAREA);
      else
        tile.fetch(stg, stg + G::TILE, nv);
    } else {
      tile.fetch(kt, kt + G::TILE, nv);
    }
    // the slot is free once its operands sit in registers: refill it now so
    // NBUF chunks stay in flight while this one is computed
    if (k + NBUF < my_chunks) issue(k + NBUF);
    tile.template compute<QB, !SHR>(pbuf, t0, nv, p.scale_log2, qsc);
  }

  // ---- merge the waves in LDS
  __syncthreads();
  float* red_m = reinterpret_cast<float*>(smem);
  float* red_l = red_m + kWaves * RP;
  float* red_acc = red_l + kWaves * RP;
  tile.spill(red_m + wave * RP, red_l + wave * RP, red_acc + (size_t)wave * RP * Tile::MS);
  __syncthreads();

  constexpr int D4 = D / 4;
  const size_t bg = (size_t)b * Hkv + g;
  const u32 acc_bytes = (u32)(p.max_splits * p.rows_max * D * 4);
  const u32 ml_bytes = (u32)(p.max_splits * p.rows_max * 2 * 4);
  const auto acc_rsrc = buf_rsrc(p.part_acc + bg * p.max_splits * p.rows_max * D, acc_bytes);
  const auto ml_rsrc = buf_rsrc(p.part_ml + bg * p.max_splits * p.rows_max * 2, ml_bytes);
  for (int e = threadIdx.x; e < rows * D4; e += kThreads) {
    const int r = e / D4, dq = e % D4;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w * RP + r]);
    float L = 0.f;
    f32x4 A = {0.f, 0.f, 0.f, 0.f};
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = red_m[w * RP + r];
        const float wt = (mw == kNegInf) ? 0.f : exp2f_fast(mw - M);
        L += wt * red_l[w * RP + r];
        A += wt * *reinterpret_cast<const f32x4*>(red_acc + ((size_t)w * RP + r) * Tile::MS + 4 * dq);
      }
    }
    if constexpr (SHR) {
      // the shared split's partial of stacked row R, read by the next kernel
      const size_t i = ((size_t)g * n_splits + s) * ((size_t)p.total_q * p.group) + rt * RP + r;
      *reinterpret_cast<f32x4*>(p.part_acc + i * D + 4 * dq) = A;
      if (dq == 0) *reinterpret_cast<f32x2*>(p.part_ml + i * 2) = f32x2{M, L};
    } else if (n_splits == 1) {
      const int h = g * p.group + r % p.group;
      if (p.shared_ml) {
        // the shared prefix's key splits, in order, after this row's own
        // keys (batches of 8 with every load issued first)
        constexpr int SB = 8;
        const size_t rows_all = (size_t)p.total_q * p.group;
        const size_t R = (size_t)(q_start + r / p.group) * p.group + r % p.group;
        for (int s0 = 0; s0 < p.shared_splits; s0 += SB) {
          f32x2 ml[SB];
          f32x4 pa[SB];
#pragma unroll
          for (int j = 0; j < SB; ++j) {
            const size_t i = ((size_t)g * p.shared_splits + min(s0 + j, p.shared_splits - 1)) * rows_all + R;
            ml[j] = *reinterpret_cast<const f32x2*>(p.shared_ml + i * 2);
            pa[j] = *reinterpret_cast<const f32x4*>(p.shared_acc + i * D + 4 * dq);
          }
          float Mn = M;
#pragma unroll
          for (int j = 0; j < SB; ++j)
            if (s0 + j < p.shared_splits) Mn = fmaxf(Mn, ml[j].x);
          const float f = M == kNegInf ? 0.f : exp2f_fast(M - Mn);
          L *= f;
          A *= f;
#pragma unroll
          for (int j = 0; j < SB; ++j) {
            const float w = (s0 + j >= p.shared_splits || ml[j].x == kNegInf) ? 0.f : exp2f_fast(ml[j].x - Mn);
            L += w * ml[j].y;
            A += w * pa[j];
          }
          M = Mn;
        }
      }
      *reinterpret_cast<f32x4*>(p.out + ((size_t)(q_start + r / p.group) * p.Hq + h) * D + 4 * dq) = A / L;
      if (p.out_lse && dq == 0) p.out_lse[(size_t)(q_start + r / p.group) * p.Hq + h] = M + __log2f(L);
    } else {
      // write-through stores: visible to the merging workgroup on any XCD
      __builtin_amdgcn_raw_buffer_store_b128(A, acc_rsrc, ((s * p.rows_max + r) * D + 4 * dq) * 4, 0, kSc1);
      if (dq == 0) {
        const f32x2 ml = {M, L};
        __builtin_amdgcn_raw_buffer_store_b64(ml, ml_rsrc, (s * p.rows_max + r) * 8, 0, kSc1);
      }
    }
  }
  if (SHR || n_splits == 1) return;

  // ---- the last workgroup of (b, g) merges every split in split order.
  // Every thread's partial stores are acknowledged (vmcnt 0) before the
  // barrier, so they are device-visible before thread 0 bumps the counter.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const u32 prev = __hip_atomic_fetch_add(p.counters + bg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (u32)(n_splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  // Each thread owns EPT elements (row, 4 dims) and takes the splits in
  // batches of SB, issuing every load of a batch before using any: one
  // memory round trip per batch instead of one per element.
  constexpr int EPT = (RP * D4 + kThreads - 1) / kThreads;
  constexpr int SB = EPT <= 2 ? 8 : (EPT <= 4 ? 4 : 2);
  float M[EPT], L[EPT];
  f32x4 A[EPT];
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    M[u] = kNegInf;
    L[u] = 0.f;
    A[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int sp0 = 0; sp0 < n_splits; sp0 += SB) {
    f32x2 ml[EPT][SB];
    f32x4 pa[EPT][SB];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = threadIdx.x + u * kThreads;
      const int r = e < rows * D4 ? e / D4 : 0, dq = e % D4;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        // splits past the end read out of range (zeros) and are dropped below
        const int sp = sp0 + j < n_splits ? sp0 + j : p.max_splits;
        ml[u][j] = __builtin_amdgcn_raw_buffer_load_b64(ml_rsrc, (sp * p.rows_max + r) * 8, 0, kSc1);
        pa[u][j] = __builtin_amdgcn_raw_buffer_load_b128(acc_rsrc, ((sp * p.rows_max + r) * D + 4 * dq) * 4, 0,
                                                         kSc1);
      }
    }
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      float Mn = M[u];
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (sp0 + j < n_splits) Mn = fmaxf(Mn, ml[u][j].x);
      if (Mn == kNegInf) continue;
      const float f = (M[u] == kNegInf) ? 0.f : exp2f_fast(M[u] - Mn);
      L[u] *= f;
      A[u] *= f;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const float wt = (sp0 + j >= n_splits || ml[u][j].x == kNegInf) ? 0.f : exp2f_fast(ml[u][j].x - Mn);
        L[u] += wt * ml[u][j].y;
        A[u] += wt * pa[u][j];
      }
      M[u] = Mn;
    }
  }
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int e = threadIdx.x + u * kThreads;
    if (e >= rows * D4) continue;
    const int r = e / D4, dq = e % D4;
    const int h = g * p.group + r % p.group;
    *reinterpret_cast<f32x4*>(p.out + ((size_t)(q_start + r / p.group) * p.Hq + h) * D + 4 * dq) = A[u] / L[u];
    if (p.out_lse && dq == 0) p.out_lse[(size_t)(q_start + r / p.group) * p.Hq + h] = M[u] + __log2f(L[u]);
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.counters + bg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ prefill kernel

// Long windows (q_len * group > 64 rows: prefill, or a long chunk of it over a
// cached prefix). A workgroup takes a query tile of kPrefillRows rows (rows =
// window tokens times the head group) of one (sequence, KV head) and streams
// every key the tile may see, 0 .. the tile's last token, through a ring of
// K/V chunks shared by its waves. Each wave owns 32 * NRB of the rows on the
// MFMA row tile (64 by default), so a K/V chunk staged once in LDS feeds all
// 256 rows; the ring is filled by direct buffer->LDS loads, each wave issuing
// an equal share of every chunk. Tiles are aligned to the end of the window, so tile 0 of every
// sequence is the one with the most keys, and the launch takes tile 0 of every
// (sequence, KV head) first (longest work first). All tiles of a (sequence,
// KV head) land on the same XCD when B * Hkv is a multiple of 8, so the K/V
// they share is served from that XCD's L2. No split of the key range: every
// tile writes its rows of `out` itself.

constexpr int kPrefillRows = 256;  // rows of a query tile (and of a shared-prefix row tile)
// Waves of a long-window workgroup: 64-row waves (NRB = 2, one wave per SIMD)
// or 32-row waves (NRB = 1, two per SIMD, so one wave's exponentials and
// waits run beside the other's matrix products).
template <int NRB>
constexpr int kLongWaves = kPrefillRows / (32 * NRB);
// 32-row waves measured 446 against 773 TFLOP/s on the whole-prompt prefill:
// at two waves per SIMD a wave gets 128 VGPRs + 128 accumulation registers and
// spills about 30 VGPRs in the chunk loop.
#ifndef PKV_LONG_NRB128
#define PKV_LONG_NRB128 2  // row blocks per wave on the head_dim-128 long-window kernels
#endif
template <int D>
constexpr int kLongNrb = D == 128 ? PKV_LONG_NRB128 : 2;
constexpr int kPrefillMaxPages = 2048;  // table entries staged per tile (524288 tokens)

template <int LPC, int A>
__device__ __forceinline__ void wait_chunks(int ahead) {
  if constexpr (A > 0) {
    if (ahead >= A) {
      wait_vmcnt<LPC * A>();
      return;
    }
    wait_chunks<LPC, A - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

// Streams keys key_begin .. key_end - 1 (key_begin a multiple of 32) of KV
// head g through the workgroup's ring of NBUF K/V chunks into the tile's
// rows. s_pages[j] is the physical page of keys (key_begin / 256 + j) * 256 ..
// (a negative entry reads as zeros). Chunks [0, n_split) take P in two bf16
// terms; chunks [n_split, n_free) are seen in full by every valid row of this
// wave and go unmasked; the rest are masked by the tile's row limits.
//
// The chunk loop is software-pipelined: while the VALU turns chunk c's
// scores into P, the matrix cores already compute chunk c + 1's scores. Each
// wave issues a quarter of every chunk's direct buffer->LDS loads. arrive(k):
// chunk k has landed once at most the chunks issued after it are pending
// (this wave's share); the barrier then covers the other waves' shares and
// tells that every wave is done with chunk k - 2 (its V was read in the
// iteration that ended before it), whose slot takes chunk k + NBUF - 2. It
// then copies chunk k's K operand out. Every wave of the workgroup must call
// this with the same key range.
template <int D, int NBUF, int NRB>
__device__ __forceinline__ void stream_keys(MfmaTile<D, NRB>& tile, char* ring, const int* s_pages,
                                            const AttnParams& p, int Hkv, int g, int key_begin, int key_end,
                                            int n_split, int n_free, float scale_log2) {
  using G = TileGeom<D, 32>;
  constexpr int TC = 32;
  constexpr int NI = G::NI;   // 1 KiB loads per K (or V) chunk
  constexpr int NC = G::NC;
  constexpr int WAVES = kLongWaves<NRB>;
  constexpr int KPW = NI / WAVES;          // this wave's share of them
  constexpr int LPC = 2 * KPW;             // load instructions per chunk per wave
  static_assert(NI % WAVES == 0, "chunk loads split evenly over the waves");
  static_assert(NBUF >= 3 && LPC * (NBUF - 3) < 64, "ring depth");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n_chunks = (key_end - key_begin + TC - 1) / TC;
  const int page_base = key_begin / kPage;

  // per-lane byte offsets of this wave's share of a chunk's direct loads
  u32 voff[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int slot = (wave * KPW + i) * 64 + lane;
    const int t = slot / NC, pos = slot % NC;
    voff[i] = t * G::RB + ((pos ^ (t & (NC - 1))) * 16);
  }
  const u32 ring_lds = lds_addr_of(ring);
  const size_t head_stride = (size_t)kPage * D;
  auto issue = [&](int c) {
    const int t0 = key_begin + c * TC;
    const int phys = __builtin_amdgcn_readfirstlane(s_pages[t0 / kPage - page_base]);
    int nvt = min(TC, key_end - t0);
    if (phys < 0) nvt = 0;
    const size_t off = ((size_t)(phys < 0 ? 0 : phys) * Hkv + g) * head_stride + (size_t)(t0 % kPage) * D;
    const u32 bytes = nvt > 0 ? (u32)(nvt * G::RB) : 0u;
    const u32x4 rk = make_rsrc(p.k_pool + off, bytes);
    const u32x4 rv = make_rsrc(p.v_pool + off, bytes);
    const u32 base = uniform(ring_lds + (c % NBUF) * 2 * G::TILE + wave * KPW * 1024);
#pragma unroll
    for (int i = 0; i < KPW; ++i) dma16(rk, voff[i], base + i * 1024);
#pragma unroll
    for (int i = 0; i < KPW; ++i) dma16(rv, voff[i], base + G::TILE + i * 1024);
  };

#pragma unroll
  for (int c = 0; c < NBUF - 2; ++c)
    if (c < n_chunks) issue(c);

  auto slot = [&](int c) { return ring + (c % NBUF) * 2 * G::TILE; };
  auto arrive = [&](int k) {
    wait_chunks<LPC, NBUF - 3>(min(NBUF - 3, n_chunks - 1 - k));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (k + NBUF - 2 < n_chunks) issue(k + NBUF - 2);
    tile.fetch_k(slot(k));
  };
  // Prologue: chunk 0's scores. Iteration c then runs, in one stretch of
  // straight-line code: chunk c's exponentials beside chunk c + 1's score
  // products, and chunk c's P.V products beside chunk c + 1's row maxima;
  // the rare rescale of chunk c + 1 closes it.
  f32x16 S[2];
  arrive(0);
  tile.qk(S);
  if (tile.template scores<true>(S, key_begin, min(TC, key_end - key_begin), scale_log2)) tile.rescale();
  auto step = [&](auto split_p, auto mask_next, int c) {
    constexpr bool kSplit = decltype(split_p)::value, kMask = decltype(mask_next)::value;
    const int cn = c + 1;  // past the last chunk its products repeat chunk c's, unused
    const int t1 = key_begin + cn * TC;
    if (cn < n_chunks) arrive(cn);
    tile.fetch_v(slot(c) + G::TILE);
    tile.template probs<kSplit>(scale_log2);
    tile.qk(S);
#pragma unroll
    for (int i = 0; i < 8 * NRB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kSplit ? 7 : 5, 0);
    }
    tile.template pv<kSplit>();
    const bool grow = tile.template scores<kMask>(S, t1, min(TC, key_end - t1), scale_log2);
#pragma unroll
    for (int i = 0; i < (kSplit ? 18 : 10) * NRB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kSplit ? 2 : 4, 0);
    }
    if (grow && cn < n_chunks) tile.rescale();
  };
  // chunk c's P: two bf16 terms for chunks below n_split and wherever a key
  // still weighs more than 1/8 of its row; chunk c + 1's mask: the unmasked
  // stretch ends one chunk early so its next chunk is unmasked too
  const int c_mask = max(n_split, n_free - 1);
  int c = 0;
  for (; c < n_split; ++c) step(std::true_type{}, std::true_type{}, c);
  while (c < n_chunks) {
    for (; c < c_mask && !tile.needs_split(); ++c) step(std::false_type{}, std::false_type{}, c);
    for (; c >= c_mask && c < n_chunks && !tile.needs_split(); ++c) step(std::false_type{}, std::true_type{}, c);
    if (c < n_chunks) step(std::true_type{}, std::true_type{}, c++);
  }
}

// The softmax of stream_keys takes scale_log2 > 0 (it scales row maxima, not
// every score, and masked scores are -inf): a negative scale becomes a
// positive one on -q (negating bf16, its sign bits, is exact), and a zero
// scale is scale 1 on q = 0 (every visible key weighs the same either way).
struct QSign {
  u32 sign, keep;
  float scale_log2;
  __device__ explicit QSign(float s)
      : sign(s < 0.f ? 0x80008000u : 0u), keep(s == 0.f ? 0u : 0xFFFFFFFFu), scale_log2(s == 0.f ? 1.f : fabsf(s)) {}
  __device__ u32x4 apply(u32x4 q) const { return (q & u32x4{keep, keep, keep, keep}) ^ u32x4{sign, sign, sign, sign}; }
};

// Loads the q rows of one wave's 64 tile rows straight into the MFMA operand
// registers; row_src(r) is the q row (element offset) of tile row r, or -1 for
// a padding row.
template <int D, int NRB, class RowSrc>
__device__ __forceinline__ void load_q_rows(MfmaTile<D, NRB>& tile, const uint16_t* q, const QSign& qs,
                                            RowSrc row_src) {
  using Tile = MfmaTile<D, NRB>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int half = lane >> 5;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const long off = row_src(wave * 32 * NRB + rb * 32 + (lane & 31));
    const u32x4* src = reinterpret_cast<const u32x4*>(q + (off < 0 ? 0 : off));
#pragma unroll
    for (int kk = 0; kk < Tile::KK; ++kk)
      tile.qb[rb][kk] = qs.apply(off >= 0 ? src[2 * kk + half] : u32x4{0u, 0u, 0u, 0u});
  }
  // wait for the q operands here: a load still pending at the chunk loop
  // would make the compiler wait for every load in flight (the whole K/V
  // ring, which it does not see) at each chunk
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int kk = 0; kk < Tile::KK; ++kk) asm volatile("" ::"v"(tile.qb[rb][kk]));
}

template <int D, int NBUF, int NRB>
__global__ __launch_bounds__(kLongWaves<NRB> * 64) void attn_prefill_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_lens, int B, int Hkv, int qtok, int W, AttnParams p) {
  using Tile = MfmaTile<D, NRB>;
  constexpr int THREADS = kLongWaves<NRB> * 64;
  constexpr int WROWS = 32 * NRB;  // rows of one wave
  using G = TileGeom<D, 32>;
  constexpr int TC = 32;
  __shared__ __attribute__((aligned(16))) char ring[NBUF * 2 * G::TILE];
  __shared__ int s_pages[kPrefillMaxPages];

  const int bh = B * Hkv;
  const int bg = blockIdx.x % bh, qr = blockIdx.x / bh;
  const int b = bg / Hkv, g = bg % Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

  // p.page_offset leading table entries (and their tokens) are skipped: a
  // shared prefix attended to elsewhere; 0 otherwise
  const int po = p.page_offset;
  const int seq_len = seq_lens[b] - po * kPage;
  const int q_len = q_lens[b];
  const RowPrefix rp = row_prefix(q_lens, b, B);
  const int q_start = rp.start;
  // the batch's row count against total_q, once per launch
  if (blockIdx.x == 0 && threadIdx.x == 0 && rp.total != p.total_q) atomicOr(p.err, PKV_EFLAG_ROWS_BIT);
  if (q_len < 0) {
    if (qr == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, PKV_EFLAG_QLEN_BIT);
    return;
  }
  if (q_len == 0 || rp.bad_before) return;
  const int n_tiles = (q_len + qtok - 1) / qtok;
  if (qr >= n_tiles) return;
  const int n_pages = (seq_len + kPage - 1) / kPage;
  if (q_len > p.max_q_len || q_len > seq_len || n_pages > W - po || n_pages > kPrefillMaxPages) {
    if (qr == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, PKV_EFLAG_QLEN_BIT);
    return;
  }
  if (q_start + q_len > p.total_q) {
    if (qr == 0 && g == 0 && threadIdx.x == 0) atomicOr(p.err, PKV_EFLAG_ROWS_BIT);
    return;
  }
  // this tile: window tokens tq0 .. tq0 + qtok - 1 (those >= 0), keys 0 .. key_end - 1
  const int tq0 = q_len - (qr + 1) * qtok;
  const int key_end = seq_len - qr * qtok;
  const int n_chunks = (key_end + TC - 1) / TC;
  const int need_pages = (key_end + kPage - 1) / kPage;
  for (int j = threadIdx.x; j < need_pages; j += THREADS) {
    int e = block_table[(size_t)b * W + po + j];
    if (e < 0 || e >= p.P) {
      atomicOr(p.err, PKV_EFLAG_PAGE_BIT);
      e = -1;
    }
    s_pages[j] = e;
  }

  // row r of the tile is window token tq0 + r / group, q head g * group + r % group
  const QSign qs(p.scale_log2);
  Tile tile;
  const int r_lo = (tq0 < 0 ? -tq0 : 0) * p.group, r_hi = qtok * p.group;
  tile.init_rows(wave * WROWS, p.group, seq_len - q_len + tq0, r_lo, r_hi);
  load_q_rows<D>(tile, p.q, qs, [&](int r) -> long {
    if (r < r_lo || r >= r_hi) return -1;
    return ((long)(q_start + tq0 + r / p.group) * p.Hq + g * p.group + r % p.group) * D;
  });
  __syncthreads();  // table entries staged

  // the first 64 keys with P in two bf16 terms: rows that see fewer than 64
  // keys see nothing else, and their few terms would not average out the
  // rounding of a single bf16 P. Then the chunks every valid row of this
  // wave sees in full go unmasked; the rest (the diagonal) are masked.
  const int n_split = min(n_chunks, 64 / TC);
  const int wrow = max(r_lo, wave * WROWS);
  const int wave_min_lim = wrow < r_hi ? seq_len - q_len + tq0 + wrow / p.group : key_end;
  const int n_free = max(n_split, min(key_end / TC, (wave_min_lim + 1) / TC));
  stream_keys<D, NBUF, NRB>(tile, ring, s_pages, p, Hkv, g, 0, key_end, n_split, n_free, qs.scale_log2);

  // rows -> out
  {
    const int half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = wave * WROWS + rb * 32 + (lane & 31);
      const float ls = tile.lacc[rb][0];
      if (r < r_lo || r >= r_hi) continue;
      const size_t th = (size_t)(q_start + tq0 + r / p.group) * p.Hq + g * p.group + r % p.group;
      float* dst = p.out + th * D;
      // the row's base-2 log-sum-exp, for a merge with keys attended elsewhere
      if (p.out_lse && half == 0) p.out_lse[th] = tile.m[rb] + __log2f(ls);
#pragma unroll
      for (int mb = 0; mb < Tile::MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = {tile.acc[rb][mb][4 * j], tile.acc[rb][mb][4 * j + 1], tile.acc[rb][mb][4 * j + 2],
                           tile.acc[rb][mb][4 * j + 3]};
          *reinterpret_cast<f32x4*>(dst + mb * 32 + 8 * j + 4 * half) = v / ls;
        }
    }
  }
}

// ------------------------------------------------------ shared-prefix path

// Attention over a batch whose sequences all begin with the same
// shared_pages pages (a deduplicated prompt prefix, ExLlamaV2 "Dynamic
// Generator" page, "Deduplication"). The shared keys are attended to once per
// KV head for every window row of the batch stacked into 256-row MFMA tiles
// (rows = total_q x group); the tails (each sequence's keys past the shared
// pages) run through the split kernel or the long-window kernel with the
// shared pages skipped. The two meet by log-sum-exp in one of three ways
// (the host picks by the plans): with one key split the tails run first,
// leaving each row normalised with its log-sum-exp, and a workgroup of this
// kernel merges its rows into theirs at once; with several key splits each
// split leaves a partial (reference max, row sum, unnormalised accumulator)
// per row, folded in by the tails' own epilogue when they run after it with
// one split each, else by shared_merge_kernel after both.
//
// Work item = (KV head g, row tile, key split), KV head fastest so that every
// item of one head lands on one XCD when Hkv is a multiple of 8.
template <int D, int NBUF, int NRB>
__global__ __launch_bounds__(kLongWaves<NRB> * 64) void attn_shared_kernel(SharedParams sp, AttnParams p) {
  using Tile = MfmaTile<D, NRB>;
  constexpr int THREADS = kLongWaves<NRB> * 64;
  constexpr int WROWS = 32 * NRB;  // rows of one wave
  using G = TileGeom<D, 32>;
  __shared__ __attribute__((aligned(16))) char ring[NBUF * 2 * G::TILE];
  __shared__ int s_pages[kPrefillMaxPages];

  const int Hkv = p.Hkv;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int rt = rest % sp.row_tiles, split = rest / sp.row_tiles;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int shared_tokens = sp.shared_pages * kPage;

  // the contract, one (sequence, shared entry) pair per thread of the grid:
  // every table starts with sequence 0's shared entries and every window row
  // sees the whole shared prefix
  for (long e = (long)blockIdx.x * THREADS + threadIdx.x; e < (long)p.B * sp.shared_pages;
       e += (long)gridDim.x * THREADS) {
    const int b = (int)(e / sp.shared_pages), j = (int)(e % sp.shared_pages);
    if (p.block_table[(size_t)b * p.W + j] != p.block_table[j]) atomicOr(p.err, PKV_EFLAG_PAGE_BIT);
    if (j == 0 && p.q_lens[b] > 0 && p.seq_lens[b] - p.q_lens[b] < shared_tokens) atomicOr(p.err, PKV_EFLAG_QLEN_BIT);
  }

  const int key_begin = split * sp.split_keys;
  const int key_end = min(key_begin + sp.split_keys, shared_tokens);
  if (key_begin >= key_end) return;
  const int page_base = key_begin / kPage, n_pg = (key_end - 1) / kPage - page_base + 1;
  for (int j = threadIdx.x; j < n_pg; j += THREADS) {
    int e = p.block_table[page_base + j];
    if (e < 0 || e >= p.P) {
      atomicOr(p.err, PKV_EFLAG_PAGE_BIT);
      e = -1;
    }
    s_pages[j] = e;
  }

  // tile row r is batch row R = rt * 256 + r: q row R / group, q head
  // g * group + R % group; every row sees every shared key
  const int rows = p.total_q * p.group;
  const int r_hi = min(kPrefillRows, rows - rt * kPrefillRows);
  const QSign qs(p.scale_log2);
  Tile tile;
  tile.init_rows(wave * WROWS, 1, 1 << 30, 0, r_hi);
  load_q_rows<D>(tile, p.q, qs, [&](int r) -> long {
    if (r >= r_hi) return -1;
    const int R = rt * kPrefillRows + r;
    return ((long)(R / p.group) * p.Hq + g * p.group + R % p.group) * D;
  });
  __syncthreads();  // table entries staged

  const int n_chunks = (key_end - key_begin) / 32;
  stream_keys<D, NBUF, NRB>(tile, ring, s_pages, p, Hkv, g, key_begin, key_end, 0, n_chunks, qs.scale_log2);

  // One key split: merge with the tail's row straight away. The tails ran
  // first and left each row normalised in out with its base-2 log-sum-exp in
  // out_lse: a partial with row sum 1 at that reference max.
  if (sp.splits == 1) {
    const int half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = wave * WROWS + rb * 32 + (lane & 31);
      if (r >= r_hi) continue;
      const int R = rt * kPrefillRows + r;
      const size_t th = (size_t)(R / p.group) * p.Hq + g * p.group + R % p.group;
      const float mt = p.out_lse[th], ms = tile.m[rb];
      const float mx = fmaxf(mt, ms);
      const float wt = exp2f_fast(mt - mx);
      const float ws = ms == kNegInf ? 0.f : exp2f_fast(ms - mx);
      const float inv = 1.f / (wt + ws * tile.lacc[rb][0]);
      float* o = p.out + th * D;
#pragma unroll
      for (int mb = 0; mb < Tile::MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4* dst = reinterpret_cast<f32x4*>(o + mb * 32 + 8 * j + 4 * half);
          const f32x4 a = {tile.acc[rb][mb][4 * j], tile.acc[rb][mb][4 * j + 1], tile.acc[rb][mb][4 * j + 2],
                           tile.acc[rb][mb][4 * j + 3]};
          *dst = (wt * *dst + ws * a) * inv;
        }
    }
    return;
  }
  // partials: (m, l) and the unnormalised accumulator of each valid row
  {
    const int half = lane >> 5;
    const size_t base = ((size_t)g * sp.splits + split) * rows + rt * kPrefillRows;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = wave * WROWS + rb * 32 + (lane & 31);
      if (r >= r_hi) continue;
      if (half == 0) {
        sp.part_ml[(base + r) * 2] = tile.m[rb];
        sp.part_ml[(base + r) * 2 + 1] = tile.lacc[rb][0];
      }
      float* dst = sp.part_acc + (base + r) * D;
#pragma unroll
      for (int mb = 0; mb < Tile::MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(dst + mb * 32 + 8 * j + 4 * half) =
              f32x4{tile.acc[rb][mb][4 * j], tile.acc[rb][mb][4 * j + 1], tile.acc[rb][mb][4 * j + 2],
                    tile.acc[rb][mb][4 * j + 3]};
    }
  }
}

// out (the tails' normalised rows, in place) and their log-sum-exp merged
// with the shared-prefix partials: one thread per (q row, q head, 4 dims),
// splits in order, in batches of 8 whose loads are all issued before any is
// used (one memory round trip per batch), with the running max rescaled per
// batch.
template <int D>
__global__ __launch_bounds__(256) void shared_merge_kernel(SharedParams sp, AttnParams p) {
  constexpr int D4 = D / 4;
  constexpr int SB = 8;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)p.total_q * p.Hq * D4) return;
  const int dq = (int)(e % D4);
  const long th = e / D4;                        // q row * Hq + q head
  const int h = (int)(th % p.Hq), t = (int)(th / p.Hq);
  const int g = h / p.group;
  const size_t rows = (size_t)p.total_q * p.group;
  const size_t R = (size_t)t * p.group + h % p.group;
  float* o = p.out + th * D + 4 * dq;
  // the tail as a partial: reference max lse, row sum 1, accumulator = its row
  float M = p.out_lse[th], L = 1.f;
  f32x4 A = *reinterpret_cast<const f32x4*>(o);
  for (int s0 = 0; s0 < sp.splits; s0 += SB) {
    f32x2 ml[SB];
    f32x4 pa[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const size_t i = ((size_t)g * sp.splits + min(s0 + j, sp.splits - 1)) * rows + R;
      ml[j] = *reinterpret_cast<const f32x2*>(sp.part_ml + i * 2);
      pa[j] = *reinterpret_cast<const f32x4*>(sp.part_acc + i * D + 4 * dq);
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < SB; ++j)
      if (s0 + j < sp.splits) Mn = fmaxf(Mn, ml[j].x);
    const float f = exp2f_fast(M - Mn);
    L *= f;
    A *= f;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const float w = (s0 + j >= sp.splits || ml[j].x == kNegInf) ? 0.f : exp2f_fast(ml[j].x - Mn);
      L += w * ml[j].y;
      A += w * pa[j];
    }
    M = Mn;
  }
  *reinterpret_cast<f32x4*>(o) = A / L;
}

template <int D, class Tile, int NBUF, int WAVES, int QB>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  // every XCD gets ceil(pairs / 8) pairs of B items (see the kernel)
  const int pairs = p.num_items / p.B;
  const int grid = kNumXcd * ((pairs + kNumXcd - 1) / kNumXcd) * p.B;
  hipLaunchKernelGGL((attn_split_kernel<D, Tile, NBUF, WAVES, QB>), dim3(grid), dim3(WAVES * 64), 0, stream,
                     p.block_table, p.seq_lens, p.q_lens, p.num_items, p.B, p.Hkv, p.pps, p.W, p);
  return hipGetLastError();
}

template <int D, int QB>
hipError_t launch_d(const AttnParams& p, const AttnPlan& plan, hipStream_t stream) {
  // the Q4 VALU ring goes deeper: a chunk of codes is a quarter of a bf16
  // chunk, and with the V codes converted straight from the slot (no V
  // staging) four slots still leave two workgroups per CU (Q8 measured no
  // better at three slots than at two)
  constexpr int kValuNbuf = QB == 8 ? PKV_VALU_Q8_NBUF : QB == 4 ? PKV_VALU_Q4_NBUF : PKV_VALU_NBUF;
  if (!plan.mfma) {
    // bf16 decode with more items than one round of four-wave workgroups
    // holds. Items of at most two pages (the tails of the shared-prefix
    // call): two-wave workgroups. The tile's registers allow two waves per
    // SIMD at head_dim 128, so a CU holds two four-wave workgroups but four
    // two-wave ones, and 800 one-page tails run in one round instead of two
    // (shared call 44.9 -> 42.4 us). Longer items (the dedup batch, 17 pages
    // each) keep four waves on one-slot rings: their chunks in flight per
    // item set their pace (two-wave workgroups: 165.6 -> 175.8 us).
    using Four = KernelCfg<D, ValuTile<D, 1>, kValuNbuf, PKV_VALU_WAVES, QB>;
    if constexpr (QB == 0 && kValuNbuf == 2 && PKV_VALU_WAVES == 4) {
      if ((long)p.num_items > (long)kNumCu * (kLdsPerCu / Four::SMEM)) {
        if (min(p.pps, p.W - p.page_offset) <= 2) return launch_one<D, ValuTile<D, 1>, 2, 2, QB>(p, stream);
        return launch_one<D, ValuTile<D, 1>, 1, PKV_VALU_WAVES, QB>(p, stream);
      }
    }
    return launch_one<D, ValuTile<D, 1>, kValuNbuf, PKV_VALU_WAVES, QB>(p, stream);
  }
  if (plan.rows <= 32) return launch_one<D, MfmaTile<D, 1>, PKV_MFMA_NBUF, PKV_MFMA_WAVES, QB>(p, stream);
  return launch_one<D, MfmaTile<D, 2>, PKV_MFMA_NBUF, PKV_MFMA_WAVES, QB>(p, stream);
}

}  // namespace

namespace {

// Workgroups of the decode / verify kernel that one round puts on the chip:
// the CUs times the workgroups one CU holds (its LDS decides).
long attn_slots(const AttnPlan& pl) {
  int smem;
  if (pl.mfma)
    smem = pl.rows <= 32 ? KernelCfg<128, MfmaTile<128, 1>, PKV_MFMA_NBUF, PKV_MFMA_WAVES>::SMEM
                         : KernelCfg<128, MfmaTile<128, 2>, PKV_MFMA_NBUF, PKV_MFMA_WAVES>::SMEM;
  else
    smem = KernelCfg<128, ValuTile<128, 1>, PKV_VALU_NBUF, PKV_VALU_WAVES>::SMEM;
  const int per_cu = kLdsPerCu / smem;
  return (long)kNumCu * (per_cu < 1 ? 1 : per_cu);
}

constexpr int kMaxPps = 64;  // the kernel stages at most 64 table entries per split

}  // namespace

AttnPlan attn_plan(int B, int Hkv, int W, int max_q_len, int group, long total_pages, int pages_per_split) {
  AttnPlan pl{};
  pl.rows = max_q_len * group;
  // VALU dot products for up to 4 rows (decode with a group of 4); from 5
  // rows the matrix cores: measured on 8 x 8192 tokens, 8 rows 70.0 -> 56.1
  // us and 12 rows 95.7 -> 56.3 us, where the VALU tile's per-row work stops
  // hiding under the K/V stream
  pl.mfma = pl.rows > kValuMaxRows;
  pl.prefill = pl.rows > PKV_MAX_ROWS;
  pl.qtok = kPrefillRows / group;
  pl.tiles = (max_q_len + pl.qtok - 1) / pl.qtok;
  if (pl.prefill) {  // no split of the key range, no partials
    pl.pps = W;
    pl.max_splits = 1;
    return pl;
  }
  const long pages = total_pages > 0 ? total_pages : (long)B * W;
  long pps;
  if (pages_per_split > 0) {
    pps = pages_per_split;  // the caller's plan (attn_best_pps on its lengths)
  } else {
    // As few splits as keep one round of workgroups on every CU. Each extra
    // split costs a partial write and read plus a merge; an idle CU costs
    // more. The pages the batch references (the caller's count, else the
    // table width for every row) spread over the CUs.
    const long slots = attn_slots(pl);
    pps = (pages * Hkv + slots - 1) / slots;
  }
  if (PKV_FORCE_PPS > 0) pps = PKV_FORCE_PPS;
  if (pps < 1) pps = 1;
  if (pps > W) pps = W;
  if (pps > kMaxPps) pps = kMaxPps;
  pl.pps = (int)pps;
  pl.max_splits = (W + pl.pps - 1) / pl.pps;
  return pl;
}

int attn_best_pps(int B, int Hkv, int W, int max_q_len, int group, int D, const int32_t* seq_lens) {
  AttnPlan pl = attn_plan(B, Hkv, W, max_q_len, group, 0, 0);
  if (pl.prefill) return 0;
  const long slots = attn_slots(pl);
  // A workgroup's fixed cost (table and q loads before its first page
  // arrives, the output or partial stores after its last), in page-stream
  // times: about 11 us against 5 us per 128 KiB page of K and V (head_dim
  // 128) at a CU's share of the HBM rate. A batch with any sequence cut into
  // several splits also waits for their merge (the partial stores'
  // acknowledgement, the count, the last split's loads): about half that.
  const long overhead = D >= 128 ? 2 : 4;
  const long merge = overhead / 2;
  const int top = W < kMaxPps ? W : kMaxPps;
  long best_cost = -1;
  int best = 1;
  for (int pps = 1; pps <= top; ++pps) {
    long busy = 0;
    bool split = false;
    for (int b = 0; b < B; ++b) {
      long n = seq_lens[b] > 0 ? seq_lens[b] : 0;
      if (n > (long)W * kPage) n = (long)W * kPage;
      const long pages = (n + kPage - 1) / kPage;
      busy += (pages + pps - 1) / pps;
      split |= pages > pps;
    }
    busy *= Hkv;
    long rounds = (busy + slots - 1) / slots;
    if (rounds < 1) rounds = 1;
    // a split's time ~ its pages plus the fixed cost (and the merge); ties
    // go to longer splits (fewer partials to merge)
    const long cost = rounds * (pps + overhead + (split ? merge : 0));
    if (best_cost < 0 || cost <= best_cost) {
      best_cost = cost;
      best = pps;
    }
  }
  return best;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

AttnWorkspace attn_workspace(int B, int Hkv, int W, int max_q_len, int group, int D, long total_pages,
                             int pages_per_split) {
  const AttnPlan pl = attn_plan(B, Hkv, W, max_q_len, group, total_pages, pages_per_split);
  AttnWorkspace ws;
  const size_t items = pl.prefill ? 0 : (size_t)B * Hkv * pl.max_splits;
  ws.err_off = 0;
  ws.counters_off = 256;
  ws.ml_off = align_up(ws.counters_off + (size_t)B * Hkv * 4, 256);
  ws.acc_off = align_up(ws.ml_off + items * pl.rows * 2 * 4, 256);
  ws.total = align_up(ws.acc_off + items * pl.rows * (size_t)D * 4, 256);
  return ws;
}

SharedPlan shared_plan(int Hkv, int total_q, int group, int shared_pages) {
  SharedPlan sp;
  const int rows = total_q * group;
  // Few rows per KV head (decode and verify batches): the decode / verify
  // kernel's matrix-core row tile over key splits of whole pages, each of its
  // waves streaming a private ring, one round of workgroups. There a 256-row
  // tile would be mostly padding and its split too short to fill its ring.
  {
    const int tr = rows <= 32 ? 32 : 64;
    const long tiles = (long)Hkv * ((rows + tr - 1) / tr);
    const int smem = tr == 32 ? KernelCfg<128, MfmaTile<128, 1>, PKV_MFMA_NBUF, PKV_MFMA_WAVES>::SMEM
                              : KernelCfg<128, MfmaTile<128, 2>, PKV_MFMA_NBUF, PKV_MFMA_WAVES>::SMEM;
    const long slots = (long)kNumCu * (kLdsPerCu / smem < 1 ? 1 : kLdsPerCu / smem);
    long splits = slots / tiles;
    if (splits > shared_pages) splits = shared_pages;
    if (PKV_SHARED_ROW_TILE && splits >= 2) {
      int pps = (int)((shared_pages + splits - 1) / splits);
      if (pps > kMaxPps) pps = kMaxPps;  // the kernel stages at most kMaxPps table entries per split
      sp.tile_rows = tr;
      sp.row_tiles = (rows + tr - 1) / tr;
      sp.split_keys = pps * kPage;
      sp.splits = (shared_pages + pps - 1) / pps;
      return sp;
    }
  }
  sp.tile_rows = 0;
  sp.row_tiles = (rows + kPrefillRows - 1) / kPrefillRows;
  const int chunks = shared_pages * kPage / 32;
  // about one workgroup per CU (one fits: the ring takes most of the LDS),
  // at least 4 chunks of 32 keys per split
  const long tiles = (long)Hkv * sp.row_tiles;
  long splits = (PKV_SHARED_WG + tiles - 1) / tiles;
  if (splits > chunks / 4) splits = chunks / 4;
  if (splits < 1) splits = 1;
  const int per = (int)((chunks + splits - 1) / splits);
  sp.split_keys = per * 32;
  sp.splits = (chunks + per - 1) / per;
  return sp;
}

template <int D, int NRB>
hipError_t launch_shared_rows(const AttnParams& p, const SharedParams& sp, hipStream_t stream) {
  AttnParams q = p;
  q.part_ml = sp.part_ml;
  q.part_acc = sp.part_acc;
  q.pps = sp.split_keys / kPage;
  q.max_splits = sp.splits;
  q.page_offset = sp.shared_pages;
  q.num_items = p.Hkv * sp.row_tiles * sp.splits;
  hipLaunchKernelGGL((attn_split_kernel<D, MfmaTile<D, NRB>, PKV_MFMA_NBUF, PKV_MFMA_WAVES, 0, true>),
                     dim3(q.num_items), dim3(PKV_MFMA_WAVES * 64), 0, stream, q.block_table, q.seq_lens, q.q_lens,
                     q.num_items, q.B, q.Hkv, q.pps, q.W, q);
  return hipGetLastError();
}

hipError_t launch_attn_shared(const AttnParams& p, const SharedParams& sp, hipStream_t stream) {
  if (sp.tile_rows == 32)
    return p.D == 64 ? launch_shared_rows<64, 1>(p, sp, stream) : launch_shared_rows<128, 1>(p, sp, stream);
  if (sp.tile_rows == 64)
    return p.D == 64 ? launch_shared_rows<64, 2>(p, sp, stream) : launch_shared_rows<128, 2>(p, sp, stream);
  const unsigned grid = (unsigned)((long)p.Hkv * sp.row_tiles * sp.splits);
  if (p.D == 64)
    hipLaunchKernelGGL((attn_shared_kernel<64, PKV_PREFILL_NBUF, kLongNrb<64>>), dim3(grid),
                       dim3(kLongWaves<kLongNrb<64>> * 64), 0, stream, sp, p);
  else
    hipLaunchKernelGGL((attn_shared_kernel<128, PKV_PREFILL_NBUF, kLongNrb<128>>), dim3(grid),
                       dim3(kLongWaves<kLongNrb<128>> * 64), 0, stream, sp, p);
  return hipGetLastError();
}

hipError_t launch_shared_merge(const AttnParams& p, const SharedParams& sp, hipStream_t stream) {
  const long n = (long)p.total_q * p.Hq * (p.D / 4);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (p.D == 64)
    hipLaunchKernelGGL((shared_merge_kernel<64>), dim3(grid), dim3(256), 0, stream, sp, p);
  else
    hipLaunchKernelGGL((shared_merge_kernel<128>), dim3(grid), dim3(256), 0, stream, sp, p);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnParams& p, const AttnPlan& plan, hipStream_t stream) {
  if (p.num_items == 0) return hipSuccess;
  if (plan.prefill) {
    if (p.D == 64)
      hipLaunchKernelGGL((attn_prefill_kernel<64, PKV_PREFILL_NBUF, kLongNrb<64>>), dim3(p.num_items),
                         dim3(kLongWaves<kLongNrb<64>> * 64), 0, stream, p.block_table, p.seq_lens, p.q_lens, p.B,
                         p.Hkv, plan.qtok, p.W, p);
    else
      hipLaunchKernelGGL((attn_prefill_kernel<128, PKV_PREFILL_NBUF, kLongNrb<128>>), dim3(p.num_items),
                         dim3(kLongWaves<kLongNrb<128>> * 64), 0, stream, p.block_table, p.seq_lens, p.q_lens, p.B,
                         p.Hkv, plan.qtok, p.W, p);
    return hipGetLastError();
  }
  if (p.D == 64) return launch_d<64, 0>(p, plan, stream);
  return launch_d<128, 0>(p, plan, stream);
}

hipError_t launch_attn_quant(const AttnParams& p, const AttnPlan& plan, int qbits, hipStream_t stream) {
  if (p.num_items == 0) return hipSuccess;
  if (plan.prefill || (qbits != 8 && qbits != 4)) return hipErrorInvalidValue;  // decode / verify rows only
  if (qbits == 8) return p.D == 64 ? launch_d<64, 8>(p, plan, stream) : launch_d<128, 8>(p, plan, stream);
  return p.D == 64 ? launch_d<64, 4>(p, plan, stream) : launch_d<128, 4>(p, plan, stream);
}

}  // namespace pkv
