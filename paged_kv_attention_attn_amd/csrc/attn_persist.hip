// Persistent paged attention for decode and verify windows on gfx950.
//
// Sources: ExLlamaV2 "Dynamic Generator" page, "Continuous Batching" (256-token
// pages reached through per-sequence block tables, indices need not be
// contiguous) and "Deduplication" (pages shared between sequences); Hugging
// Face "Assisted Generation" page, "How Assisted Generation works" (one pass
// over the cache scores every position of the draft window). The pages give no
// kernel design; this one is the library's own.
//
// Why persistent. Decode and verify read every cached K/V byte once, so the
// kernel is bound by HBM. A one-shot grid (one work item per workgroup) ends
// on its slowest compute units: the eight XCDs stream at different rates, and
// every workgroup pays its start-up and merge latency on the critical path.
// Here each compute unit runs one workgroup for the whole call and takes work
// units (sequence b, KV head g, unit s of U pages) from an atomic ticket, so
// fast XCDs take more units; the next unit's K/V streams in while the current
// one is computed.
//
// Workgroup = four compute waves + one scheduler wave.
//  * The compute waves take the 32-token chunks of a unit in turn (chunk c to
//    wave c % 4), each through a private ring of LDS slots filled by direct
//    buffer->LDS loads, each with its own softmax state over all q rows of the
//    unit and all head dims: four independent chunk streams per compute unit,
//    so one wave's latencies hide behind the others' work. At the end of a
//    unit the four partial results are merged in LDS in wave order (a fixed
//    chain w0, w1, w2, w3), so the result never depends on timing.
//  * The scheduler wave owns everything that waits on global memory outside
//    the K/V stream: the ticket atomic, the q rows of the next units (direct
//    loads into LDS), and the stores of each merged unit (its output rows, or
//    its partial for the cross-unit merge). The compute waves issue no other
//    memory operations, so their hand-counted waits on the K/V loads stay
//    exact; they never wait on the scheduler's round trips.
//  * Waves synchronise through counters in LDS, never through s_barrier.
//
// Determinism. A unit's result depends only on the unit's keys (fixed chunk
// to wave assignment, fixed merge chain), never on which workgroup ran it or
// what ran before it, and persist_merge_kernel combines the units of a
// (b, g) pair in unit order. Results are bit-identical under any assignment
// of units to compute units.

#include "device.h"

namespace pkv {
namespace {

constexpr int kPRows = 32;      // q rows of the tile: one 32-row MFMA block (q_len x head group)
constexpr int kPWaves = 4;      // compute waves
constexpr int kPQueue = 8;      // unit queue entries in LDS
constexpr int kPQBufs = 2;      // q row buffers in LDS
constexpr int kPLookahead = 1;  // units published ahead of the one wave 0 issues from
constexpr int kPSpin = 1 << 22; // polls before a wait gives up (a broken invariant, never reached)
constexpr int kPThreads = (kPWaves + 1) * 64;

template <int D>
struct PCfg {
  static constexpr int TC = 32;  // tokens per chunk
  using G = TileGeom<D, TC>;
  static constexpr int NC = G::NC;
  static constexpr int RB = G::RB;
  static constexpr int TILE = G::TILE;  // bytes of one K (or V) chunk
  static constexpr int SLOT = 2 * TILE;
  static constexpr int NI = G::NI;      // 1 KiB loads per K (or V) chunk
  static constexpr int OPS = 2 * NI;    // load instructions per chunk
};

// One published work unit. u < 0 marks the end of the workgroup's queue.
struct PEntry {
  int32_t u, b, g, s;
  int32_t seq_len, q_len, q_start, n_units;  // n_units: units of the (b, g) pair
  int32_t n_chunks, qready, pad0, pad1;
};

struct PCtrl {
  int32_t qdone[4];  // per compute wave: units it has finished (q rows no longer read)
  int32_t chain;     // merge chain position: 4 j + w once waves < w have merged unit j
  int32_t tail;      // entries the scheduler has published
  int32_t iu;        // unit compute wave 0 issues from
  int32_t sfree;     // units whose merged result the scheduler has stored
  int32_t scan[16];  // block-scan scratch
  PEntry q[kPQueue];
};

typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

__device__ __forceinline__ int lds_ld(const int32_t* p) { return *(volatile const lds_i32*)(p); }
__device__ __forceinline__ void lds_st(int32_t* p, int v) { *(volatile lds_i32*)(p) = v; }
// Four consecutive words (16-byte aligned) in one LDS read.
__device__ __forceinline__ i32x4 lds_ld4(const int32_t* p) { return *(volatile const lds_i32x4*)(p); }

__device__ __forceinline__ int lds_min4(const int32_t* a) {
  const i32x4 v = lds_ld4(a);
  return min(min(v.x, v.y), min(v.z, v.w));
}

// Spin (sleeping between polls) until *a >= v. False after kPSpin polls,
// which only a broken invariant could cause.
__device__ __forceinline__ bool spin_ge(const int32_t* a, int v) {
  for (int i = 0; i < kPSpin; ++i) {
    if (lds_ld(a) >= v) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Wait until at most n (a multiple of 4 in 0..60) of this wave's vector
// memory operations are outstanding.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define PKV_W(i) \
  case i: wait_vmcnt<i>(); break;
    PKV_W(60) PKV_W(56) PKV_W(52) PKV_W(48) PKV_W(44) PKV_W(40) PKV_W(36) PKV_W(32) PKV_W(28) PKV_W(24)
    PKV_W(20) PKV_W(16) PKV_W(12) PKV_W(8) PKV_W(4)
#undef PKV_W
    default: wait_vmcnt<0>();
  }
}

// Row tile of one compute wave: 32 q rows x all D dims. Scores S^T = K.Q^T
// put one q row in each lane column (lane % 32), so the softmax state is per
// lane. Softmax in base 2 with a lazy reference max: a row keeps its max m
// until a chunk exceeds it by 2^8, so P = 2^(x - m) may reach 2^8 and the
// weights' ratios are unchanged; the rare rescale multiplies the
// accumulators. Row sums come from the matrix cores (an all-ones block in
// place of V^T), over the same bf16 P that multiplies V, so each output row is
// an exact weighted mean of the rounded weights. Where a key could weigh more
// than 1/8 of its row sum so far, P enters as two bf16 terms (its rounding and
// the remainder), about 16 significant bits.
template <int D>
struct WTile {
  static constexpr int NC = D / 8;
  static constexpr int KK = D / 16;  // k-steps of the score product
  static constexpr int MB = D / 32;  // 32-dim blocks of the output
  static constexpr float kLazyLog2 = 8.f;
  static constexpr float kSplitWeight = 1.f / 8.f;

  const char* qlds;  // the unit's q rows in LDS (swizzled like the K tiles)
  int rows;
  float m;
  int lim;
  f32x16 acc[MB], lacc;
  float xs[16], cmax;
  u32x4 pb[2], pl[2];

  // rows r < rows are window token r / group, visible keys 0 .. lim; the q
  // rows stay in LDS for the whole unit (padding rows repeat the last one:
  // their scores are finite and never stored)
  __device__ __forceinline__ void begin(const char* q, int group, int nrows, int seq_len, int q_len) {
    const int row = threadIdx.x & 31;
    qlds = q;
    rows = nrows;
    m = kNegInf;
    lim = row < rows ? seq_len - q_len + row / group : -1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][i] = 0.f;
      lacc[i] = 0.f;
    }
  }

  // S^T = K.Q^T on the matrix cores, K rows (lane row = token) and q rows
  // read from LDS as the A and B operands.
  __device__ __forceinline__ void qk(f32x16& S, const char* kt) const {
    int lane = threadIdx.x & 63;
    // recomputed per chunk: hoisting the per-lane operand addresses out of the
    // chunk loop would cost more registers than their arithmetic costs time
    asm volatile("" : "+v"(lane));
    const int row = lane & 31, half = lane >> 5;
    const int qrow = min(row, rows - 1);
    const u32x4* ql = reinterpret_cast<const u32x4*>(qlds);
    const u32x4* kl = reinterpret_cast<const u32x4*>(kt);
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
    // operands read in batches of KB k-steps: all reads of a batch issued
    // before its products
    constexpr int KB = KK / 2;
#pragma unroll
    for (int k0 = 0; k0 < KK; k0 += KB) {
      u32x4 kv[KB], qv[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int c = 2 * (k0 + j) + half;
        kv[j] = kl[row * NC + (c ^ (row & (NC - 1)))];
        qv[j] = ql[qrow * NC + (c ^ (qrow & (NC - 1)))];
      }
#pragma unroll
      for (int j = 0; j < KB; ++j)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv[j]), __builtin_bit_cast(bf16x8, qv[j]),
                                                    S, 0, 0, 0);
    }
  }

  // V^T of the chunk at k-step ks as the A operands of O^T, va[mb] for dims
  // [32 mb, 32 mb + 32), by transposing LDS reads
  // (ds_read_b64_tr_b16): within each 16-lane group, destination lane i
  // receives element i % 4 of source lanes i / 4, i / 4 + 4, i / 4 + 8,
  // i / 4 + 12. With source lane j at token t0 + j / 4, dims d0 + 4 (j % 4) ..
  // + 3, lane i gets tokens t0 .. t0 + 3 of dim d0 + i; k index j of lane half
  // h at k-step ks is token 16 ks + 8 (j / 4) + 4 h + j % 4, where P sits in
  // the S^T result. All reads are issued before any is used.
  __device__ __forceinline__ void vt_operands(const char* vt, int ks, u32x4 (&va)[MB]) const {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));  // recomputed per chunk (see qk)
    const int half = lane >> 5;
    const int tq = (lane & 15) >> 2;
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int d = mb * 32 + dsub;
      u32x2 w[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int t = 16 * ks + 8 * hh + 4 * half + tq;
        const char* src = vt + (t * NC + ((d >> 3) ^ (t & (NC - 1)))) * 16 + (d & 7) * 2;
        w[hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src));
      }
      va[mb] = u32x4{w[0].x, w[0].y, w[1].x, w[1].y};
    }
  }

  // Scaled scores S^T * scale * log2(e) (masked unless MASK is false, for
  // chunks every row sees in full) into xs and the chunk's row maxima into
  // cmax; whether some row of the wave outgrew its reference max by 2^8. This
  // lane holds tokens 8 (i / 4) + 4 half + i % 4.
  template <bool MASK>
  __device__ __forceinline__ bool scores(const f32x16& S, int tok0, int nv, float scale_log2) {
    const int half = (threadIdx.x & 63) >> 5;
    float cm = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tt = 8 * (i >> 2) + 4 * half + (i & 3);
      if constexpr (MASK)
        xs[i] = (tok0 + tt <= lim && tt < nv) ? S[i] * scale_log2 : kNegInf;
      else
        xs[i] = S[i] * scale_log2;
      cm = fmaxf(cm, xs[i]);
    }
    cmax = max_xor32(cm);
    return __builtin_amdgcn_ballot_w64(cmax > m + kLazyLog2) != 0;
  }

  // moves the reference max of the rows that outgrew it and rescales their
  // sums and accumulators
  __device__ __forceinline__ void rescale() {
    const bool g = cmax > m + kLazyLog2;
    const float alpha = g ? exp2f_fast(m - cmax) : 1.f;
    m = g ? cmax : m;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
    lacc *= alpha;
  }

  // whether some row of the wave has a key of this chunk weighing more than
  // kSplitWeight of its row sum so far (a key's final weight is only lower)
  __device__ __forceinline__ bool needs_split() const {
    const float mu = (m == kNegInf) ? 0.f : m;
    return __builtin_amdgcn_ballot_w64(exp2f_fast(cmax - mu) > kSplitWeight * lacc[0]) != 0;
  }

  template <bool SPLIT>
  __device__ __forceinline__ void probs() {
    const float mu = (m == kNegInf) ? 0.f : m;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = exp2f_fast(xs[i] - mu);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = pack_bf16(p[8 * ks + 2 * e], p[8 * ks + 2 * e + 1]);
      pb[ks] = u32x4{h[0], h[1], h[2], h[3]};
      if constexpr (SPLIT) {
        u32 lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lo[e] = pack_bf16(p[8 * ks + 2 * e] - bf16lo(h[e]), p[8 * ks + 2 * e + 1] - bf16hi(h[e]));
        pl[ks] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
    }
  }

  // O^T += V^T . P^T and the row sums, from probs() and the V tile in LDS
  template <bool SPLIT>
  __device__ __forceinline__ void pv(const char* vt) {
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 va[MB];
      vt_operands(vt, ks, va);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mb]),
                                                          __builtin_bit_cast(bf16x8, pb[ks]), acc[mb], 0, 0, 0);
        if constexpr (SPLIT)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mb]),
                                                            __builtin_bit_cast(bf16x8, pl[ks]), acc[mb], 0, 0, 0);
      }
      lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ones),
                                                     __builtin_bit_cast(bf16x8, pb[ks]), lacc, 0, 0, 0);
      if constexpr (SPLIT)
        lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ones),
                                                       __builtin_bit_cast(bf16x8, pl[ks]), lacc, 0, 0, 0);
    }
  }

  // First half of a chunk of 32 keys at absolute token tok0 (nv inside the
  // sequence): the scores (K read from LDS) and the softmax update; after it
  // the K half of the slot is free. first: the wave's first chunk of the unit
  // (P in two terms, as its row sums hold few keys yet). Returns whether P
  // takes two terms.
  __device__ __forceinline__ bool scores_step(const char* kt, int tok0, int nv, bool mask, bool first,
                                              float scale_log2) {
    f32x16 S;
    qk(S, kt);
    const bool grow = mask ? scores<true>(S, tok0, nv, scale_log2) : scores<false>(S, tok0, nv, scale_log2);
    if (grow) rescale();
    return first || needs_split();
  }

  // Second half: P and P.V (V read from LDS); after it the V half is free.
  __device__ __forceinline__ void value_step(const char* vt, bool split) {
    if (split) {
      probs<true>();
      pv<true>(vt);
    } else {
      probs<false>();
      pv<false>(vt);
    }
  }
};

// Exclusive prefix sums of a[0..n) and c[0..n) in place, over the workgroup;
// a[n] and c[n] receive the totals. Each thread scans a contiguous segment.
__device__ void block_scan2(int32_t* a, int32_t* c, int n, int32_t* scratch) {
  constexpr int WAVES = kPThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (n + kPThreads - 1) / kPThreads;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int sa = 0, sc = 0;
  for (int i = lo; i < hi; ++i) {
    sa += a[i];
    sc += c[i];
  }
  int ia = sa, ic = sc;  // inclusive wave scans
  for (int d = 1; d < 64; d <<= 1) {
    const int ya = __builtin_amdgcn_ds_bpermute(((lane - d) & 63) << 2, ia);
    const int yc = __builtin_amdgcn_ds_bpermute(((lane - d) & 63) << 2, ic);
    if (lane >= d) {
      ia += ya;
      ic += yc;
    }
  }
  if (lane == 63) {
    scratch[wave] = ia;
    scratch[8 + wave] = ic;
  }
  __syncthreads();
  int oa = 0, oc = 0, ta = 0, tc = 0;
  for (int w = 0; w < WAVES; ++w) {
    if (w < wave) {
      oa += scratch[w];
      oc += scratch[8 + w];
    }
    ta += scratch[w];
    tc += scratch[8 + w];
  }
  int ra = oa + ia - sa, rc = oc + ic - sc;
  for (int i = lo; i < hi; ++i) {
    const int va = a[i], vc = c[i];
    a[i] = ra;
    c[i] = rc;
    ra += va;
    rc += vc;
  }
  if (threadIdx.x == 0) {
    a[n] = ta;
    c[n] = tc;
  }
  __syncthreads();
}

// The sequence that owns unit u: the last b with upre[b] <= u (upre is the
// exclusive prefix of units per sequence, upre[B] = total > u). One wave.
__device__ __forceinline__ int owner_seq(const int32_t* upre, int B, int u) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int i0 = 0; i0 <= B; i0 += 64) {
    const int i = i0 + lane;
    const bool le = i <= B && upre[i] <= u;
    cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
  }
  return cnt - 1;
}

template <int D>
__global__ __launch_bounds__(kPThreads) void attn_persist_kernel(
    // leading scalars, preloaded into SGPRs at wave launch
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_lens, int B, int Hkv, int W, int U, int nb, AttnParams p, PersistLayout L) {
  using C = PCfg<D>;
  constexpr int NC = C::NC;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* qarea = smem + L.off_q;
  char* stage = smem + L.off_stage;
  PCtrl* ctl = reinterpret_cast<PCtrl*>(smem + L.off_ctrl);
  int32_t* s_upre = reinterpret_cast<int32_t*>(smem + L.off_seq);  // [B + 1] units before sequence b
  int32_t* s_qpre = s_upre + (B + 1);                              // [B + 1] window rows before b
  int32_t* s_len = s_qpre + (B + 1);                               // [B] seq_len, or -1 if skipped
  int32_t* s_ql = s_len + B;                                       // [B] q_len
  int32_t* s_tab = s_ql + B;                                       // [B * W] block table
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rows_max = p.rows_max;
  // merged unit: acc [rows_max][kSRow], then (m, l) [rows_max]; the row pitch
  // of D + 4 floats puts a column's 32 rows in distinct banks
  constexpr int kSRow = D + 4;
  float* sacc = reinterpret_cast<float*>(stage);
  float* sml = sacc + rows_max * kSRow;

  // ---- start-up: lengths, windows and the table into LDS; per-sequence units
  // and window rows; their prefix sums. Broken per-sequence contracts skip the
  // sequence (no units) and are flagged by workgroup 0.
  u32 flags = 0;
  for (int i = threadIdx.x; i < B * W; i += kPThreads) s_tab[i] = block_table[i];
  for (int b = threadIdx.x; b < B; b += kPThreads) {
    const int len = seq_lens[b], ql = q_lens[b];
    const int npg = len > 0 ? (len + kPage - 1) / kPage : 0;
    bool ok = ql > 0;
    if (ql < 0 || (ql > 0 && (ql > p.max_q_len || ql > len || npg > W))) {
      flags |= PKV_EFLAG_QLEN_BIT;
      ok = false;
    }
    s_len[b] = ok ? len : -1;
    s_ql[b] = ql;
    s_upre[b] = ok ? Hkv * ((npg + U - 1) / U) : 0;
    s_qpre[b] = ql > 0 ? ql : 0;
  }
  if (threadIdx.x < 4) lds_st(&ctl->qdone[threadIdx.x], 0);
  if (threadIdx.x == 0) {
    lds_st(&ctl->chain, 0);
    lds_st(&ctl->tail, 0);
    lds_st(&ctl->iu, 0);
    lds_st(&ctl->sfree, 0);
  }
  __syncthreads();
  block_scan2(s_upre, s_qpre, B, ctl->scan);
  // table entries a sequence needs must name a pool page; a bad one reads as
  // zeros (the sequence's rows are then undefined) and is flagged
  for (int i = threadIdx.x; i < B * W; i += kPThreads) {
    const int b = i / W, j = i - b * W;
    const int len = s_len[b];
    if (len > 0 && j < (len + kPage - 1) / kPage) {
      const int e = s_tab[i];
      if (e < 0 || e >= p.P) {
        s_tab[i] = -1;
        flags |= PKV_EFLAG_PAGE_BIT;
      }
    }
  }
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0 && s_qpre[B] != p.total_q) flags |= PKV_EFLAG_ROWS_BIT;
    if (flags) atomicOr(p.err, flags);
  }
  __syncthreads();
  const int n_units = s_upre[B];

  auto entry = [&](int j) -> PEntry* { return &ctl->q[j & (kPQueue - 1)]; };

  if (wave == kPWaves) {
    // =========================== scheduler wave ===========================
    int tail = 0, sj = 0;
    bool first = true, ended = false;
    const u32 q_bytes = (u32)p.total_q * p.Hq * D * 2;
    const u32x4 rq = make_rsrc(p.q, q_bytes);
    for (int idle = 0; idle < kPSpin;) {
      bool did = false;
      // store the oldest unit once the last wave of the chain has merged it
      if (sj < tail && lds_ld(&ctl->chain) >= kPWaves * (sj + 1)) {
        const PEntry* e = entry(sj);
        const i32x4 f0 = lds_ld4(&e->u), f1 = lds_ld4(&e->seq_len);
        const int b = f0.y, g = f0.z, s = f0.w;
        const int q_len = f1.y, q_start = f1.z, nu = f1.w;
        const int rows = q_len * p.group;
        constexpr int D4 = D / 4;
        if (nu == 1) {  // the pair's only unit: normalised rows straight to out
          for (int e4 = lane; e4 < rows * D4; e4 += 64) {
            const int r = e4 / D4, dq = e4 - r * D4;
            const f32x4 a = *reinterpret_cast<const f32x4*>(sacc + r * kSRow + 4 * dq);
            const float lr = sml[2 * r + 1];
            const int h = g * p.group + r % p.group;
            *reinterpret_cast<f32x4*>(p.out + ((size_t)(q_start + r / p.group) * p.Hq + h) * D + 4 * dq) = a / lr;
          }
        } else {
          const size_t pidx = ((size_t)b * Hkv + g) * p.max_splits + s;
          float* pacc = p.part_acc + pidx * rows_max * D;
          float* pml = p.part_ml + pidx * rows_max * 2;
          for (int e4 = lane; e4 < rows * D4; e4 += 64) {
            const int r = e4 / D4, dq = e4 - r * D4;
            *reinterpret_cast<f32x4*>(pacc + 4 * e4) = *reinterpret_cast<const f32x4*>(sacc + r * kSRow + 4 * dq);
          }
          if (lane < rows) *reinterpret_cast<f32x2*>(pml + 2 * lane) = *reinterpret_cast<const f32x2*>(sml + 2 * lane);
        }
        wait_lgkm0();  // the merged values are in registers: the stage may be refilled
        ++sj;
        lds_st(&ctl->sfree, sj);
        did = true;
      }
      // publish the next unit while wave 0 issues from within kPLookahead units
      // of the queue's end, an entry slot and a q buffer are free
      if (!ended && tail - lds_ld(&ctl->iu) < kPLookahead && tail - sj < kPQueue &&
          (tail < kPQBufs || lds_min4(ctl->qdone) >= tail - kPQBufs + 1)) {
        int u;
        if (first) {
          u = blockIdx.x;
          first = false;
        } else {
          // one lane takes the ticket (a wave-wide atomic would take 64)
          int t = 0;
          if (lane == 0) t = (int)__hip_atomic_fetch_add(p.counters, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          u = (int)gridDim.x + __builtin_amdgcn_readfirstlane(t);
        }
        PEntry* e = entry(tail);
        if (u >= n_units) {
          lds_st(&e->u, -1);
          wait_lgkm0();
          ++tail;
          lds_st(&ctl->tail, tail);
          ended = true;
        } else {
          const int b = owner_seq(s_upre, B, u);
          const int r = u - s_upre[b];
          const int seq_len = s_len[b], q_len = s_ql[b], q_start = s_qpre[b];
          const int npg = (seq_len + kPage - 1) / kPage;
          const int per = (npg + U - 1) / U;  // units of each (b, g) pair
          const int g = r / per, s = r - g * per;
          if (q_start + q_len > p.total_q) {  // rows past out: skipped, flagged
            if (lane == 0) atomicOr(p.err, PKV_EFLAG_ROWS_BIT);
            continue;
          }
          const int t0 = s * U * kPage;
          const int t1 = min(seq_len, t0 + U * kPage);
          lds_st(&e->u, u);
          lds_st(&e->b, b);
          lds_st(&e->g, g);
          lds_st(&e->s, s);
          lds_st(&e->seq_len, seq_len);
          lds_st(&e->q_len, q_len);
          lds_st(&e->q_start, q_start);
          lds_st(&e->n_units, per);
          lds_st(&e->n_chunks, (t1 - t0 + C::TC - 1) / C::TC);
          lds_st(&e->qready, 0);
          wait_lgkm0();
          ++tail;
          lds_st(&ctl->tail, tail);
          // q rows of (b, g) into the unit's q buffer, swizzled like the K
          // tiles; rows past the window read out of range as zeros
          const int rows = q_len * p.group;
          const int ops = (rows * NC + 63) / 64;
          const u32 qbase = lds_addr_of(qarea + ((tail - 1) & (kPQBufs - 1)) * L.qbytes);
          for (int i = 0; i < ops; ++i) {
            const int pc = i * 64 + lane;
            const int rr = pc / NC, pos = pc % NC;
            u32 off = q_bytes;
            if (rr < rows) {
              const int c = pos ^ (rr & (NC - 1));
              off = (u32)(((q_start + rr / p.group) * p.Hq + g * p.group + rr % p.group) * D) * 2u + c * 16;
            }
            dma16(rq, off, uniform(qbase + i * 1024));
          }
          wait_vmcnt<0>();
          lds_st(&e->qready, 1);
        }
        did = true;
      }
      if (ended && sj == tail - 1) break;
      if (did) {
        idle = 0;
      } else {
        ++idle;
        __builtin_amdgcn_s_sleep(8);  // it shares a SIMD with a compute wave
      }
    }
    return;
  }

  // ============================ compute waves ============================
  const int w = wave;
  char* ring = smem + w * nb * C::SLOT;
  const u32 ring_lds = lds_addr_of(ring);
  u32 voff[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int slot = i * 64 + lane;
    const int t = slot / NC, pos = slot % NC;
    voff[i] = t * C::RB + ((pos ^ (t & (NC - 1))) * 16);
  }
  const float scale_log2 = p.scale_log2;

  // This wave's chunk stream: its chunks of each unit in turn. A slot's K
  // half is refilled as soon as the scores have read it, its V half once P.V
  // has; the loads of chunk j are issued K then V, before any of chunk j + 1.
  int c_k = 0, c_v = 0;  // chunks whose K / V half this wave has issued
  int iu = 0, ic = w;    // issue cursor: unit, chunk within it
  bool i_open = false;   // the issue unit's fields are loaded
  int i_b = 0, i_g = 0, i_t0 = 0, i_len = 0, i_nch = 0;
  int known_tail = 0;
  bool i_ended = false;
  u32x4 pend_rv = {0u, 0u, 0u, 0u};  // V descriptor and slot of chunk c_v while c_v < c_k
  u32 pend_base = 0;

  // Published entry j (waits for the scheduler); false at the end of the queue.
  auto wait_entry = [&](int j) -> bool {
    for (int i = 0; j >= known_tail; ++i) {
      if (i >= kPSpin) return false;
      known_tail = lds_ld(&ctl->tail);
      if (j < known_tail) break;
      __builtin_amdgcn_s_sleep(1);
    }
    return lds_ld(&entry(j)->u) >= 0;
  };

  // K half of this wave's next chunk into its slot (the caller knows it is
  // free). False if the next unit is not published yet or the queue ended.
  auto issue_k = [&]() -> bool {
    while (!i_open) {
      if (i_ended) return false;
      if (iu >= known_tail) {
        known_tail = lds_ld(&ctl->tail);
        if (iu >= known_tail) return false;
      }
      const PEntry* e = entry(iu);
      const i32x4 f0 = lds_ld4(&e->u), f1 = lds_ld4(&e->seq_len), f2 = lds_ld4(&e->n_chunks);
      if (f0.x < 0) {
        i_ended = true;
        return false;
      }
      i_b = f0.y;
      i_g = f0.z;
      i_t0 = f0.w * U * kPage;
      i_len = f1.x;
      i_nch = f2.x;
      if (w < i_nch) {
        ic = w;
        i_open = true;
      } else {  // no chunk of this unit for this wave
        ++iu;
        if (w == 0) lds_st(&ctl->iu, iu);
      }
    }
    const int t0 = i_t0 + ic * C::TC;
    const int phys = __builtin_amdgcn_readfirstlane(s_tab[i_b * W + (t0 >> 8)]);
    const int nvt = phys < 0 ? 0 : min(C::TC, i_len - t0);
    const size_t tok = ((size_t)(phys < 0 ? 0 : phys) * Hkv + i_g) * kPage + (t0 & (kPage - 1));
    const u32 bytes = nvt > 0 ? (u32)(nvt * C::RB) : 0u;
    const u32x4 rk = make_rsrc(p.k_pool + tok * D, bytes);
    pend_rv = make_rsrc(p.v_pool + tok * D, bytes);
    const u32 base = uniform(ring_lds + (c_k % nb) * C::SLOT);
    pend_base = uniform(base + C::TILE);
#pragma unroll
    for (int i = 0; i < C::NI; ++i) dma16(rk, voff[i], base + i * 1024);
    ++c_k;
    ic += kPWaves;
    if (ic >= i_nch) {
      i_open = false;
      ++iu;
      if (w == 0) lds_st(&ctl->iu, iu);
    }
    return true;
  };
  auto issue_v = [&]() {
    const u32x4 rv = {uniform(pend_rv.x), uniform(pend_rv.y), uniform(pend_rv.z), uniform(pend_rv.w)};
    const u32 vb = uniform(pend_base);
#pragma unroll
    for (int i = 0; i < C::NI; ++i) dma16(rv, voff[i], vb + i * 1024);
    ++c_v;
  };

  WTile<D> tile;
  int k = 0;  // this wave's chunks computed
  for (int ju = 0; ju < kPSpin; ++ju) {
    if (!wait_entry(ju)) break;
    const PEntry* e = entry(ju);
    const i32x4 f0 = lds_ld4(&e->u), f1 = lds_ld4(&e->seq_len), f2 = lds_ld4(&e->n_chunks);
    const int c_t0 = f0.w * U * kPage;
    const int c_len = f1.x, c_ql = f1.y, n_chunks = f2.x;
    const int rows = c_ql * p.group;
    // chunks starting before t_free hold only keys every row sees
    const int t_free = c_len - c_ql + 1 - C::TC;
    const bool mine = w < n_chunks;
    if (mine) {
      if (!spin_ge(&e->qready, 1)) return;
      tile.begin(qarea + (ju & (kPQBufs - 1)) * L.qbytes, p.group, rows, c_len, c_ql);
      for (int c = w; c < n_chunks; c += kPWaves) {
        // keep the ring full; this chunk must be in flight
        for (int i = 0; c_v < k + nb; ++i) {
          if (c_k == c_v && !issue_k()) {
            if (c_v > k) break;  // chunk k is in flight: go on
            if (i >= kPSpin) return;
            __builtin_amdgcn_s_sleep(1);  // the scheduler has not published its unit yet
            continue;
          }
          issue_v();
        }
        wait_vm((c_k + c_v - 2 - 2 * k) * C::NI);
        const char* slot = ring + (k % nb) * C::SLOT;
        const int t0 = c_t0 + c * C::TC;
        const bool split = tile.scores_step(slot, t0, min(C::TC, c_len - t0), t0 >= t_free, c < kPWaves, scale_log2);
        wait_lgkm0();  // the K half is free
        if (c_k == c_v && c_k < k + 1 + nb) issue_k();
        tile.value_step(slot + C::TILE, split);
        wait_lgkm0();  // the V half is free
        if (c_v < c_k) issue_v();
        ++k;
      }
    }
    // ---- merge chain for unit ju: wave 0 writes its result into the stage
    // (once the scheduler has stored the previous unit), each later wave with
    // keys in the unit folds its result in, in wave order
    if (w == 0 && !spin_ge(&ctl->sfree, ju)) return;
    if (!spin_ge(&ctl->chain, kPWaves * ju + w)) return;
    const int row = lane & 31, half = lane >> 5;
    if (mine && row < rows) {
      const float lw = tile.lacc[0];
      float fs = 0.f, fw = 1.f;
      float mo = tile.m, lo = lw;
      if (w > 0) {
        const f32x2 ml = *reinterpret_cast<const f32x2*>(sml + 2 * row);
        const float M = fmaxf(ml.x, tile.m);
        fs = ml.x == kNegInf ? 0.f : exp2f_fast(ml.x - M);
        fw = tile.m == kNegInf ? 0.f : exp2f_fast(tile.m - M);
        mo = M;
        lo = fs * ml.y + fw * lw;
      }
      constexpr int MB = WTile<D>::MB;
      f32x4* dst = reinterpret_cast<f32x4*>(sacc + row * kSRow + 4 * half);  // + 8 mb + 2 j (f32x4 units)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4 old[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) old[j] = w > 0 ? dst[8 * mb + 2 * j] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = {tile.acc[mb][4 * j], tile.acc[mb][4 * j + 1], tile.acc[mb][4 * j + 2],
                           tile.acc[mb][4 * j + 3]};
          dst[8 * mb + 2 * j] = fs * old[j] + fw * v;
        }
      }
      if (half == 0) *reinterpret_cast<f32x2*>(sml + 2 * row) = f32x2{mo, lo};
    }
    wait_lgkm0();  // this wave's stage writes and q reads of the unit are done
    lds_st(&ctl->qdone[w], ju + 1);
    lds_st(&ctl->chain, kPWaves * ju + w + 1);
  }
}

// Merge of the (b, g) pairs with more than one unit: out = sum_s 2^(m_s - M)
// acc_s / sum_s 2^(m_s - M) l_s over the pair's units in unit order. One
// thread per (row, 4 dims); it also resets the ticket for the next call.
template <int D>
__global__ __launch_bounds__(256) void persist_merge_kernel(const int32_t* __restrict__ seq_lens,
                                                            const int32_t* __restrict__ q_lens, int B, int Hkv,
                                                            int W, int U, AttnParams p) {
  constexpr int D4 = D / 4;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *p.counters = 0u;
  const int b = blockIdx.x / Hkv, g = blockIdx.x - b * Hkv;
  const int len = seq_lens[b], ql = q_lens[b];
  const int npg = len > 0 ? (len + kPage - 1) / kPage : 0;
  if (ql <= 0 || ql > p.max_q_len || ql > len || npg > W) return;
  const int n = (npg + U - 1) / U;
  if (n <= 1) return;
  // q_start: sum of the non-negative q_lens before b
  int qs = 0;
  {
    const int lane = threadIdx.x & 63;
    for (int i = lane; i < b; i += 64) qs += max(q_lens[i], 0);
    for (int m = 32; m >= 1; m >>= 1) qs += __builtin_amdgcn_ds_bpermute(((lane ^ m) << 2), qs);
  }
  if (qs + ql > p.total_q) return;
  const int rows = ql * p.group;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e >= rows * D4) return;
  const int r = e / D4, dq = e - r * D4;
  const size_t base = ((size_t)b * Hkv + g) * p.max_splits;
  constexpr int SB = 8;
  float M = kNegInf, Lsum = 0.f;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n; s0 += SB) {
    f32x2 ml[SB];
    f32x4 pa[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const int s = min(s0 + j, n - 1);
      ml[j] = *reinterpret_cast<const f32x2*>(p.part_ml + ((base + s) * p.rows_max + r) * 2);
      pa[j] = *reinterpret_cast<const f32x4*>(p.part_acc + ((base + s) * p.rows_max + r) * D + 4 * dq);
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < SB; ++j)
      if (s0 + j < n) Mn = fmaxf(Mn, ml[j].x);
    if (Mn == kNegInf) continue;
    const float f = (M == kNegInf) ? 0.f : exp2f_fast(M - Mn);
    Lsum *= f;
    A *= f;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const float wt = (s0 + j >= n || ml[j].x == kNegInf) ? 0.f : exp2f_fast(ml[j].x - Mn);
      Lsum += wt * ml[j].y;
      A += wt * pa[j];
    }
    M = Mn;
  }
  const int h = g * p.group + r % p.group;
  *reinterpret_cast<f32x4*>(p.out + ((size_t)(qs + r / p.group) * p.Hq + h) * D + 4 * dq) = A / Lsum;
}

template <int D>
hipError_t launch_d(const AttnParams& p, const AttnPlan& plan, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_persist_kernel<D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsPerCu);
    attr_set = true;
  }
  const PersistLayout& L = plan.layout;
  hipLaunchKernelGGL((attn_persist_kernel<D>), dim3(kNumCu), dim3(kPThreads), L.bytes, stream, p.block_table,
                     p.seq_lens, p.q_lens, p.B, p.Hkv, p.W, p.pps, plan.nb, p, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int blocks_y = (kPRows * D / 4 + 255) / 256;
  hipLaunchKernelGGL((persist_merge_kernel<D>), dim3(p.B * p.Hkv, blocks_y), dim3(256), 0, stream, p.seq_lens,
                     p.q_lens, p.B, p.Hkv, p.W, p.pps, p);
  return hipGetLastError();
}

}  // namespace

// LDS layout of the persistent kernel for a shape: each compute wave's ring
// of nb K/V chunks (the deepest of 2..4 that fits, with at most 128 KiB of
// ring in all), the q buffers, the merge stage, the control block, the
// per-sequence arrays and the table; false if it does not fit one compute
// unit's LDS.
bool persist_layout(int B, int W, int rows, int D, PersistLayout* L, int* nb) {
  if (rows > kPRows || rows < 1 || (D != 64 && D != 128)) return false;
  const int slot = 2 * 32 * D * 2;
  const int nc = D / 8;
  L->qbytes = (rows * nc + 63) / 64 * 1024;
  const long fixed = (long)kPQBufs * L->qbytes + (long)rows * (D + 6) * 4 + 16 + (long)sizeof(PCtrl) +
                     (4L * B + 2 + (long)B * W) * 4;
  for (int n = 4; n >= 2; --n) {
    const long ring = (long)kPWaves * n * slot;
    if (ring > 128 * 1024 || ring + fixed > kLdsPerCu) continue;
    *nb = n;
    L->off_q = (int)ring;
    L->off_stage = L->off_q + kPQBufs * L->qbytes;
    L->off_ctrl = (L->off_stage + rows * (D + 6) * 4 + 15) / 16 * 16;
    L->off_seq = L->off_ctrl + (int)sizeof(PCtrl);
    L->bytes = L->off_seq + (4 * B + 2 + B * W) * 4;
    return L->bytes <= kLdsPerCu;
  }
  return false;
}

hipError_t launch_attn_persist(const AttnParams& p, const AttnPlan& plan, hipStream_t stream) {
  return p.D == 64 ? launch_d<64>(p, plan, stream) : launch_d<128>(p, plan, stream);
}

}  // namespace pkv
