// Greedy speculative accept for gfx950: a vocab-wide argmax per logits row,
// then the left-to-right draft comparison with one kept base-model token and
// the draft-window update.
//
// Source: Hugging Face "Assisted Generation" page, "Assisted Generation loop":
// the base model's predictions are compared with the candidates from the
// left; at the first mismatch its own token is kept and the later candidates
// dropped; the window grows by 2 after a full match and shrinks by 1
// otherwise.
//
// Kernel 1 scans row chunks (an HBM-bound fp32 stream; one row alone is far
// too small to fill the chip, so rows are cut into chunks) and writes a
// (value, index) pair per chunk. Kernel 2 gives one wave per sequence: it
// merges the chunk pairs of the sequence's rows and applies the accept rule.
// argmax order: larger value first; NaN above every number; lower index on
// equal values (and between NaNs), so the result is exact and unique.

#include "internal.h"

#include <climits>

#include "pkv.h"

namespace pkv {
namespace {

using u32 = uint32_t;
constexpr int kThreads = 256;

// (a, ia) ranks before (b, ib): the larger value, a NaN above every number,
// the lower index on equal values (and between NaNs). Branch-free.
__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  const bool na = a != a, nb = b != b;
  const bool lt = ia < ib;
  const bool num = (a > b) | ((a == b) & lt);
  return (na & (!nb | lt)) | (!na & !nb & num);
}

// Running maximum of one thread that visits indices in increasing order: the
// first element is taken; a later one replaces the best only if strictly
// larger, or if it is the first NaN.
__device__ __forceinline__ void scan_one(float x, int e, float& bv, int& bi) {
  const bool take = (bi == INT_MAX) | (x > bv) | ((x != x) & (bv == bv));
  bv = take ? x : bv;
  bi = take ? e : bi;
}

__device__ __forceinline__ void shfl_pair(float& v, int& i, int m) {
  const int lane = threadIdx.x & 63;
  const float ov = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __float_as_int(v)));
  const int oi = __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

__device__ __forceinline__ void wave_best(float& v, int& i) {
  for (int m = 32; m >= 1; m >>= 1) shfl_pair(v, i, m);
}

#ifndef PKV_ARG_THREADS
#define PKV_ARG_THREADS 512
#endif
#ifndef PKV_ARG_UNROLL
#define PKV_ARG_UNROLL 8
#endif
constexpr int kArgThreads = PKV_ARG_THREADS;  // threads per argmax workgroup
constexpr int kArgUnroll = PKV_ARG_UNROLL;    // float4 loads in flight per thread
constexpr int kSc1 = 16;       // cache-policy bit: coherent across XCDs

__device__ __forceinline__ int wave_sum(int s) {
  const int lane = threadIdx.x & 63;
  for (int m = 32; m >= 1; m >>= 1) s += __builtin_amdgcn_ds_bpermute(((lane ^ m) << 2), s);
  return s;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = threadIdx.x & 63;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute(((lane - d) & 63) << 2, x);
    if (lane >= d) x += y;
  }
  return x;
}

// One kernel for the whole accept step. Workgroup (c, r) scans chunk c of
// logits row r with every load of a thread issued before any is consumed,
// reduces to a (value, index) pair and publishes it with a write-through
// store; the last workgroup of a sequence (a per-sequence counter) merges its
// rows' pairs in chunk order and applies the accept rule.
template <bool VEC4>
__global__ __launch_bounds__(kArgThreads) void accept_fused_kernel(
    // leading scalars: what the first loads need, preloaded into SGPRs at
    // wave launch instead of read from the argument buffer
    const float* __restrict__ logits, const int32_t* __restrict__ n_draft, int V, int chunk_len, int B,
    AcceptParams p) {
  const int c = blockIdx.x;
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float sv[kArgThreads / 64];
  __shared__ int si[kArgThreads / 64];
  __shared__ int s_seq[4];   // b, first row, first draft, n_draft
  __shared__ int s_last;

  const int begin = c * chunk_len;
  const int end = min(V, begin + chunk_len);
  const float* row = logits + (size_t)r * V;
  float bv = -__builtin_inff();
  int bi = INT_MAX;
  float4 x[kArgUnroll];
  if (VEC4) {
#pragma unroll
    for (int u = 0; u < kArgUnroll; ++u) {
      const int e = begin + (u * kArgThreads + threadIdx.x) * 4;
      x[u] = e < end ? *reinterpret_cast<const float4*>(row + e) : float4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // wave 0 finds the sequence that owns row r while the loads are in flight
  if (wave == 0) {
    int rb = 0, db = 0, found_b = -1, fr0 = 0, fd0 = 0, fn = 0;
    for (int i0 = 0; i0 < B && found_b < 0; i0 += 64) {
      const int i = i0 + lane;
      const int n = i < B ? n_draft[i] : 0;
      const int inc_r = wave_scan(i < B ? n + 1 : 0);
      const int inc_d = wave_scan(i < B ? n : 0);
      const int my_r0 = rb + inc_r - (n + 1), my_d0 = db + inc_d - n;
      const bool mine = i < B && r >= my_r0 && r < my_r0 + n + 1;
      const unsigned long long ballot = __ballot(mine);
      if (ballot) {
        const int src = __ffsll((long long)ballot) - 1;
        found_b = __shfl(i, src);
        fr0 = __shfl(my_r0, src);
        fd0 = __shfl(my_d0, src);
        fn = __shfl(n, src);
      }
      rb += __shfl(inc_r, 63);
      db += __shfl(inc_d, 63);
    }
    if (lane == 0) {
      s_seq[0] = found_b;
      s_seq[1] = fr0;
      s_seq[2] = fd0;
      s_seq[3] = fn;
    }
  }
  if (VEC4) {
    // each thread visits its elements in increasing index order
#pragma unroll
    for (int u = 0; u < kArgUnroll; ++u) {
      const int e = begin + (u * kArgThreads + threadIdx.x) * 4;
      if (e < end) {
        scan_one(x[u].x, e + 0, bv, bi);
        scan_one(x[u].y, e + 1, bv, bi);
        scan_one(x[u].z, e + 2, bv, bi);
        scan_one(x[u].w, e + 3, bv, bi);
      }
    }
  } else {
    for (int e = begin + threadIdx.x; e < end; e += kArgThreads) scan_one(row[e], e, bv, bi);
  }
  wave_best(bv, bi);
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  const int b = s_seq[0], r0 = s_seq[1], d0 = s_seq[2], n = s_seq[3];
  // a row no sequence owns, or a sequence breaking its contract: nothing to do
  const bool ok = b >= 0 && n >= 0 && n <= p.max_draft && r0 + n + 1 <= p.total_rows &&
                  d0 + n <= p.total_rows - B;
  const auto val_rsrc = __builtin_amdgcn_make_buffer_rsrc(p.chunk_val, 0, (u32)(p.total_rows * p.chunks * 4),
                                                          0x00020000);
  const auto idx_rsrc = __builtin_amdgcn_make_buffer_rsrc(p.chunk_idx, 0, (u32)(p.total_rows * p.chunks * 4),
                                                          0x00020000);
  if (wave == 0) {
    float v = lane < kArgThreads / 64 ? sv[lane] : -__builtin_inff();
    int i = lane < kArgThreads / 64 ? si[lane] : INT_MAX;
    wave_best(v, i);
    if (lane == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), val_rsrc, (r * p.chunks + c) * 4, 0, kSc1);
      __builtin_amdgcn_raw_buffer_store_b32((u32)i, idx_rsrc, (r * p.chunks + c) * 4, 0, kSc1);
      __builtin_amdgcn_s_waitcnt(0);  // the pair is device-visible before the count
      int last = 0;
      if (ok) {
        const u32 prev = __hip_atomic_fetch_add(p.counters + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = prev == (u32)((n + 1) * p.chunks - 1);
      } else if (b >= 0 && c == 0 && r == r0) {
        p.out_accept[b] = 0;
        p.out_next[b] = -1;
      }
      s_last = last;
    }
  }
  __syncthreads();
  if (!s_last || wave != 0) return;

  // ---- last workgroup of sequence b: per-row argmax over chunks, then accept.
  // Everything it reads is requested up front, in one batch.
  const int w_old = p.window ? p.window[b] : 0;
  int draft[PKV_MAX_Q_LEN - 1];
#pragma unroll
  for (int i = 0; i < PKV_MAX_Q_LEN - 1; ++i) draft[i] = -1;
  if (n > 0) {
    // clamped, unconditional loads: all in flight together
#pragma unroll
    for (int i = 0; i < PKV_MAX_Q_LEN - 1; ++i) draft[i] = p.draft_ids[d0 + min(i, n - 1)];
  }
  // lane c holds chunk c of every row of the sequence (64 chunks per pass)
  float rv[PKV_MAX_Q_LEN];
  int ri[PKV_MAX_Q_LEN];
#pragma unroll
  for (int i = 0; i < PKV_MAX_Q_LEN; ++i) {
    rv[i] = -__builtin_inff();
    ri[i] = INT_MAX;
  }
  for (int c0 = 0; c0 < p.chunks; c0 += 64) {
    const int cc = c0 + lane;
    float cv[PKV_MAX_Q_LEN];
    int ci[PKV_MAX_Q_LEN];
#pragma unroll
    for (int i = 0; i < PKV_MAX_Q_LEN; ++i) {
      // rows past the sequence and chunks past the row read out of range: zeros, skipped below
      const int off = (i <= n && cc < p.chunks ? (r0 + i) * p.chunks + cc : p.total_rows * p.chunks) * 4;
      cv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(val_rsrc, off, 0, kSc1));
      ci[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(idx_rsrc, off, 0, kSc1);
    }
#pragma unroll
    for (int i = 0; i < PKV_MAX_Q_LEN; ++i) {
      const bool take = (i <= n) & (cc < p.chunks) & better(cv[i], ci[i], rv[i], ri[i]);
      rv[i] = take ? cv[i] : rv[i];
      ri[i] = take ? ci[i] : ri[i];
    }
  }
  int m = n, next = 0;
  bool found = false;
#pragma unroll
  for (int i = 0; i < PKV_MAX_Q_LEN; ++i) {
    if (i <= n) {
      wave_best(rv[i], ri[i]);
      // drafts compared from the left; the first mismatch keeps the base token
      if (!found && (i == n || ri[i] != draft[i < PKV_MAX_Q_LEN - 1 ? i : 0])) {
        m = i;
        next = ri[i];
        found = true;
      }
    }
  }
  if (lane == 0) {
    p.out_accept[b] = m + 1;
    p.out_next[b] = next;
    if (p.window) p.window[b] = (m == n) ? w_old + 2 : max(1, w_old - 1);
    __hip_atomic_store(p.counters + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

AcceptWorkspace accept_workspace(int B, int total_rows, int V) {
  AcceptWorkspace ws;
  // each workgroup scans what one round of its threads' loads covers
  const int len = kArgThreads * kArgUnroll * 4;
  const int chunks = (V + len - 1) / len;
  ws.chunks = chunks;
  ws.chunk_len = len;
  const size_t n = (size_t)total_rows * chunks;
  ws.counters_off = 0;
  ws.val_off = ((size_t)B * 4 + 255) / 256 * 256;
  ws.idx_off = ws.val_off + (n * 4 + 255) / 256 * 256;
  ws.total = ws.idx_off + (n * 4 + 255) / 256 * 256;
  if (ws.total == 0) ws.total = 256;
  return ws;
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t stream) {
  if (p.B == 0 || p.total_rows == 0) return hipSuccess;
  dim3 grid(p.chunks, p.total_rows);
  if (p.V % 4 == 0 && p.chunk_len <= kArgThreads * kArgUnroll * 4)
    hipLaunchKernelGGL(accept_fused_kernel<true>, grid, dim3(kArgThreads), 0, stream, p.logits, p.n_draft, p.V,
                       p.chunk_len, p.B, p);
  else
    hipLaunchKernelGGL(accept_fused_kernel<false>, grid, dim3(kArgThreads), 0, stream, p.logits, p.n_draft, p.V,
                       p.chunk_len, p.B, p);
  return hipGetLastError();
}

}  // namespace pkv
