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
// Two kernels. argmax_kernel scans row chunks (an HBM-bound fp32 stream; one
// row alone is far too small to fill the chip) and folds each chunk's
// (value, index) into its row's 64-bit key with one atomic max, issued and
// never waited on. accept_rule_kernel, one workgroup launched behind it on
// the same stream, reads the row keys, applies the accept rule and the
// window update, and clears the keys for the next call. The kernel boundary
// is the only synchronisation between the two.
//
// argmax order: larger value first; NaN above every number; lower index on
// equal values (and between NaNs); -0 equals +0. The key encodes exactly this
// order, so the result is exact and unique.

#include "internal.h"

#include <climits>

#include "pkv.h"

namespace pkv {
namespace {

using u32 = uint32_t;
using u64 = unsigned long long;

#ifndef PKV_ARG_THREADS
#define PKV_ARG_THREADS 512
#endif
constexpr int kArgThreads = PKV_ARG_THREADS;  // threads per argmax workgroup
constexpr int kArgUnroll = 8;                 // float4 loads in flight per thread, at most
#ifndef PKV_ARG_TARGET_WGS
#define PKV_ARG_TARGET_WGS 768
#endif
constexpr int kArgTargetWgs = PKV_ARG_TARGET_WGS;  // about three workgroups per CU
constexpr int kRuleThreads = 1024;

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

// Order-preserving 64-bit key of (value, index): unsigned comparison of keys
// is `better` on pairs. High word: the float's bits mapped to an unsigned
// order (negatives flipped, positives offset), every NaN above +inf, -0 as
// +0. Low word: the index inverted, so the lower index is the larger key.
// Key 0 is below every pair (an untouched row).
__device__ __forceinline__ u64 argmax_key(float v, int i) {
  u32 hi;
  if (v != v) {
    hi = 0xFFFFFFFFu;
  } else {
    const u32 bits = __float_as_uint(v == 0.f ? 0.f : v);
    hi = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  }
  return ((u64)hi << 32) | (u64)(0xFFFFFFFFu - (u32)i);
}

__device__ __forceinline__ int key_index(u64 k) { return (int)(0xFFFFFFFFu - (u32)(k & 0xFFFFFFFFull)); }

// Workgroup (c, r): chunk c of logits row r. Every load of a thread is issued
// before any is consumed; the chunk's best pair goes into the row key.
template <bool VEC4>
__global__ __launch_bounds__(kArgThreads) void argmax_kernel(
    // leading scalars, preloaded into SGPRs at wave launch
    const float* __restrict__ logits, int V, int chunk_len, u64* __restrict__ keys) {
  const int c = blockIdx.x;
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float sv[kArgThreads / 64];
  __shared__ int si[kArgThreads / 64];

  const int begin = c * chunk_len;
  const int end = min(V, begin + chunk_len);
  const float* row = logits + (size_t)r * V;
  float bv = -__builtin_inff();
  int bi = INT_MAX;
  if (VEC4) {
    float4 x[kArgUnroll];
#pragma unroll
    for (int u = 0; u < kArgUnroll; ++u) {
      const int e = begin + (u * kArgThreads + threadIdx.x) * 4;
      x[u] = e < end ? *reinterpret_cast<const float4*>(row + e) : float4{0.f, 0.f, 0.f, 0.f};
    }
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
  if (wave != 0) return;
  float v = lane < kArgThreads / 64 ? sv[lane] : -__builtin_inff();
  int i = lane < kArgThreads / 64 ? si[lane] : INT_MAX;
  wave_best(v, i);
  if (lane == 0 && i != INT_MAX)
    __hip_atomic_fetch_max(keys + r, argmax_key(v, i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// One workgroup: thread b (in tiles of kRuleThreads sequences) finds its
// sequence's first logits row by a block-wide prefix sum of n_draft + 1,
// reads its rows' keys and drafts (all requested together), applies the
// accept rule and the window update. Then every row key is cleared.
__global__ __launch_bounds__(kRuleThreads) void accept_rule_kernel(AcceptParams p) {
  constexpr int kWaves = kRuleThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int s_wsum[kWaves];
  __shared__ int s_carry;
  __shared__ u64 s_keys[kRuleThreads];
  __shared__ int s_draft[kRuleThreads];
  // Up to kRuleThreads rows, every key and draft is fetched up front, in the
  // same memory round trip as n_draft, and read from LDS below.
  const bool staged = p.total_rows <= kRuleThreads;
  if (staged) {
    if ((int)threadIdx.x < p.total_rows) s_keys[threadIdx.x] = p.keys[threadIdx.x];
    if ((int)threadIdx.x < p.total_rows - p.B) s_draft[threadIdx.x] = p.draft_ids[threadIdx.x];
  }
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int t0 = 0; t0 < p.B; t0 += kRuleThreads) {
    const int b = t0 + threadIdx.x;
    const int n = b < p.B ? p.n_draft[b] : 0;
    const int w_old = (b < p.B && p.window) ? p.window[b] : 0;
    const int inc = wave_scan(b < p.B ? n + 1 : 0);
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    const int r0 = before + inc - (n + 1);  // first row of sequence b
    const int d0 = r0 - b;                  // first draft: the sum of n_draft before b
    if (b < p.B) {
      const bool ok = n >= 0 && n <= p.max_draft && r0 >= 0 && r0 + n + 1 <= p.total_rows && d0 >= 0 &&
                      d0 + n <= p.total_rows - p.B;
      if (!ok) {
        p.out_accept[b] = 0;
        p.out_next[b] = -1;
      } else {
        // clamped, unconditional loads: all in flight together
        u64 key[PKV_MAX_Q_LEN];
        int draft[PKV_MAX_Q_LEN - 1];
#pragma unroll
        for (int i = 0; i < PKV_MAX_Q_LEN; ++i) key[i] = staged ? s_keys[r0 + min(i, n)] : p.keys[r0 + min(i, n)];
#pragma unroll
        for (int i = 0; i < PKV_MAX_Q_LEN - 1; ++i)
          draft[i] = n <= 0 ? -1 : staged ? s_draft[d0 + min(i, n - 1)] : p.draft_ids[d0 + min(i, n - 1)];
        // drafts compared from the left; the first mismatch keeps the base token
        int m = n;
#pragma unroll
        for (int i = PKV_MAX_Q_LEN - 2; i >= 0; --i)
          if (i < n && key_index(key[i]) != draft[i]) m = i;
        int next = 0;
#pragma unroll
        for (int i = 0; i < PKV_MAX_Q_LEN; ++i)
          if (i == m) next = key_index(key[i]);
        p.out_accept[b] = m + 1;
        p.out_next[b] = next;
        if (p.window) p.window[b] = (m == n) ? w_old + 2 : max(1, w_old - 1);
      }
    }
    __syncthreads();
    if (threadIdx.x == kRuleThreads - 1) s_carry = before + inc;
    __syncthreads();
  }
  // every key has been read (its value was used before the barrier): clear
  // all rows, owned or not, for the next call
  for (int r = threadIdx.x; r < p.total_rows; r += kRuleThreads) p.keys[r] = 0ull;
}

}  // namespace

AcceptWorkspace accept_workspace(int B, int total_rows, int V) {
  (void)B;
  AcceptWorkspace ws;
  // about three workgroups per CU; a chunk is at most one round of every
  // thread's loads and at least one float4 per thread
  const long rows = total_rows > 0 ? total_rows : 1;
  long chunks = (kArgTargetWgs + rows - 1) / rows;
  const long most = ((long)V + (long)kArgThreads * 4 - 1) / ((long)kArgThreads * 4);
  const long least = ((long)V + (long)kArgThreads * kArgUnroll * 4 - 1) / ((long)kArgThreads * kArgUnroll * 4);
  if (chunks > most) chunks = most;
  if (chunks < least) chunks = least;
  if (chunks < 1) chunks = 1;
  long len = (V + chunks - 1) / chunks;
  len = (len + 3) / 4 * 4;
  ws.chunk_len = (int)len;
  ws.chunks = (int)((V + len - 1) / len);
  ws.keys_off = 0;
  ws.total = ((size_t)total_rows * 8 + 255) / 256 * 256;
  if (ws.total == 0) ws.total = 256;
  return ws;
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t stream) {
  if (p.B == 0 || p.total_rows == 0) return hipSuccess;
  dim3 grid(p.chunks, p.total_rows);
  const bool vec4 = p.V % 4 == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0 &&
                    p.chunk_len <= kArgThreads * kArgUnroll * 4;
  if (vec4)
    hipLaunchKernelGGL(argmax_kernel<true>, grid, dim3(kArgThreads), 0, stream, p.logits, p.V, p.chunk_len, p.keys);
  else
    hipLaunchKernelGGL(argmax_kernel<false>, grid, dim3(kArgThreads), 0, stream, p.logits, p.V, p.chunk_len,
                       p.keys);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_rule_kernel, dim3(1), dim3(kRuleThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
