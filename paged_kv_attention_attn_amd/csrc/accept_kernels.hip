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
// One kernel. Its workgroups scan row chunks (an HBM-bound fp32 stream; one
// row alone is far too small to fill the chip) and store each chunk's best
// (value, index) as a 64-bit key, which is never zero, into the chunk's slot.
// The last workgroup of the grid (so started after every other one) polls
// the slots until every key has arrived, takes the largest chunk key of every
// row, applies the accept rule and the window update, and clears the slots
// for the next call; on large grids it is a workgroup of its own, which
// scans nothing. No workgroup waits for its own store
// and nothing is counted, so the chain after the stream is one memory round
// trip: the last key's store, seen by the next poll.
//
// Ordering. The slots are only touched by agent-scope atomics (stores,
// loads, exchanges, and maxima with 0 to read a key that is read twice), and
// the hardware performs the atomics on one address at one place for every
// XCD, one after another; a key is read only once it has been seen, so every
// key read comes after its write, and the slots are zero again before the
// call ends. Only these slots carry data between workgroups, so none of the
// language model's L2-wide write-back and invalidate is needed.
//
// argmax order: larger value first; NaN above every number; lower index on
// equal values (and between NaNs); -0 equals +0. The key encodes exactly this
// order, so the result is exact and unique.

#include "internal.h"

#include <climits>
#include <mutex>

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
constexpr long kChipCus = 256;                     // MI355X compute units

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

// Workgroup barrier for LDS traffic only. __syncthreads also waits for the
// wave's global stores to be acknowledged, a memory round trip that nothing
// here needs: every global access of these kernels that another wave reads
// is an atomic.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = threadIdx.x & 63;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute(((lane - d) & 63) << 2, x);
    if (lane >= d) x += y;
  }
  return x;
}

// Key of a chunk with no element: below every pair, and not zero, which
// marks a slot whose key has not arrived.
constexpr u64 kEmptyKey = 1;
// How long the last workgroup polls for a key before it gives up: 2^30 ticks
// of the constant-rate wall clock (about 11 s at its 100 MHz), far beyond any
// call, also while other streams' kernels hold CUs that the call's other
// workgroups still wait for.
constexpr long long kPollTicks = 1ll << 30;
constexpr int kPollBatch = 4;  // slots polled at once per thread

// Run by the last workgroup: polls every chunk key of the call until it has
// arrived (slots are zero between calls and keys never are), calling
// take(e, key) once per slot e as it is first seen, each thread for its own
// slots, several at a time. Returns false if some key did not arrive within
// kPollTicks.
template <class Take>
__device__ __forceinline__ bool take_keys(const AcceptParams& p, Take take) {
  const int ns = p.total_rows * p.chunks;
  const long long t0 = wall_clock64();
  bool ok = true;
  for (int e0 = 0; e0 < ns; e0 += kPollBatch * kArgThreads) {
    u32 pending = 0;
#pragma unroll
    for (int u = 0; u < kPollBatch; ++u)
      if (e0 + u * kArgThreads + (int)threadIdx.x < ns) pending |= 1u << u;
    while (pending != 0 && wall_clock64() - t0 < kPollTicks) {
      u64 x[kPollBatch];
#pragma unroll
      for (int u = 0; u < kPollBatch; ++u)
        x[u] = (pending >> u) & 1u ? __hip_atomic_load(p.slots + e0 + u * kArgThreads + threadIdx.x,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0ull;
#pragma unroll
      for (int u = 0; u < kPollBatch; ++u)
        if (((pending >> u) & 1u) && x[u] != 0ull) {
          pending &= ~(1u << u);
          take(e0 + u * kArgThreads + (int)threadIdx.x, x[u]);
        }
      if (pending != 0) __builtin_amdgcn_s_sleep(1);
    }
    ok = ok && pending == 0;
  }
  return ok;
}

// Chunk key of (row, chunk), read by the last workgroup.
__device__ __forceinline__ u64 read_slot(const AcceptParams& p, int r, int c) {
  // a max with 0 leaves the key as it is
  return __hip_atomic_fetch_max(p.slots + (size_t)r * p.chunks + c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The row's key: the largest of its chunk keys.
__device__ __forceinline__ u64 row_key(const AcceptParams& p, int r) {
  u64 k = 0;
  for (int c = 0; c < p.chunks; ++c) {
    u64 x = read_slot(p, r, c);
    x = x == kEmptyKey ? 0ull : x;
    k = x > k ? x : k;
  }
  return k;
}

// Sequence b's accept decision from its rows' keys and its drafts (both
// indexed from the sequence's first row r0 / first draft d0 through `key_at`
// and `draft_at`), written to the outputs; out_accept = 0, out_next = -1 for
// a sequence whose rows or drafts break the contract.
template <class KeyAt, class DraftAt>
__device__ __forceinline__ void decide(const AcceptParams& p, int b, int n, int w_old, int r0, int d0, KeyAt key_at,
                                       DraftAt draft_at) {
  const bool ok = n >= 0 && n <= p.max_draft && r0 >= 0 && r0 + n + 1 <= p.total_rows && d0 >= 0 &&
                  d0 + n <= p.total_rows - p.B;
  if (!ok) {
    p.out_accept[b] = 0;
    p.out_next[b] = -1;
    return;
  }
  // clamped, unconditional reads: all in flight together
  u64 key[PKV_MAX_Q_LEN];
  int draft[PKV_MAX_Q_LEN - 1];
#pragma unroll
  for (int i = 0; i < PKV_MAX_Q_LEN; ++i) key[i] = key_at(r0 + min(i, n));
#pragma unroll
  for (int i = 0; i < PKV_MAX_Q_LEN - 1; ++i) draft[i] = n <= 0 ? -1 : draft_at(d0 + min(i, n - 1));
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

// The accept rule, run by the workgroup that finished last, for up to
// kArgThreads logits rows (so at most as many sequences): thread b takes
// sequence b. Every input and every chunk key is requested at once; the
// chunk keys are taken and cleared by atomic exchanges and reduced per row
// in LDS; a block-wide prefix sum of n_draft + 1 gives each sequence its
// first row.
__device__ void accept_rule_small(const AcceptParams& p) {
  constexpr int kWaves = kArgThreads / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ int s_wsum[kWaves];
  __shared__ u64 s_keys[kArgThreads];
  __shared__ int s_draft[kArgThreads];
  __shared__ int s_ok;
  const int n = t < p.B ? p.n_draft[t] : 0;
  const int w_old = (t < p.B && p.window) ? p.window[t] : 0;
  const int d = t < p.total_rows - p.B ? p.draft_ids[t] : 0;
  s_keys[t] = 0;
  if (t == 0) s_ok = 1;
  lds_barrier();
  // each key is taken into its row's maximum as soon as it is seen, and its
  // slot cleared for the next call
  const bool ok = take_keys(p, [&](int e, u64 x) {
    atomicMax(&s_keys[e / p.chunks], x == kEmptyKey ? 0ull : x);
    __hip_atomic_store(p.slots + e, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
  if (!ok) s_ok = 0;
  s_draft[t] = d;
  const int inc = wave_scan(t < p.B ? n + 1 : 0);
  if (lane == 63) s_wsum[wave] = inc;
  lds_barrier();
  if (t >= p.B) return;
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wsum[w];
  const int r0 = before + inc - (n + 1);  // first row of sequence t
  if (!s_ok) {  // a chunk key that never came: the contract-break outputs
    p.out_accept[t] = 0;
    p.out_next[t] = -1;
    return;
  }
  decide(p, t, n, w_old, r0, r0 - t, [&](int r) { return s_keys[r]; }, [&](int i) { return s_draft[i]; });
}

// The same rule for any number of rows: thread b of each tile of
// kArgThreads sequences; row keys are read from their chunk keys (atomic
// maxima with 0, which leave them as they are) and cleared at the end.
__device__ void accept_rule_tiled(const AcceptParams& p) {
  constexpr int kWaves = kArgThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int s_wsum[kWaves];
  __shared__ int s_carry;
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    s_carry = 0;
    s_ok = 1;
  }
  lds_barrier();
  if (!take_keys(p, [](int, u64) {})) s_ok = 0;
  lds_barrier();
  for (int t0 = 0; t0 < p.B; t0 += kArgThreads) {
    const int b = t0 + threadIdx.x;
    const int n = b < p.B ? p.n_draft[b] : 0;
    const int w_old = (b < p.B && p.window) ? p.window[b] : 0;
    const int inc = wave_scan(b < p.B ? n + 1 : 0);
    if (lane == 63) s_wsum[wave] = inc;
    lds_barrier();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    const int r0 = before + inc - (n + 1);  // first row of sequence b
    if (b < p.B && !s_ok) {
      p.out_accept[b] = 0;
      p.out_next[b] = -1;
    } else if (b < p.B) {
      decide(p, b, n, w_old, r0, r0 - b, [&](int r) { return row_key(p, r); },
             [&](int i) { return p.draft_ids[i]; });
    }
    lds_barrier();
    if (threadIdx.x == kArgThreads - 1) s_carry = before + inc;
    lds_barrier();
  }
  // every chunk key has been read (before the last barrier): clear them
  for (int e = threadIdx.x; e < p.total_rows * p.chunks; e += kArgThreads)
    __hip_atomic_exchange(p.slots + e, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The rule, in one workgroup: it waits for every chunk key first.
__device__ __forceinline__ void accept_rule(const AcceptParams& p) {
  if (p.total_rows <= kArgThreads)
    accept_rule_small(p);
  else
    accept_rule_tiled(p);
}

// Workgroup (c, r), r < rows: chunk c of logits row r. Every load of a
// thread is issued before any is consumed; the chunk's best pair is stored as
// its chunk key. The rule runs in a workgroup that the dispatcher starts after
// every chunk workgroup. With own_rule the grid has one row more, whose first
// workgroup scans nothing and polls from its start (the others end at once):
// on grids larger than one round of the chip the chunk workgroups start over
// microseconds, and the last of them starts last. Otherwise the last chunk
// workgroup scans its chunk and then applies the rule.
template <bool VEC4>
__global__ __launch_bounds__(kArgThreads) void accept_kernel(
    // leading scalars, preloaded into SGPRs at wave launch
    const float* __restrict__ logits, int V, int chunk_len, int own_rule, AcceptParams p) {
  const int c = blockIdx.x;
  const int r = blockIdx.y;
  if (own_rule && r == (int)gridDim.y - 1) {
    if (c == 0) accept_rule(p);
    return;
  }
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
  lds_barrier();
  if (wave == 0) {
    float v = lane < kArgThreads / 64 ? sv[lane] : -__builtin_inff();
    int i = lane < kArgThreads / 64 ? si[lane] : INT_MAX;
    wave_best(v, i);
    // the chunk's key, nonzero; nothing waits for it here
    if (lane == 0)
      __hip_atomic_store(p.slots + (size_t)r * gridDim.x + c, i != INT_MAX ? argmax_key(v, i) : kEmptyKey,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!own_rule && c == (int)gridDim.x - 1 && r == (int)gridDim.y - 1) accept_rule(p);
}

// Fills n 32-bit words with zero (a kernel, not a memset, so that a caller
// capturing the stream into a graph records nothing but kernels).
__global__ __launch_bounds__(256) void zero_words(u32* __restrict__ w, u32 n) {
  for (u32 i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) w[i] = 0u;
}

}  // namespace

// Workspace of the allocation-free accept entry point: one copy per GPU in
// the code object's device memory, alive until the process ends. Host code
// never passes this name to a kernel (on the host it is only a stand-in);
// it uses the device address that accept_scratch looks up for the current
// device.
static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];
}  // namespace

hipError_t accept_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the accept protocol needs the workspace zero before a call (and
    // leaves it zero); clear this device's copy once, on the caller's stream
    hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, static_cast<u32*>(ptr),
                       (u32)(kAcceptScratchBytes / 4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

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
  // the chunk keys, zero between calls
  ws.slots_off = 0;
  ws.total = ((size_t)total_rows * ws.chunks * 8 + 255) / 256 * 256;
  return ws;
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t stream) {
  if (p.B == 0 || p.total_rows == 0) return hipSuccess;
  // one workgroup per (row, chunk); past one round of the chip, a row more
  // for the rule
  const int own_rule = (long)p.chunks * p.total_rows > kChipCus && p.total_rows < 65535 ? 1 : 0;
  const dim3 grid(p.chunks, p.total_rows + own_rule);
  const bool vec4 = p.V % 4 == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0 &&
                    p.chunk_len <= kArgThreads * kArgUnroll * 4;
  if (vec4)
    hipLaunchKernelGGL(accept_kernel<true>, grid, dim3(kArgThreads), 0, stream, p.logits, p.V, p.chunk_len,
                       own_rule, p);
  else
    hipLaunchKernelGGL(accept_kernel<false>, grid, dim3(kArgThreads), 0, stream, p.logits, p.V, p.chunk_len,
                       own_rule, p);
  return hipGetLastError();
}

}  // namespace pkv
