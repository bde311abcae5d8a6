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

namespace pkv {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  const bool na = a != a, nb = b != b;
  if (na || nb) return na && (!nb || ia < ib);
  if (a != b) return a > b;
  return ia < ib;
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

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void argmax_chunk_kernel(AcceptParams p) {
  const int c = blockIdx.x;
  const int r = blockIdx.y;
  const int begin = c * p.chunk_len;
  const int end = min(p.V, begin + p.chunk_len);
  const float* row = p.logits + (size_t)r * p.V;
  float bv = -__builtin_inff();
  int bi = INT_MAX;
  if (VEC4) {
    // begin and V are multiples of 4 here: aligned float4 loads, in index order per thread
    for (int e = begin + threadIdx.x * 4; e < end; e += kThreads * 4) {
      const float4 x = *reinterpret_cast<const float4*>(row + e);
      if (better(x.x, e + 0, bv, bi)) { bv = x.x; bi = e + 0; }
      if (better(x.y, e + 1, bv, bi)) { bv = x.y; bi = e + 1; }
      if (better(x.z, e + 2, bv, bi)) { bv = x.z; bi = e + 2; }
      if (better(x.w, e + 3, bv, bi)) { bv = x.w; bi = e + 3; }
    }
  } else {
    for (int e = begin + threadIdx.x; e < end; e += kThreads) {
      const float x = row[e];
      if (better(x, e, bv, bi)) { bv = x; bi = e; }
    }
  }
  wave_best(bv, bi);
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    p.chunk_val[(size_t)r * p.chunks + c] = bv;
    p.chunk_idx[(size_t)r * p.chunks + c] = bi;
  }
}

__device__ __forceinline__ int wave_sum(int s) {
  const int lane = threadIdx.x & 63;
  for (int m = 32; m >= 1; m >>= 1) s += __builtin_amdgcn_ds_bpermute(((lane ^ m) << 2), s);
  return s;
}

__global__ __launch_bounds__(kThreads) void accept_kernel(AcceptParams p) {
  const int b = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (b >= p.B) return;
  const int lane = threadIdx.x & 63;
  int rs = 0, ds = 0;
  for (int i = lane; i < b; i += 64) {
    const int n = p.n_draft[i];
    rs += n + 1;
    ds += n;
  }
  const int r0 = wave_sum(rs), d0 = wave_sum(ds);
  const int n = p.n_draft[b];
  // rows and drafts of this sequence must lie inside logits [total_rows] and
  // draft_ids [total_rows - B]
  if (n < 0 || n > p.max_draft || r0 + n + 1 > p.total_rows || d0 + n > p.total_rows - p.B) {
    if (lane == 0) {
      p.out_accept[b] = 0;
      p.out_next[b] = -1;
    }
    return;
  }
  int m = n, next = 0;
  for (int i = 0; i <= n; ++i) {
    float v = -__builtin_inff();
    int ix = INT_MAX;
    for (int c = lane; c < p.chunks; c += 64) {
      const float cv = p.chunk_val[(size_t)(r0 + i) * p.chunks + c];
      const int ci = p.chunk_idx[(size_t)(r0 + i) * p.chunks + c];
      if (better(cv, ci, v, ix)) { v = cv; ix = ci; }
    }
    wave_best(v, ix);
    if (i == n || ix != p.draft_ids[d0 + i]) {
      m = i;
      next = ix;
      break;
    }
  }
  if (lane == 0) {
    p.out_accept[b] = m + 1;
    p.out_next[b] = next;
    if (p.window) {
      const int w = p.window[b];
      p.window[b] = (m == n) ? w + 2 : max(1, w - 1);
    }
  }
}

}  // namespace

AcceptWorkspace accept_workspace(int total_rows, int V) {
  AcceptWorkspace ws;
  int chunks = total_rows > 0 ? (2048 + total_rows - 1) / total_rows : 1;
  chunks = chunks < 1 ? 1 : (chunks > 64 ? 64 : chunks);
  int len = (V + chunks - 1) / chunks;
  len = (len + 3) / 4 * 4;
  if (len < 4) len = 4;
  chunks = (V + len - 1) / len;
  ws.chunks = chunks;
  ws.chunk_len = len;
  ws.val_off = 0;
  const size_t n = (size_t)total_rows * chunks;
  ws.idx_off = (n * 4 + 255) / 256 * 256;
  ws.total = ws.idx_off + (n * 4 + 255) / 256 * 256;
  if (ws.total == 0) ws.total = 256;
  return ws;
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  if (p.total_rows > 0) {
    dim3 grid(p.chunks, p.total_rows);
    if (p.V % 4 == 0)
      hipLaunchKernelGGL(argmax_chunk_kernel<true>, grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(argmax_chunk_kernel<false>, grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int blocks = (p.B + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(accept_kernel, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
