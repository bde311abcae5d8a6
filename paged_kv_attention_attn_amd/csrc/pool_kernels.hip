// Page moves of the paged cache for gfx950: copying whole pages between slots
// of the K and V pools (the data movement of a defragmentation) and rewriting
// block tables through a page remap.
//
// Source: ExLlamaV2 "Dynamic Generator" page, "Continuous Batching": the cache
// can be defragmented (the generator does it for unreferenced pages when its
// queue is empty); a batch changes by rewriting block indices only.
//
// A page of one pool is Hkv * 256 * D bf16 values, contiguous. The copy grid
// is (block, pool, move), flattened: every workgroup moves one 64 KiB block of
// one page of one pool, each thread issuing all its 16-byte loads before any store, so
// a move is 2 * page_bytes / 64 KiB independent workgroups (plain loads: a
// non-temporal hint halved the rate). The HBM roofline is
// 2 bytes of traffic (one read, one write) per byte moved.

#include "internal.h"

#include "pkv.h"

namespace pkv {
namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kPerThread = 16;                               // 16-byte pieces per thread
constexpr long kBlockBytes = kCopyThreads * kPerThread * 16;  // 64 KiB

__global__ __launch_bounds__(kCopyThreads) void copy_pages_kernel(PageMoveParams p, int blocks) {
  // workgroup -> (block of the page, pool, move), block fastest
  const int blk = blockIdx.x % blocks;
  const int pool = (blockIdx.x / blocks) & 1;
  const int move = blockIdx.x / (2 * blocks);
  const int s = p.src[move], d = p.dst[move];
  if (s < 0 || s >= p.P || d < 0 || d >= p.P) {
    if (blk == 0 && pool == 0 && threadIdx.x == 0 && p.err) atomicOr(p.err, PKV_EFLAG_PAGE);
    return;
  }
  char* base = reinterpret_cast<char*>(pool ? p.v_pool : p.k_pool);
  const long off = (long)blk * kBlockBytes;
  const u32x4* from = reinterpret_cast<const u32x4*>(base + (long)s * p.page_bytes + off);
  u32x4* to = reinterpret_cast<u32x4*>(base + (long)d * p.page_bytes + off);
  const long n16 = (p.page_bytes - off) / 16;  // the last block of a page may be short
  u32x4 v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const long e = (long)i * kCopyThreads + threadIdx.x;
    if (e < n16) v[i] = from[e];
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const long e = (long)i * kCopyThreads + threadIdx.x;
    if (e < n16) to[e] = v[i];
  }
}

__global__ __launch_bounds__(256) void table_remap_kernel(int32_t* table, int32_t n, const int32_t* remap,
                                                          int32_t P, uint32_t* err) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int t = table[i];
  if (t < 0) return;
  if (t >= P) {
    if (err) atomicOr(err, PKV_EFLAG_PAGE);
    return;
  }
  table[i] = remap[t];
}

}  // namespace

hipError_t launch_copy_pages(const PageMoveParams& p, hipStream_t stream) {
  const int blocks = (int)((p.page_bytes + kBlockBytes - 1) / kBlockBytes);
  hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)(2L * blocks * p.n_moves)), dim3(kCopyThreads), 0, stream,
                     p, blocks);
  return hipGetLastError();
}

hipError_t launch_table_remap(int32_t* table, int32_t n, const int32_t* remap, int32_t P, uint32_t* err,
                              hipStream_t stream) {
  hipLaunchKernelGGL(table_remap_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, table, n, remap,
                     P, err);
  return hipGetLastError();
}

}  // namespace pkv
