// Writing a verify window's K/V into the paged cache, and releasing the
// rejected part after the accept step, for gfx950.
//
// Sources (cited by page title and section):
//  - ExLlamaV2 "Dynamic Generator" page, "Continuous Batching": sequences grow
//    into 256-token pages reached through block tables; changing a batch only
//    rewrites block indices; pages freed by a job leave holes that later jobs
//    fill, so indices need not be contiguous.
//  - Hugging Face "Assisted Generation" page, "Assisted Generation loop",
//    step 4: candidates after the first mismatch are discarded; the kept
//    tokens are the accepted count of the accept step.
//
// Free pages form a stack free_pages[0 .. *free_count). An append pops pages
// from the top, sequences in index order and each sequence's new pages in
// table order; a rollback pushes released pages on top in the same order. The
// order comes from block-wide prefix sums, so it is deterministic.
//
// Each call checks every contract before it changes anything: a violation
// sets a bit in the workspace error word and leaves all buffers unchanged.
//
// append = kv_append_plan_kernel (one workgroup: checks, page allocation,
// table and length updates, and the destination token of every window row)
// then kv_append_copy_kernel (16-byte pieces of the rows into the pools), or
// for quantized pools kv_append_quant_kernel (each row vector encoded into
// its slot's codes and scale).
// rollback = kv_rollback_kernel (one workgroup).

#include "internal.h"

#include "pkv.h"
#include "quant_encode.h"

namespace pkv {
namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kCopyThreads = 256;

__device__ __forceinline__ int pages_of(int tokens) { return (tokens + kPage - 1) / kPage; }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute(((lane - d) & 63) << 2, x);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive prefix sum of x over the workgroup (kPlanThreads threads); *total
// receives the sum. Every thread must call it.
__device__ int block_excl_scan(int x, int* total, int* s_wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(x);
  __syncthreads();
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kPlanWaves; ++w) {
    const int v = s_wsum[w];
    before += w < wave ? v : 0;
    all += v;
  }
  *total = all;
  return before + inc - x;
}

// ------------------------------------------------------------------ append

__global__ __launch_bounds__(kPlanThreads) void kv_append_plan_kernel(KvParams p) {
  __shared__ int s_wsum[kPlanWaves];
  __shared__ u32 s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int count = *p.free_count;
  // pass 1: contracts, pages and rows needed
  int need_all = 0, rows_all = 0;
  for (int t0 = 0; t0 < p.B; t0 += kPlanThreads) {
    const int b = t0 + threadIdx.x;
    int need = 0, rows = 0;
    if (b < p.B) {
      const int L = p.seq_lens[b], n = p.q_lens[b];
      u32 bad = 0;
      if (L < 0 || n < 0 || (long)L + n > (long)p.W * kPage) {
        bad |= PKV_EFLAG_QLEN;
      } else {
        need = pages_of(L + n) - pages_of(L);
        rows = n;
        // the partly filled last page receives tokens: its entry must be a page
        if (n > 0 && L % kPage != 0) {
          const int pg = p.block_table[(size_t)b * p.W + L / kPage];
          if (pg < 0 || pg >= p.P) bad |= PKV_EFLAG_PAGE;
        }
      }
      if (bad) atomicOr(&s_bad, bad);
    }
    int tn, tr;
    block_excl_scan(need, &tn, s_wsum);
    block_excl_scan(rows, &tr, s_wsum);
    need_all += tn;
    rows_all += tr;
  }
  __syncthreads();
  u32 bad = s_bad;
  if (rows_all != p.total_q) bad |= PKV_EFLAG_ROWS;
  if (count < 0 || need_all > count || count > p.P) bad |= PKV_EFLAG_SPACE;
  if (!bad) {
    // the pages about to be handed out must be pages
    for (int k = threadIdx.x; k < need_all; k += kPlanThreads) {
      const int pg = p.free_pages[count - 1 - k];
      if (pg < 0 || pg >= p.P) atomicOr(&s_bad, (u32)PKV_EFLAG_SPACE);
    }
    __syncthreads();
    bad |= s_bad;
  }
  if (bad) {
    if (threadIdx.x == 0) {
      atomicOr(p.err, bad);
      *p.go = 0;
    }
    return;
  }
  // pass 2: hand out pages, record each row's destination token, grow lengths
  int need_base = 0, row_base = 0;
  for (int t0 = 0; t0 < p.B; t0 += kPlanThreads) {
    const int b = t0 + threadIdx.x;
    int L = 0, n = 0, need = 0;
    if (b < p.B) {
      L = p.seq_lens[b];
      n = p.q_lens[b];
      need = pages_of(L + n) - pages_of(L);
    }
    int tn, tr;
    const int need_off = need_base + block_excl_scan(need, &tn, s_wsum);
    const int row_off = row_base + block_excl_scan(n, &tr, s_wsum);
    if (b < p.B) {
      const int have = pages_of(L);
      int32_t* row = p.block_table + (size_t)b * p.W;
      for (int j = 0; j < need; ++j) row[have + j] = p.free_pages[count - 1 - (need_off + j)];
      for (int i = 0; i < n; ++i) {
        const int pos = L + i, jp = pos / kPage;
        const int pg = jp < have ? row[jp] : p.free_pages[count - 1 - (need_off + jp - have)];
        p.row_tok[row_off + i] = pg * kPage + pos % kPage;
      }
      p.seq_lens[b] = L + n;
    }
    need_base += tn;
    row_base += tr;
  }
  if (threadIdx.x == 0) {
    *p.free_count = count - need_all;
    *p.go = 1;
  }
}

// One thread per 16-byte piece: piece e covers (row r, KV head g, pool K or
// V, 8-dim slice c) with c fastest, then the pool, then g, then r.
__global__ __launch_bounds__(kCopyThreads) void kv_append_copy_kernel(KvParams p) {
  const int nc = p.D / 8;
  const long e = (long)blockIdx.x * kCopyThreads + threadIdx.x;
  const long n_pieces = (long)p.total_q * p.Hkv * 2 * nc;
  if (e >= n_pieces || *p.go == 0) return;
  const int c = (int)(e % nc);
  const int kind = (int)((e / nc) % 2);
  const int g = (int)((e / (2 * nc)) % p.Hkv);
  const int r = (int)(e / (2L * nc * p.Hkv));
  const int tok = p.row_tok[r];
  const int page = tok / kPage, slot = tok % kPage;
  const uint16_t* src = (kind ? p.v_new : p.k_new) + ((size_t)r * p.Hkv + g) * p.D + c * 8;
  uint16_t* dst = (kind ? p.v_pool : p.k_pool) + (((size_t)page * p.Hkv + g) * kPage + slot) * p.D + c * 8;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
}

// Quantized pools: one wave per vector w = (row r, KV head g, pool K or V),
// the pool fastest, encodes the row's D values straight into the codes and
// scale of its destination slot.
template <int QBITS, int D>
__global__ __launch_bounds__(kCopyThreads) void kv_append_quant_kernel(KvParams p) {
  const long w = (long)blockIdx.x * (kCopyThreads / 64) + (threadIdx.x >> 6);
  if (w >= (long)p.total_q * p.Hkv * 2 || *p.go == 0) return;
  const int kind = (int)(w % 2);
  const int g = (int)((w / 2) % p.Hkv);
  const int r = (int)(w / (2L * p.Hkv));
  const int tok = p.row_tok[r];
  const size_t slot = ((size_t)(tok / kPage) * p.Hkv + g) * kPage + tok % kPage;  // vector index in the pool
  const uint16_t* src = (kind ? p.v_new : p.k_new) + ((size_t)r * p.Hkv + g) * D;
  char* codes = reinterpret_cast<char*>(kind ? p.v_pool : p.k_pool) + slot * (D * QBITS / 8);
  float* scale = (kind ? p.v_scales : p.k_scales) + slot;
  if constexpr (QBITS == 8)
    q8_encode_wave<D>(src, reinterpret_cast<int8_t*>(codes), scale);
  else
    q4_encode_wave<D>(src, reinterpret_cast<uint8_t*>(codes), scale);
}

// ----------------------------------------------------------------- rollback

__global__ __launch_bounds__(kPlanThreads) void kv_rollback_kernel(KvParams p) {
  __shared__ int s_wsum[kPlanWaves];
  __shared__ u32 s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int count = *p.free_count;
  int rel_all = 0;
  for (int t0 = 0; t0 < p.B; t0 += kPlanThreads) {
    const int b = t0 + threadIdx.x;
    int rel = 0;
    if (b < p.B) {
      const int S = p.seq_lens[b], n = p.q_lens[b], a = p.accepted[b];
      if (a < 0 || a > n || n > S || pages_of(S) > p.W)
        atomicOr(&s_bad, (u32)PKV_EFLAG_QLEN);
      else
        rel = pages_of(S) - pages_of(S - n + a);
    }
    int tr;
    block_excl_scan(rel, &tr, s_wsum);
    rel_all += tr;
  }
  __syncthreads();
  u32 bad = s_bad;
  if (count < 0 || (long)count + rel_all > p.P) bad |= PKV_EFLAG_SPACE;
  if (bad) {
    if (threadIdx.x == 0) atomicOr(p.err, bad);
    return;
  }
  int rel_base = 0;
  for (int t0 = 0; t0 < p.B; t0 += kPlanThreads) {
    const int b = t0 + threadIdx.x;
    int S = 0, keep = 0, rel = 0;
    if (b < p.B) {
      S = p.seq_lens[b];
      keep = S - p.q_lens[b] + p.accepted[b];
      rel = pages_of(S) - pages_of(keep);
    }
    int tr;
    const int off = rel_base + block_excl_scan(rel, &tr, s_wsum);
    if (b < p.B) {
      int32_t* row = p.block_table + (size_t)b * p.W;
      const int first = pages_of(keep);
      for (int j = 0; j < rel; ++j) {
        p.free_pages[count + off + j] = row[first + j];
        row[first + j] = -1;
      }
      p.seq_lens[b] = keep;
    }
    rel_base += tr;
  }
  if (threadIdx.x == 0) *p.free_count = count + rel_all;
}

}  // namespace

KvWorkspace kv_workspace(int total_q) {
  KvWorkspace ws;
  ws.err_off = 0;
  ws.go_off = 4;
  ws.rows_off = 256;
  ws.total = ws.rows_off + ((size_t)(total_q > 0 ? total_q : 1) * 4 + 255) / 256 * 256;
  return ws;
}

hipError_t launch_kv_append(const KvParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.total_q == 0) return e;
  if (p.qbits != 0) {
    const long vecs = (long)p.total_q * p.Hkv * 2;
    const dim3 grid((unsigned)((vecs + kCopyThreads / 64 - 1) / (kCopyThreads / 64)));
    if (p.qbits == 8 && p.D == 128) hipLaunchKernelGGL((kv_append_quant_kernel<8, 128>), grid, dim3(kCopyThreads), 0, stream, p);
    else if (p.qbits == 8) hipLaunchKernelGGL((kv_append_quant_kernel<8, 64>), grid, dim3(kCopyThreads), 0, stream, p);
    else if (p.D == 128) hipLaunchKernelGGL((kv_append_quant_kernel<4, 128>), grid, dim3(kCopyThreads), 0, stream, p);
    else hipLaunchKernelGGL((kv_append_quant_kernel<4, 64>), grid, dim3(kCopyThreads), 0, stream, p);
    return hipGetLastError();
  }
  const long pieces = (long)p.total_q * p.Hkv * 2 * (p.D / 8);
  const int grid = (int)((pieces + kCopyThreads - 1) / kCopyThreads);
  hipLaunchKernelGGL(kv_append_copy_kernel, dim3(grid), dim3(kCopyThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_rollback(const KvParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kv_rollback_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
