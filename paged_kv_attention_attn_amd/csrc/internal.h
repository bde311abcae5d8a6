// Internal launch interface between the C ABI (host.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kPage = 256;
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* q_lens;
  float* out;
  float* part_acc;      // [items][rows_max][D]
  float* part_ml;       // [items][rows_max][2] = (running max (log2 units), sum)
  uint32_t* counters;   // [B * Hkv] splits finished per (sequence, KV head)
  uint32_t* err;        // error word
  int32_t B, Hq, Hkv, group, D, P, W, total_q, max_q_len, rows_max;
  int32_t pps;          // pages per split
  int32_t max_splits;   // ceil(W / pps)
  int32_t num_items;    // B * Hkv * max_splits
  float scale_log2;     // scale * log2(e)
  int32_t page_offset;  // leading table entries skipped (a shared prefix attended to elsewhere), 0 otherwise
  float* out_lse;       // nullable: [total_q, Hq] base-2 log-sum-exp of each row's scaled scores
  const float* k_scales;  // quantized caches only: [P, Hkv, 256] per-token scales (k_pool / v_pool hold codes)
  const float* v_scales;
  // nullable: shared-prefix partials [Hkv][shared_splits][total_q * group] of
  // (m, l) and [D], merged in split order into each single-split row before
  // it is written (the shared-prefix call's tails)
  const float* shared_ml;
  const float* shared_acc;
  int32_t shared_splits;
};

// Workspace layout for a shape (byte offsets from the workspace base).
struct AttnWorkspace {
  size_t err_off, counters_off, ml_off, acc_off, total;
};

// Plan: pages per split and the kernel variant for a shape.
struct AttnPlan {
  int pps;
  int max_splits;
  int rows;      // rows_max = max_q_len * group
  bool mfma;     // row tile on matrix cores (rows >= 5)
  bool prefill;  // rows > PKV_MAX_ROWS: the long-window kernel
  int qtok;      // prefill: window tokens per query tile
  int tiles;     // prefill: query tiles of the longest window
};

// Shared-prefix path: key splits of the shared pages and their partials.
struct SharedParams {
  float* part_ml;       // [Hkv][splits][total_q * group][2] = (reference max (log2 units), row sum)
  float* part_acc;      // [Hkv][splits][total_q * group][D] unnormalised
  int32_t shared_pages, splits, split_keys, row_tiles, tile_rows;
};

struct SharedPlan {
  int splits, split_keys, row_tiles;
  // 0: the long-window kernel's 256-row tiles; 32 or 64: the decode / verify
  // kernel's matrix-core row tile (few rows per KV head), row_tiles of that size
  int tile_rows;
};

AttnPlan attn_plan(int B, int Hkv, int W, int max_q_len, int group, long total_pages, int pages_per_split);
// Pages per split for these host-side lengths: the least modelled time
// (rounds of workgroups x (split pages + a workgroup's fixed cost)); 0 for
// shapes on the long-window kernel.
int attn_best_pps(int B, int Hkv, int W, int max_q_len, int group, int D, const int32_t* seq_lens);
SharedPlan shared_plan(int Hkv, int total_q, int group, int shared_pages);
hipError_t launch_attn_shared(const AttnParams& p, const SharedParams& sp, hipStream_t stream);
hipError_t launch_shared_merge(const AttnParams& p, const SharedParams& sp, hipStream_t stream);
AttnWorkspace attn_workspace(int B, int Hkv, int W, int max_q_len, int group, int D, long total_pages,
                             int pages_per_split);
hipError_t launch_attn(const AttnParams& p, const AttnPlan& plan, hipStream_t stream);
// Same over a quantized cache (p.k_pool / p.v_pool: codes, qbits 8 = int8 or
// 4 = two nibbles per byte; p.k_scales / p.v_scales); decode / verify plans only.
hipError_t launch_attn_quant(const AttnParams& p, const AttnPlan& plan, int qbits, hipStream_t stream);
hipError_t launch_q8_encode(const uint16_t* src, int8_t* codes, float* scales, long rows, int D,
                            hipStream_t stream);
hipError_t launch_q4_encode(const uint16_t* src, uint8_t* codes, float* scales, long rows, int D,
                            hipStream_t stream);

struct AcceptParams {
  const float* logits;
  const int32_t* draft_ids;
  const int32_t* n_draft;
  int32_t* out_accept;
  int32_t* out_next;
  int32_t* window;              // nullable
  unsigned long long* slots;    // [total_rows][chunks] argmax key of each row chunk; zero between calls
  int32_t B, V, total_rows, max_draft, chunks, chunk_len;
};

struct AcceptWorkspace {
  size_t slots_off, total;
  int chunks, chunk_len;
};

struct KvParams {
  const uint16_t* k_new;     // [total_q, Hkv, D] bf16 bits
  const uint16_t* v_new;
  uint16_t* k_pool;          // [P, Hkv, 256, D]
  uint16_t* v_pool;
  int32_t* block_table;      // [B, W]
  int32_t* seq_lens;         // [B]
  const int32_t* q_lens;     // [B]
  const int32_t* accepted;   // [B] (rollback only)
  int32_t* free_pages;       // [P] stack of free page ids
  int32_t* free_count;       // stack height
  uint32_t* err;             // workspace error word
  uint32_t* go;              // append: 1 once the plan passed its checks
  int32_t* row_tok;          // append: [total_q] destination page * 256 + slot
  float* k_scales;           // quantized append: [P, Hkv, 256] (k_pool / v_pool hold codes)
  float* v_scales;
  int32_t qbits;             // 0: bf16 pools; 8 or 4: quantized (codes encoded from k_new / v_new)
  int32_t B, Hkv, D, P, W, total_q;
};

struct KvWorkspace {
  size_t err_off, go_off, rows_off, total;
};

KvWorkspace kv_workspace(int total_q);
hipError_t launch_kv_append(const KvParams& p, hipStream_t stream);
hipError_t launch_kv_rollback(const KvParams& p, hipStream_t stream);

struct PageMoveParams {
  uint16_t* k_pool;          // [P, Hkv, 256, D]
  uint16_t* v_pool;
  const int32_t* src;        // [n_moves]
  const int32_t* dst;
  uint32_t* err;             // nullable
  int32_t n_moves, P;
  long page_bytes;           // bytes of one page of one pool (all KV heads)
};

hipError_t launch_copy_pages(const PageMoveParams& p, hipStream_t stream);
hipError_t launch_table_remap(int32_t* table, int32_t n, const int32_t* remap, int32_t P, uint32_t* err,
                              hipStream_t stream);

AcceptWorkspace accept_workspace(int B, int total_rows, int V);
hipError_t launch_accept(const AcceptParams& p, hipStream_t stream);
// Allocation-free accept: the workspace is a fixed device array of
// kAcceptScratchBytes per GPU. accept_scratch returns its address on the
// current device (looked up, and zero-filled on `stream`, at the first call
// per device).
constexpr size_t kAcceptScratchBytes = PKV_ACCEPT_SCRATCH_BYTES;
hipError_t accept_scratch(hipStream_t stream, void** out);

}  // namespace pkv
