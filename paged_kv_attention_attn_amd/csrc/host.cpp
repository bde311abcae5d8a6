// C ABI of the pkv library: host-side validation, workspace sizing, and
// kernel launch on the caller's stream. Declarations and the contract of each
// call are in include/pkv.h.

#include "pkv.h"
#include "internal.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>

namespace {

bool attn_shape_ok(const pkv_attn_shape* s) {
  if (!s) return false;
  if (s->num_seqs < 0 || s->num_q_heads < 1 || s->num_kv_heads < 1) return false;
  if (s->num_q_heads % s->num_kv_heads) return false;
  if (s->head_dim != 64 && s->head_dim != 128) return false;
  if (s->page_size != PKV_PAGE_SIZE) return false;
  if (s->num_pages < 1 || s->max_pages_per_seq < 1 || s->total_q < 0) return false;
  // windows up to the table's capacity; a head group up to the rows of one wave
  if (s->max_q_len < 1 || (long)s->max_q_len > (long)s->max_pages_per_seq * PKV_PAGE_SIZE) return false;
  if (s->num_q_heads / s->num_kv_heads > PKV_MAX_ROWS) return false;
  if (!std::isfinite(s->scale)) return false;
  if (s->total_pages < 0) return false;
  if (s->pages_per_split < 0 || s->pages_per_split > 64) return false;
  // 32-bit indexing limits inside the kernels
  if ((long)s->num_seqs * s->max_pages_per_seq > (1L << 31) - 1) return false;
  if ((long)s->num_pages * s->num_kv_heads * PKV_PAGE_SIZE * s->head_dim > (1L << 40)) return false;
  // work items, with every XCD's share of (KV head, split) pairs padded to a whole pair
  if ((long)s->num_seqs * ((long)s->num_kv_heads * s->max_pages_per_seq + 8) > (1L << 30)) return false;
  if ((long)s->total_q * s->num_q_heads * s->head_dim * 2 >= (1L << 32)) return false;  // q buffer offsets
  // long windows: one work item per (sequence, KV head, 256-row query tile)
  const int group = s->num_q_heads / s->num_kv_heads;
  if ((long)s->max_q_len * group > PKV_MAX_ROWS) {
    const long qtok = 256 / group;
    if ((long)s->num_seqs * s->num_kv_heads * ((s->max_q_len + qtok - 1) / qtok) > (1L << 30)) return false;
  }
  return true;
}

bool accept_shape_ok(const pkv_accept_shape* s) {
  if (!s) return false;
  if (s->num_seqs < 0 || s->vocab < 1 || s->total_rows < 0) return false;
  if (s->max_draft < 0 || s->max_draft > PKV_MAX_Q_LEN - 1) return false;
  if (s->total_rows < s->num_seqs) return false;
  if ((long)s->total_rows * s->vocab > (1L << 40)) return false;
  if (s->total_rows > 65535) return false;  // one grid row per logits row
  return true;
}

bool kv_shape_ok(const pkv_kv_shape* s) {
  if (!s) return false;
  if (s->num_seqs < 0 || s->num_kv_heads < 1 || s->total_q < 0) return false;
  if (s->head_dim != 64 && s->head_dim != 128) return false;
  if (s->page_size != PKV_PAGE_SIZE) return false;
  if (s->num_pages < 1 || s->max_pages_per_seq < 1) return false;
  // 32-bit indexing limits inside the kernels
  if ((long)s->num_pages * PKV_PAGE_SIZE > (1L << 31) - 1) return false;                  // page * 256 + slot
  if ((long)s->max_pages_per_seq * PKV_PAGE_SIZE > (1L << 31) - 1) return false;          // token positions
  if ((long)s->total_q * s->num_kv_heads * s->head_dim > (1L << 31) - 1) return false;     // copy pieces
  return true;
}

pkv::KvParams kv_params(const pkv_kv_shape* s, void* workspace) {
  const pkv::KvWorkspace ws = pkv::kv_workspace(s->total_q);
  char* w = static_cast<char*>(workspace);
  pkv::KvParams p{};
  p.err = reinterpret_cast<uint32_t*>(w + ws.err_off);
  p.go = reinterpret_cast<uint32_t*>(w + ws.go_off);
  p.row_tok = reinterpret_cast<int32_t*>(w + ws.rows_off);
  p.B = s->num_seqs;
  p.Hkv = s->num_kv_heads;
  p.D = s->head_dim;
  p.P = s->num_pages;
  p.W = s->max_pages_per_seq;
  p.total_q = s->total_q;
  return p;
}

pkv::AttnParams attn_params(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* q_lens, float* out, const pkv_attn_shape* s,
                            void* workspace, const pkv::AttnWorkspace& ws, const pkv::AttnPlan& plan,
                            int32_t page_offset) {
  char* w = static_cast<char*>(workspace);
  pkv::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = static_cast<const uint16_t*>(k_pool);
  p.v_pool = static_cast<const uint16_t*>(v_pool);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.q_lens = q_lens;
  p.out = out;
  p.err = reinterpret_cast<uint32_t*>(w + ws.err_off);
  p.counters = reinterpret_cast<uint32_t*>(w + ws.counters_off);
  p.part_ml = reinterpret_cast<float*>(w + ws.ml_off);
  p.part_acc = reinterpret_cast<float*>(w + ws.acc_off);
  p.B = s->num_seqs;
  p.Hq = s->num_q_heads;
  p.Hkv = s->num_kv_heads;
  p.group = s->num_q_heads / s->num_kv_heads;
  p.D = s->head_dim;
  p.P = s->num_pages;
  p.W = s->max_pages_per_seq;
  p.total_q = s->total_q;
  p.max_q_len = s->max_q_len;
  p.rows_max = plan.rows;
  p.pps = plan.pps;
  p.max_splits = plan.max_splits;
  p.num_items = s->num_seqs * s->num_kv_heads * (plan.prefill ? plan.tiles : plan.max_splits);
  p.scale_log2 = static_cast<float>(static_cast<double>(s->scale) * 1.4426950408889634);
  p.page_offset = page_offset;
  p.out_lse = nullptr;
  return p;
}

// The shared-prefix call: at least one page of every table past the shared
// ones (the tails run the split kernel, or the long-window kernel for windows
// of more than PKV_MAX_ROWS rows).
bool shared_shape_ok(const pkv_attn_shape* s, int32_t shared_pages) {
  if (!attn_shape_ok(s) || shared_pages < 0) return false;
  if (shared_pages == 0) return true;
  if (shared_pages >= s->max_pages_per_seq) return false;
  if ((long)s->total_q * (s->num_q_heads / s->num_kv_heads) > (1L << 24)) return false;
  return true;
}

// Workspace of the shared-prefix call: the tails' attention workspace (planned
// for the table width past the shared pages), each row's log-sum-exp, and the
// shared partials (none with a single key split).
struct SharedLayout {
  pkv::AttnWorkspace tail;
  pkv::AttnPlan plan;
  pkv::SharedPlan sp;
  size_t lse_off, ml_off, acc_off, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

SharedLayout shared_layout(const pkv_attn_shape* s, int32_t shared_pages) {
  SharedLayout L;
  const int group = s->num_q_heads / s->num_kv_heads;
  const int tail_w = s->max_pages_per_seq - shared_pages;
  // the tails reference the batch's pages less the shared ones of every row
  const long tail_pages = s->total_pages > 0 ? std::max(1L, s->total_pages - (long)s->num_seqs * shared_pages) : 0;
  // (a split length the caller planned for whole rows does not carry over)
  L.tail =
      pkv::attn_workspace(s->num_seqs, s->num_kv_heads, tail_w, s->max_q_len, group, s->head_dim, tail_pages, 0);
  L.plan = pkv::attn_plan(s->num_seqs, s->num_kv_heads, tail_w, s->max_q_len, group, tail_pages, 0);
  L.sp = pkv::shared_plan(s->num_kv_heads, s->total_q, group, shared_pages);
  const size_t rows = (size_t)s->total_q * group;
  // partials only with several key splits (one split merges in place)
  const size_t parts = L.sp.splits > 1 ? (size_t)s->num_kv_heads * L.sp.splits * rows : 0;
  L.lse_off = align256(L.tail.total);
  L.ml_off = align256(L.lse_off + (size_t)s->total_q * s->num_q_heads * 4);
  L.acc_off = align256(L.ml_off + parts * 2 * 4);
  L.total = align256(L.acc_off + parts * s->head_dim * 4);
  return L;
}

}  // namespace

extern "C" {

size_t pkv_attn_workspace_bytes(const pkv_attn_shape* s) {
  if (!attn_shape_ok(s)) return 0;
  const int group = s->num_q_heads / s->num_kv_heads;
  return pkv::attn_workspace(s->num_seqs, s->num_kv_heads, s->max_pages_per_seq, s->max_q_len, group,
                             s->head_dim, s->total_pages, s->pages_per_split)
      .total;
}

int pkv_attn_plan(pkv_attn_shape* s, const int32_t* seq_lens_host) {
  if (!s) return PKV_ERR_NULL;
  if (!attn_shape_ok(s)) return PKV_ERR_SHAPE;
  if (s->num_seqs > 0 && !seq_lens_host) return PKV_ERR_NULL;
  long pages = 0;
  for (int b = 0; b < s->num_seqs; ++b) {
    long n = std::min<long>(std::max<int32_t>(seq_lens_host[b], 0), (long)s->max_pages_per_seq * PKV_PAGE_SIZE);
    pages += (n + PKV_PAGE_SIZE - 1) / PKV_PAGE_SIZE;
  }
  const int group = s->num_q_heads / s->num_kv_heads;
  s->total_pages = (int32_t)std::min<long>(pages, INT32_MAX);
  s->pages_per_split = pkv::attn_best_pps(s->num_seqs, s->num_kv_heads, s->max_pages_per_seq, s->max_q_len, group,
                                          s->head_dim, seq_lens_host);
  return PKV_OK;
}

int pkv_attn_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return PKV_ERR_NULL;
  if (hipMemsetAsync(workspace, 0, bytes, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PKV_ERR_HIP;
  return PKV_OK;
}

int pkv_attn_fwd(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                 const int32_t* seq_lens, const int32_t* q_lens, float* out, const pkv_attn_shape* s,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!s) return PKV_ERR_NULL;
  if (!attn_shape_ok(s)) return PKV_ERR_SHAPE;
  if (s->num_seqs == 0 || s->total_q == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !q_lens || !out) return PKV_ERR_NULL;
  const int group = s->num_q_heads / s->num_kv_heads;
  const pkv::AttnWorkspace ws = pkv::attn_workspace(s->num_seqs, s->num_kv_heads, s->max_pages_per_seq,
                                                    s->max_q_len, group, s->head_dim, s->total_pages,
                                                    s->pages_per_split);
  if (!workspace || workspace_bytes < ws.total) return PKV_ERR_WORKSPACE;
  const pkv::AttnPlan plan = pkv::attn_plan(s->num_seqs, s->num_kv_heads, s->max_pages_per_seq,
                                            s->max_q_len, group, s->total_pages, s->pages_per_split);
  const pkv::AttnParams p =
      attn_params(q, k_pool, v_pool, block_table, seq_lens, q_lens, out, s, workspace, ws, plan, 0);
  if (pkv::launch_attn(p, plan, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

namespace {

int attn_fwd_quant(int qbits, const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                   const float* v_scales, const int32_t* block_table, const int32_t* seq_lens,
                   const int32_t* q_lens, float* out, const pkv_attn_shape* s, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!s) return PKV_ERR_NULL;
  if (!attn_shape_ok(s)) return PKV_ERR_SHAPE;
  if ((long)s->max_q_len * (s->num_q_heads / s->num_kv_heads) > PKV_MAX_ROWS) return PKV_ERR_SHAPE;
  if (s->num_seqs == 0 || s->total_q == 0) return PKV_OK;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !block_table || !seq_lens || !q_lens || !out)
    return PKV_ERR_NULL;
  const int group = s->num_q_heads / s->num_kv_heads;
  const pkv::AttnWorkspace ws = pkv::attn_workspace(s->num_seqs, s->num_kv_heads, s->max_pages_per_seq,
                                                    s->max_q_len, group, s->head_dim, s->total_pages,
                                                    s->pages_per_split);
  if (!workspace || workspace_bytes < ws.total) return PKV_ERR_WORKSPACE;
  const pkv::AttnPlan plan = pkv::attn_plan(s->num_seqs, s->num_kv_heads, s->max_pages_per_seq,
                                            s->max_q_len, group, s->total_pages, s->pages_per_split);
  pkv::AttnParams p =
      attn_params(q, k_codes, v_codes, block_table, seq_lens, q_lens, out, s, workspace, ws, plan, 0);
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  if (pkv::launch_attn_quant(p, plan, qbits, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

}  // namespace

int pkv_attn_fwd_q8(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                    const float* v_scales, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* q_lens, float* out, const pkv_attn_shape* s, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return attn_fwd_quant(8, q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens, out, s,
                        workspace, workspace_bytes, stream);
}

int pkv_attn_fwd_q4(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                    const float* v_scales, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* q_lens, float* out, const pkv_attn_shape* s, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return attn_fwd_quant(4, q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens, out, s,
                        workspace, workspace_bytes, stream);
}

int pkv_q8_encode(const void* src, void* codes, float* scales, int64_t rows, int32_t head_dim, void* stream) {
  if (rows < 0 || rows > (int64_t(1) << 32) || (head_dim != 64 && head_dim != 128)) return PKV_ERR_SHAPE;
  if (rows == 0) return PKV_OK;
  if (!src || !codes || !scales) return PKV_ERR_NULL;
  if (pkv::launch_q8_encode(static_cast<const uint16_t*>(src), static_cast<int8_t*>(codes), scales, (long)rows,
                            head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PKV_ERR_HIP;
  return PKV_OK;
}

int pkv_q4_encode(const void* src, void* codes, float* scales, int64_t rows, int32_t head_dim, void* stream) {
  if (rows < 0 || rows > (int64_t(1) << 32) || (head_dim != 64 && head_dim != 128)) return PKV_ERR_SHAPE;
  if (rows == 0) return PKV_OK;
  if (!src || !codes || !scales) return PKV_ERR_NULL;
  if (pkv::launch_q4_encode(static_cast<const uint16_t*>(src), static_cast<uint8_t*>(codes), scales, (long)rows,
                            head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PKV_ERR_HIP;
  return PKV_OK;
}

size_t pkv_attn_shared_workspace_bytes(const pkv_attn_shape* s, int32_t shared_pages) {
  if (!shared_shape_ok(s, shared_pages)) return 0;
  if (shared_pages == 0) return pkv_attn_workspace_bytes(s);
  return shared_layout(s, shared_pages).total;
}

int32_t pkv_shared_prefix_pages(const int32_t* table, const int32_t* seq_lens, const int32_t* q_lens,
                                const pkv_attn_shape* s) {
  if (!s) return PKV_ERR_NULL;
  if (!attn_shape_ok(s)) return PKV_ERR_SHAPE;
  if (s->num_seqs == 0) return 0;
  if (!table || !seq_lens || !q_lens) return PKV_ERR_NULL;
  const long W = s->max_pages_per_seq;
  bool any_window = false;
  long n = W - 1;  // at least one entry past the shared ones
  for (long b = 0; b < s->num_seqs; ++b) {
    if (q_lens[b] > 0) {  // every window row sees the whole shared prefix
      any_window = true;
      n = std::min<long>(n, std::max<long>(0, ((long)seq_lens[b] - q_lens[b]) / PKV_PAGE_SIZE));
    }
    long j = 0;  // every table starts with row 0's shared entries
    while (j < n && table[b * W + j] == table[j]) ++j;
    n = j;
  }
  return any_window ? (int32_t)n : 0;
}

int pkv_attn_fwd_shared(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                        const int32_t* seq_lens, const int32_t* q_lens, float* out, const pkv_attn_shape* s,
                        int32_t shared_pages, void* workspace, size_t workspace_bytes, void* stream) {
  if (!s) return PKV_ERR_NULL;
  if (!shared_shape_ok(s, shared_pages)) return PKV_ERR_SHAPE;
  if (shared_pages == 0)
    return pkv_attn_fwd(q, k_pool, v_pool, block_table, seq_lens, q_lens, out, s, workspace, workspace_bytes,
                        stream);
  if (s->num_seqs == 0 || s->total_q == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !q_lens || !out) return PKV_ERR_NULL;
  const SharedLayout L = shared_layout(s, shared_pages);
  if (!workspace || workspace_bytes < L.total) return PKV_ERR_WORKSPACE;
  char* w = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the tails: the split kernel (or, for long windows, the long-window
  // kernel) with the shared pages skipped, leaving each row's log-sum-exp too
  pkv::AttnParams p =
      attn_params(q, k_pool, v_pool, block_table, seq_lens, q_lens, out, s, workspace, L.tail, L.plan, shared_pages);
  p.out_lse = reinterpret_cast<float*>(w + L.lse_off);
  pkv::SharedParams sp{};
  sp.part_ml = reinterpret_cast<float*>(w + L.ml_off);
  sp.part_acc = reinterpret_cast<float*>(w + L.acc_off);
  sp.shared_pages = shared_pages;
  sp.splits = L.sp.splits;
  sp.split_keys = L.sp.split_keys;
  sp.row_tiles = L.sp.row_tiles;
  sp.tile_rows = L.sp.tile_rows;
  if (sp.splits == 1) {
    // tails first; the shared kernel merges its single split into them
    if (pkv::launch_attn(p, L.plan, st) != hipSuccess) return PKV_ERR_HIP;
    return pkv::launch_attn_shared(p, sp, st) != hipSuccess ? PKV_ERR_HIP : PKV_OK;
  }
  if (!L.plan.prefill && L.plan.max_splits == 1) {
    // decode / verify tails of one split each: the shared splits first, then
    // the tails, which merge them into their rows before writing them
    if (pkv::launch_attn_shared(p, sp, st) != hipSuccess) return PKV_ERR_HIP;
    pkv::AttnParams pt = p;
    pt.out_lse = nullptr;
    pt.shared_ml = sp.part_ml;
    pt.shared_acc = sp.part_acc;
    pt.shared_splits = sp.splits;
    return pkv::launch_attn(pt, L.plan, st) != hipSuccess ? PKV_ERR_HIP : PKV_OK;
  }
  // otherwise: tails, shared splits, then the merge
  if (pkv::launch_attn(p, L.plan, st) != hipSuccess) return PKV_ERR_HIP;
  if (pkv::launch_attn_shared(p, sp, st) != hipSuccess) return PKV_ERR_HIP;
  if (pkv::launch_shared_merge(p, sp, st) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

int pkv_attn_check_errors(void* workspace, void* stream, uint32_t* flags) {
  if (!workspace || !flags) return PKV_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return PKV_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return PKV_ERR_HIP;
  if (hipMemsetAsync(workspace, 0, 4, st) != hipSuccess) return PKV_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return PKV_ERR_HIP;
  *flags = v;
  return PKV_OK;
}

size_t pkv_accept_workspace_bytes(const pkv_accept_shape* s) {
  if (!accept_shape_ok(s)) return 0;
  return pkv::accept_workspace(s->num_seqs, s->total_rows, s->vocab).total;
}

// Checks shared by both accept entry points; PKV_OK when the call may go on
// (*skip set when there is nothing to do).
static int accept_args_ok(const float* logits, const int32_t* draft_ids, const int32_t* n_draft,
                          const int32_t* out_accept, const int32_t* out_next, const pkv_accept_shape* s,
                          bool* skip) {
  *skip = false;
  if (!s) return PKV_ERR_NULL;
  if (!accept_shape_ok(s)) return PKV_ERR_SHAPE;
  if (s->num_seqs == 0) {
    *skip = true;
    return PKV_OK;
  }
  if (!logits || !n_draft || !out_accept || !out_next) return PKV_ERR_NULL;
  if (!draft_ids && s->total_rows > s->num_seqs) return PKV_ERR_NULL;
  return PKV_OK;
}

static int accept_launch(const float* logits, const int32_t* draft_ids, const int32_t* n_draft, int32_t* out_accept,
                         int32_t* out_next, int32_t* window, const pkv_accept_shape* s,
                         const pkv::AcceptWorkspace& ws, void* workspace, void* stream) {
  char* w = static_cast<char*>(workspace);
  pkv::AcceptParams p;
  p.logits = logits;
  p.draft_ids = draft_ids;
  p.n_draft = n_draft;
  p.out_accept = out_accept;
  p.out_next = out_next;
  p.window = window;
  p.slots = reinterpret_cast<unsigned long long*>(w + ws.slots_off);
  p.B = s->num_seqs;
  p.V = s->vocab;
  p.total_rows = s->total_rows;
  p.max_draft = s->max_draft;
  p.chunks = ws.chunks;
  p.chunk_len = ws.chunk_len;
  if (pkv::launch_accept(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

int pkv_accept(const float* logits, const int32_t* draft_ids, const int32_t* n_draft, int32_t* out_accept,
               int32_t* out_next, int32_t* window, const pkv_accept_shape* s, void* workspace,
               size_t workspace_bytes, void* stream) {
  bool skip;
  const int rc = accept_args_ok(logits, draft_ids, n_draft, out_accept, out_next, s, &skip);
  if (rc != PKV_OK || skip) return rc;
  const pkv::AcceptWorkspace ws = pkv::accept_workspace(s->num_seqs, s->total_rows, s->vocab);
  if (!workspace || workspace_bytes < ws.total) return PKV_ERR_WORKSPACE;
  return accept_launch(logits, draft_ids, n_draft, out_accept, out_next, window, s, ws, workspace, stream);
}

int pkv_accept_noalloc(const float* logits, const int32_t* draft_ids, const int32_t* n_draft, int32_t* out_accept,
                       int32_t* out_next, int32_t* window, const pkv_accept_shape* s, void* stream) {
  bool skip;
  const int rc = accept_args_ok(logits, draft_ids, n_draft, out_accept, out_next, s, &skip);
  if (rc != PKV_OK || skip) return rc;
  const pkv::AcceptWorkspace ws = pkv::accept_workspace(s->num_seqs, s->total_rows, s->vocab);
  if (ws.total > pkv::kAcceptScratchBytes) return PKV_ERR_SCRATCH;
  void* scratch = nullptr;
  if (pkv::accept_scratch(static_cast<hipStream_t>(stream), &scratch) != hipSuccess) return PKV_ERR_HIP;
  return accept_launch(logits, draft_ids, n_draft, out_accept, out_next, window, s, ws, scratch, stream);
}

size_t pkv_kv_workspace_bytes(const pkv_kv_shape* s) {
  if (!kv_shape_ok(s)) return 0;
  return pkv::kv_workspace(s->total_q).total;
}

int pkv_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, int32_t* block_table,
                  int32_t* seq_lens, const int32_t* q_lens, int32_t* free_pages, int32_t* free_count,
                  const pkv_kv_shape* s, void* workspace, size_t workspace_bytes, void* stream) {
  if (!s) return PKV_ERR_NULL;
  if (!kv_shape_ok(s)) return PKV_ERR_SHAPE;
  if (s->num_seqs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !block_table || !seq_lens || !q_lens || !free_pages || !free_count) return PKV_ERR_NULL;
  if (s->total_q > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
  if (!workspace || workspace_bytes < pkv::kv_workspace(s->total_q).total) return PKV_ERR_WORKSPACE;
  pkv::KvParams p = kv_params(s, workspace);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_pool = static_cast<uint16_t*>(k_pool);
  p.v_pool = static_cast<uint16_t*>(v_pool);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.q_lens = q_lens;
  p.free_pages = free_pages;
  p.free_count = free_count;
  if (pkv::launch_kv_append(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

namespace {

int kv_append_quant(int qbits, const void* k_new, const void* v_new, void* k_codes, float* k_scales, void* v_codes,
                    float* v_scales, int32_t* block_table, int32_t* seq_lens, const int32_t* q_lens,
                    int32_t* free_pages, int32_t* free_count, const pkv_kv_shape* s, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!s) return PKV_ERR_NULL;
  if (!kv_shape_ok(s)) return PKV_ERR_SHAPE;
  if (s->num_seqs == 0) return PKV_OK;
  if (!k_codes || !v_codes || !k_scales || !v_scales || !block_table || !seq_lens || !q_lens || !free_pages ||
      !free_count)
    return PKV_ERR_NULL;
  if (s->total_q > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
  if (!workspace || workspace_bytes < pkv::kv_workspace(s->total_q).total) return PKV_ERR_WORKSPACE;
  pkv::KvParams p = kv_params(s, workspace);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_pool = static_cast<uint16_t*>(k_codes);
  p.v_pool = static_cast<uint16_t*>(v_codes);
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  p.qbits = qbits;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.q_lens = q_lens;
  p.free_pages = free_pages;
  p.free_count = free_count;
  if (pkv::launch_kv_append(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

}  // namespace

int pkv_kv_append_q8(const void* k_new, const void* v_new, void* k_codes, float* k_scales, void* v_codes,
                     float* v_scales, int32_t* block_table, int32_t* seq_lens, const int32_t* q_lens,
                     int32_t* free_pages, int32_t* free_count, const pkv_kv_shape* s, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return kv_append_quant(8, k_new, v_new, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens,
                         free_pages, free_count, s, workspace, workspace_bytes, stream);
}

int pkv_kv_append_q4(const void* k_new, const void* v_new, void* k_codes, float* k_scales, void* v_codes,
                     float* v_scales, int32_t* block_table, int32_t* seq_lens, const int32_t* q_lens,
                     int32_t* free_pages, int32_t* free_count, const pkv_kv_shape* s, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return kv_append_quant(4, k_new, v_new, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens,
                         free_pages, free_count, s, workspace, workspace_bytes, stream);
}

int pkv_kv_rollback(int32_t* block_table, int32_t* seq_lens, const int32_t* q_lens, const int32_t* accepted,
                    int32_t* free_pages, int32_t* free_count, const pkv_kv_shape* s, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!s) return PKV_ERR_NULL;
  if (!kv_shape_ok(s)) return PKV_ERR_SHAPE;
  if (s->num_seqs == 0) return PKV_OK;
  if (!block_table || !seq_lens || !q_lens || !accepted || !free_pages || !free_count) return PKV_ERR_NULL;
  if (!workspace || workspace_bytes < pkv::kv_workspace(s->total_q).total) return PKV_ERR_WORKSPACE;
  pkv::KvParams p = kv_params(s, workspace);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.q_lens = q_lens;
  p.accepted = accepted;
  p.free_pages = free_pages;
  p.free_count = free_count;
  if (pkv::launch_kv_rollback(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

int pkv_kv_check_errors(void* workspace, void* stream, uint32_t* flags) {
  return pkv_attn_check_errors(workspace, stream, flags);  // same word at offset 0
}

int32_t pkv_window_next(int32_t window, int32_t n_draft, int32_t accepted) {
  if (accepted == n_draft + 1) return window + 2;
  return window - 1 < 1 ? 1 : window - 1;
}

int pkv_pool_copy_pages(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int32_t n_moves,
                        int32_t num_pages, int32_t num_kv_heads, int32_t head_dim, uint32_t* err, void* stream) {
  if (n_moves < 0 || num_pages < 1 || num_kv_heads < 1 || (head_dim != 64 && head_dim != 128))
    return PKV_ERR_SHAPE;
  if (n_moves == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src || !dst) return PKV_ERR_NULL;
  if ((long)num_pages * num_kv_heads * PKV_PAGE_SIZE * head_dim > (1L << 40)) return PKV_ERR_SHAPE;
  pkv::PageMoveParams p{};
  p.k_pool = static_cast<uint16_t*>(k_pool);
  p.v_pool = static_cast<uint16_t*>(v_pool);
  p.src = src;
  p.dst = dst;
  p.err = err;
  p.n_moves = n_moves;
  p.P = num_pages;
  p.page_bytes = static_cast<long>(num_kv_heads) * PKV_PAGE_SIZE * head_dim * 2;
  if (pkv::launch_copy_pages(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

int pkv_pool_copy_page_bytes(void* pool_a, void* pool_b, const int32_t* src, const int32_t* dst, int32_t n_moves,
                              int32_t num_pages, int64_t page_bytes, uint32_t* err, void* stream) {
  if (n_moves < 0 || num_pages < 1 || page_bytes < 16 || page_bytes % 16 != 0) return PKV_ERR_SHAPE;
  if ((long)num_pages * page_bytes > (1L << 40)) return PKV_ERR_SHAPE;
  if (n_moves == 0) return PKV_OK;
  if (!pool_a || !pool_b || !src || !dst) return PKV_ERR_NULL;
  pkv::PageMoveParams p{};
  p.k_pool = static_cast<uint16_t*>(pool_a);
  p.v_pool = static_cast<uint16_t*>(pool_b);
  p.src = src;
  p.dst = dst;
  p.err = err;
  p.n_moves = n_moves;
  p.P = num_pages;
  p.page_bytes = static_cast<long>(page_bytes);
  if (pkv::launch_copy_pages(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

int pkv_table_remap(int32_t* block_table, int32_t rows, int32_t width, const int32_t* remap, int32_t num_pages,
                    uint32_t* err, void* stream) {
  if (rows < 0 || width < 1 || num_pages < 1 || (long)rows * width > (1L << 31) - 1) return PKV_ERR_SHAPE;
  if (rows == 0) return PKV_OK;
  if (!block_table || !remap) return PKV_ERR_NULL;
  if (pkv::launch_table_remap(block_table, rows * width, remap, num_pages, err, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return PKV_ERR_HIP;
  return PKV_OK;
}

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "shape field out of range";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch or runtime call failed";
    case PKV_ERR_SPACE: return "not enough pages";
    case PKV_ERR_STATE: return "a page is not in the state the call needs";
    case PKV_ERR_SCRATCH: return "shape needs more than the fixed scratch of the allocation-free call";
    default: return "unknown status";
  }
}

int pkv_version(void) { return 100; }

}  // extern "C"
