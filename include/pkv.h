/*
 * pkv -- paged K/V attention and greedy speculative accept for AMD MI355X
 * (gfx950). C ABI: plain pointers and sizes; no C++ or framework types cross
 * this boundary.
 *
 * Sources (cited by page title and section):
 *  - ExLlamaV2 "Dynamic Generator" page, "Continuous Batching": the K/V cache
 *    is reached through per-sequence block tables of fixed 256-token pages;
 *    growing or shrinking a batch only rewrites block indices; freed pages
 *    leave holes, so a table's indices need not be contiguous.
 *  - Same page, "Deduplication": several sequences may index the same page,
 *    so a shared prefix is stored once.
 *  - Hugging Face "Assisted Generation" page, "How Assisted Generation works"
 *    and "Assisted Generation loop": one forward pass scores every position of
 *    a draft window; the base model's tokens are compared with the drafts from
 *    the left; at the first mismatch its own token is kept and the rest
 *    dropped; the window (5 at first) grows by 2 after a full match and
 *    shrinks by 1 otherwise.
 *
 * Conventions for every entry point:
 *  - Device pointers are caller-owned device memory. The library allocates no
 *    device memory and keeps no per-call state (the one host object is the
 *    page allocator's, from pkv_pool_create until pkv_pool_destroy); every
 *    kernel is enqueued on `stream` (a hipStream_t; NULL means the default
 *    stream) and only the *_check_errors calls synchronise.
 *  - Shapes are checked on the host before any launch. Contents of device
 *    arrays are a caller contract (listed per call). Kernels never read or
 *    write outside the documented extents even when the contract is broken:
 *    an offending sequence is skipped and a bit is set in the workspace's
 *    error word (read it with pkv_attn_check_errors).
 *  - Return value: PKV_OK or a negative pkv_status. C++ exceptions never
 *    cross this boundary.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_PAGE_SIZE 256 /* tokens per page; fixed by the Dynamic Generator page */
#define PKV_MAX_Q_LEN 16  /* longest verify window (k drafts + 1) of the accept step   */
#define PKV_MAX_ROWS 64   /* q_len * (Hq / Hkv) served by the decode / verify kernel;
                             longer windows run the long-window (prefill) kernel     */

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,      /* a required pointer is NULL                         */
  PKV_ERR_SHAPE = -2,     /* a shape field is out of range (see each call)      */
  PKV_ERR_WORKSPACE = -3, /* workspace NULL or smaller than the queried size    */
  PKV_ERR_HIP = -4,       /* a HIP launch or runtime call failed                */
  PKV_ERR_SPACE = -5,     /* page allocator: not enough pages (nothing changed) */
  PKV_ERR_STATE = -6,     /* page allocator: a page is not in the state the call
                             needs, e.g. released more often than referenced    */
  PKV_ERR_SCRATCH = -7    /* allocation-free call: the shape needs more than its
                             fixed device scratch                               */
} pkv_status;

/* Error-word bits a kernel sets when a device array breaks its contract. */
#define PKV_EFLAG_PAGE 1u  /* a block-table entry the sequence needs is not in [0, num_pages) */
#define PKV_EFLAG_QLEN 2u  /* q_len > max_q_len, q_len > seq_len, or seq_len > max_pages_per_seq*256 */
#define PKV_EFLAG_ROWS 4u  /* sum(q_lens) exceeds total_q (append: differs from total_q)           */
#define PKV_EFLAG_SPACE 8u /* append: too few free pages, or a page on the free stack is not in
                              [0, num_pages); rollback: the free stack would pass num_pages        */

/* ------------------------------------------------------------------ attention */

typedef struct {
  int32_t num_seqs;          /* B >= 0                                              */
  int32_t num_q_heads;       /* Hq >= 1                                             */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0                             */
  int32_t head_dim;          /* D, 64 or 128                                        */
  int32_t page_size;         /* must be PKV_PAGE_SIZE                               */
  int32_t num_pages;         /* P >= 1: pages in each pool                          */
  int32_t max_pages_per_seq; /* W >= 1: row stride of block_table                   */
  int32_t total_q;           /* rows of q and out; must equal sum(q_lens)           */
  int32_t max_q_len;         /* 1 .. W * 256, >= every q_lens[b]; Hq/Hkv <= 64      */
  float scale;               /* softmax scale applied to q.k (e.g. 1/sqrt(D))       */
  int32_t total_pages;       /* planning hint, >= 0: the pages the batch's sequences
                                reference, sum of ceil(seq_len / 256), as the host
                                knows it; 0 = unknown (every row taken as W pages).
                                The key range is cut into splits from it, so a
                                ragged batch keeps every CU busy; any value gives
                                correct results, only the speed and the workspace
                                size depend on it                                    */
  int32_t pages_per_split;   /* 0..64: pages of K/V one workgroup streams; 0 = derived
                                from total_pages (pkv_attn_plan sets both from the
                                host's lengths). Speed and workspace size only     */
} pkv_attn_shape;

/* Bytes of device workspace pkv_attn_fwd needs for this shape (0 on a bad
 * shape). The workspace holds an error word, one merge counter per
 * (sequence, KV head) and per-split partial results. It must be zero-filled
 * before its first use and again before it is reused for a different shape
 * (pkv_attn_workspace_init does it); every call leaves the counters at zero. */
size_t pkv_attn_workspace_bytes(const pkv_attn_shape* shape);

/* Host-side plan for a batch whose lengths the host knows (seq_lens_host:
 * num_seqs int32 in host memory, read only; values past max_pages_per_seq * 256
 * count as that). Sets shape->total_pages and shape->pages_per_split to the
 * split length that models fastest: rounds of workgroups over the chip times
 * (split pages + a workgroup's fixed cost), so a ragged batch neither leaves
 * CUs idle behind a few long splits nor spills a second round of workgroups.
 * Only speed and pkv_attn_workspace_bytes change; results stay correct for any
 * plan. Returns PKV_OK, PKV_ERR_NULL or PKV_ERR_SHAPE. */
int pkv_attn_plan(pkv_attn_shape* shape, const int32_t* seq_lens_host);

/* Enqueue a zero fill of `bytes` bytes of workspace on `stream`. */
int pkv_attn_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * Paged attention for decode (q_len = 1) and speculative verification
 * (q_len = k + 1, causal inside the window), in one kernel; and for long
 * windows (a prompt prefill, or a chunk of one over cached tokens) with the
 * same definition: when max_q_len * (Hq/Hkv) > PKV_MAX_ROWS the whole batch
 * runs the long-window kernel (query tiles of 256 rows, no split of the key
 * range). Sources: the Dynamic Generator page, "Deduplication" (a job whose
 * prompt prefix is already cached only processes the rest: a window over
 * cached tokens), and the Assisted Generation page, "How Assisted Generation
 * works" (one pass scores every position of a window).
 *
 * q           bf16 [total_q, Hq, D]; rows packed by sequence, then window row.
 * k_pool      bf16 [P, Hkv, 256, D]: K of page p, KV head g, slot s at
 * v_pool            ((p * Hkv + g) * 256 + s) * D. Read only.
 * block_table int32 [B, W]: token t of sequence b is slot t % 256 of page
 *             block_table[b * W + t / 256]. Only the first ceil(seq_len/256)
 *             entries of a row are read; they may repeat across rows (shared
 *             pages) and appear in any order.
 * seq_lens    int32 [B]: tokens in the cache per sequence, window included.
 * q_lens      int32 [B]: window rows per sequence, 0..max_q_len, <= seq_len.
 *             Window row i of sequence b attends to tokens
 *             0 .. seq_len - q_len + i. q_len = 0 skips the sequence.
 * out         fp32 [total_q, Hq, D]: softmax(scale * q.K^T) V per row; q head h
 *             reads KV head h / (Hq / Hkv).
 * workspace   pkv_attn_workspace_bytes(shape) bytes (see there); one call at a
 *             time per workspace.
 * Slots past seq_len and unreferenced pages may hold anything (NaN included):
 * they never affect `out`. Results are deterministic: they depend only on the
 * contents a sequence references, not on which physical pages hold them.
 * Contract: block-table entries a sequence needs lie in [0, P); sum(q_lens) ==
 * total_q; q_len <= max_q_len; q_len <= seq_len <= W * 256; on the long-window
 * kernel also seq_len <= 2048 * 256 (longer sequences are skipped and flagged
 * PKV_EFLAG_QLEN).
 * Precision: fp32 scores and softmax; P enters P.V rounded to bf16 (rows =
 * q_len * Hq/Hkv <= 4 run on VALU dot products, more rows on the matrix
 * cores). On the matrix cores P enters as two bf16 terms (about 16
 * significant bits) wherever a key weighs more than 1/8 of its row sum so
 * far, and on the long-window kernel also for the first 64 keys: rows that a
 * few keys dominate would not average the rounding out.
 */
int pkv_attn_fwd(const void* q, const void* k_pool, const void* v_pool,
                 const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_lens,
                 float* out, const pkv_attn_shape* shape,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention over a batch whose sequences all begin with the same shared_pages
 * pages: a deduplicated prompt prefix (Dynamic Generator page,
 * "Deduplication": every job references the same cached pages). Windows of
 * any length: decode, verify, or the prefill of each job's private tail. Same
 * arguments, layouts and result as pkv_attn_fwd; the shared keys are attended
 * to once per KV head for all window rows of the batch (matrix cores, rows of
 * every sequence stacked, so a short window pads nothing on its own), the rest
 * of every sequence as in pkv_attn_fwd, and the two are merged by
 * log-sum-exp.
 * shared_pages = 0 is pkv_attn_fwd. Workspace: pkv_attn_shared_workspace_bytes
 * (zero-filled before its first use, like pkv_attn_fwd's; every call leaves
 * it ready for the next).
 * Contract, besides pkv_attn_fwd's: block_table[b][j] == block_table[0][j] for
 * j < shared_pages and every sequence b; seq_len - q_len >= shared_pages * 256
 * (every window row sees the whole shared prefix) for every sequence with
 * q_len > 0; 1 <= shared_pages < max_pages_per_seq. A sequence breaking it
 * gets undefined rows, and PKV_EFLAG_PAGE / PKV_EFLAG_QLEN is set.
 */
size_t pkv_attn_shared_workspace_bytes(const pkv_attn_shape* shape, int32_t shared_pages);

/* Host helper for the shared-prefix call: the largest shared_pages its
 * contract allows for this batch, from host copies of the block table
 * (block_table_host int32 [num_seqs, max_pages_per_seq]), seq_lens and q_lens
 * (int32 [num_seqs] each): the length of the table prefix every row shares
 * with row 0, cut so that every window row sees all of it (seq_len - q_len >=
 * shared_pages * 256 where q_len > 0) and at least one table entry stays past
 * it; 0 when nothing is shared or no sequence has a window. Returns that
 * count, or a negative pkv_status (PKV_ERR_NULL, PKV_ERR_SHAPE). */
int32_t pkv_shared_prefix_pages(const int32_t* block_table_host, const int32_t* seq_lens_host,
                                const int32_t* q_lens_host, const pkv_attn_shape* shape);
int pkv_attn_fwd_shared(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_lens,
                        float* out, const pkv_attn_shape* shape, int32_t shared_pages,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ Q8 cache */

/*
 * An 8-bit K/V cache. Source: the Dynamic Generator page, "Usage" (a
 * quantized cache mode takes the place of the plain one; an 8-bit mode is
 * announced as about as compact as FP8 and more accurate). The page gives no
 * format; this library's: every vector of head_dim values (one token of one
 * KV head) is stored as int8 codes with one fp32 scale,
 *   scale = max|x| / 127,  code = x / scale rounded to nearest (ties to even),
 * in IEEE binary32, codes in [-127, 127]; a zero vector has scale 0, a vector
 * holding a non-finite value scale NaN, both with codes 0. The cached value of
 * an element is bf16(code * scale): the fp32 product rounded to bf16, nearest
 * even. A token costs head_dim + 4 bytes per KV head (132 at D = 128, against
 * 256 in bf16).
 * Pool layouts: codes int8 [P, Hkv, 256, D], scales fp32 [P, Hkv, 256].
 */

/* Encode `rows` bf16 vectors src[rows, head_dim] into codes[rows, head_dim]
 * (int8) and scales[rows] (fp32), all device memory owned by the caller; a
 * whole pool is rows = P * Hkv * 256. rows in 0 .. 2^32, head_dim 64 or 128,
 * else PKV_ERR_SHAPE. Bit-exact: the same codes and scales for the same
 * input on any launch. */
int pkv_q8_encode(const void* src, void* codes, float* scales, int64_t rows, int32_t head_dim, void* stream);

/*
 * pkv_attn_fwd over a Q8 cache: the same result as pkv_attn_fwd over bf16
 * pools holding the cached values bf16(code * scale) (each chunk of keys is
 * decoded into LDS inside the gather, then attended to as bf16 keys are).
 * Arguments as pkv_attn_fwd's, with k_codes / v_codes int8 [P, Hkv, 256, D]
 * and k_scales / v_scales fp32 [P, Hkv, 256] in place of the bf16 pools;
 * workspace: pkv_attn_workspace_bytes. Decode / verify shapes only
 * (max_q_len * Hq/Hkv <= PKV_MAX_ROWS), else PKV_ERR_SHAPE. Slots past a
 * sequence's end are never read, codes nor scales.
 */
int pkv_attn_fwd_q8(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                    const float* v_scales, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* q_lens, float* out, const pkv_attn_shape* shape, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * A 4-bit K/V cache: the same scheme at 4 bits (the Dynamic Generator page,
 * "Usage", names a Q4 cache mode as the generator's quantized cache; it gives
 * no format): scale = max|x| / 7, code = x / scale rounded to nearest even,
 * codes in [-7, 7]; zero and non-finite vectors as for Q8. Codes are stored as
 * the nibble code + 8, two per byte: dim 2i in the low nibble of byte i. The
 * cached value is bf16(code * scale). A token costs head_dim / 2 + 4 bytes
 * per KV head (68 at D = 128).
 * Pool layouts: codes uint8 [P, Hkv, 256, D / 2], scales fp32 [P, Hkv, 256].
 */

/* Encode `rows` bf16 vectors src[rows, head_dim] into codes[rows, head_dim / 2]
 * (uint8, packed) and scales[rows] (fp32), as pkv_q8_encode. */
int pkv_q4_encode(const void* src, void* codes, float* scales, int64_t rows, int32_t head_dim, void* stream);

/* pkv_attn_fwd_q8 over a Q4 cache (k_codes / v_codes uint8 [P, Hkv, 256, D / 2]):
 * the same result as pkv_attn_fwd over the decoded values; same arguments,
 * workspace and limits. */
int pkv_attn_fwd_q4(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                    const float* v_scales, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* q_lens, float* out, const pkv_attn_shape* shape, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Synchronise `stream`, copy the error word of `workspace` into *flags
 * (PKV_EFLAG_* bits; 0 = every contract held) and clear it. It synchronises,
 * so it is not for use under stream (graph) capture. */
int pkv_attn_check_errors(void* workspace, void* stream, uint32_t* flags);

/* -------------------------------------------------------------------- accept */

typedef struct {
  int32_t num_seqs;   /* B >= 0                                   */
  int32_t vocab;      /* V >= 1                                   */
  int32_t total_rows; /* rows of logits, <= 65535; must equal sum(n_draft + 1) */
  int32_t max_draft;  /* >= every n_draft[b]; 0..PKV_MAX_Q_LEN - 1   */
} pkv_accept_shape;

/* Bytes of device workspace pkv_accept needs (0 on a bad shape). It holds one
 * 64-bit argmax key per chunk of each logits row; it must be zero-filled
 * before its first use, and every call leaves it zero again (so it can serve
 * any later shape whose workspace is no larger). */
size_t pkv_accept_workspace_bytes(const pkv_accept_shape* shape);

/*
 * Greedy accept over a verified window.
 *
 * logits     fp32 [total_rows, V]; sequence b owns n_draft[b] + 1 consecutive
 *            rows (same order as the attention rows). Row i < n predicts the
 *            token after window token i; row n is the bonus row.
 * draft_ids  int32 packed [sum(n_draft)]: the drafts of sequence b in order.
 * n_draft    int32 [B]: drafts per sequence (0 = plain decode).
 * out_accept int32 [B]: m + 1, where m is the first i < n with
 *            argmax(row i) != draft i (m = n if every draft matches); the +1
 *            is the base model's own token at position m.
 * out_next   int32 [B]: argmax(row m) -- the correction token, or the bonus
 *            token when every draft matched.
 * window     int32 [B] or NULL: if given, updated in place by the window
 *            rule (pkv_window_next).
 * argmax: lowest index among equal maxima; a NaN counts as the maximum and the
 * first NaN wins. Results are bit-exact.
 * A sequence whose rows or drafts break the contract gets out_accept = 0 and
 * out_next = -1. One call at a time per workspace. The call's last workgroup
 * waits for the others' chunk results; if they have not all arrived after
 * about 10 seconds (other work holding the GPU's compute units all that
 * time), every sequence gets out_accept = 0, out_next = -1 and the workspace
 * must be zero-filled again before its next use.
 * Contract: sum(n_draft + 1) == total_rows; n_draft[b] <= max_draft.
 */
int pkv_accept(const float* logits, const int32_t* draft_ids, const int32_t* n_draft,
               int32_t* out_accept, int32_t* out_next, int32_t* window,
               const pkv_accept_shape* shape, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * pkv_accept without a workspace argument and without any device allocation,
 * for callers that cannot allocate: code under stream (graph) capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments (less the
 * workspace), results, contract and errors as pkv_accept.
 *
 * The workspace is a fixed array of PKV_ACCEPT_SCRATCH_BYTES in each GPU's
 * device memory, held until the process ends. The first call on a device
 * looks up that device's copy and enqueues a zero fill of it (a kernel) on
 * `stream`; every call leaves it zero again. A shape whose workspace
 * (pkv_accept_workspace_bytes) exceeds PKV_ACCEPT_SCRATCH_BYTES returns
 * PKV_ERR_SCRATCH before anything is launched.
 * All calls on one GPU share its copy: calls that may overlap in time on one
 * GPU (other streams, other threads) race and give wrong results; order them
 * on one stream.
 */
#define PKV_ACCEPT_SCRATCH_BYTES (1u << 20)
int pkv_accept_noalloc(const float* logits, const int32_t* draft_ids, const int32_t* n_draft,
                       int32_t* out_accept, int32_t* out_next, int32_t* window,
                       const pkv_accept_shape* shape, void* stream);

/* The draft-window rule on the host: window + 2 when accepted == n_draft + 1
 * (every draft matched, including n_draft == 0), else max(1, window - 1). */
int32_t pkv_window_next(int32_t window, int32_t n_draft, int32_t accepted);

/* -------------------------------------------------------- cache append / rollback */

/*
 * Sources: ExLlamaV2 "Dynamic Generator" page, "Continuous Batching" (sequences
 * grow into 256-token pages reached through block tables; a batch changes by
 * rewriting block indices; freed pages leave holes that later jobs fill) and
 * Hugging Face "Assisted Generation" page, "Assisted Generation loop", step 4
 * (candidates after the first mismatch are discarded).
 *
 * One verify step runs: pkv_kv_append (the window's K/V into the pages,
 * seq_lens grows by q_len) -> pkv_attn_fwd (seq_lens includes the window) ->
 * pkv_accept -> pkv_kv_rollback (keep the accepted tokens, release pages).
 *
 * Free pages are a caller-owned device stack free_pages[0 .. *free_count) of
 * capacity num_pages. Allocation pops from the top, sequences in index order,
 * each sequence's new pages in table order; release pushes on top in the same
 * order. Page placement is therefore deterministic. A page that receives
 * appended tokens must belong to that sequence alone (shared dedup pages are
 * full prefix pages).
 *
 * Both calls check every contract before changing anything: on a violation
 * they set PKV_EFLAG_* bits in the workspace error word (read with
 * pkv_kv_check_errors) and leave every buffer as it was.
 */

typedef struct {
  int32_t num_seqs;          /* B >= 0                                              */
  int32_t num_kv_heads;      /* Hkv >= 1                                            */
  int32_t head_dim;          /* D, 64 or 128                                        */
  int32_t page_size;         /* must be PKV_PAGE_SIZE                               */
  int32_t num_pages;         /* P >= 1: pages in each pool; capacity of free_pages  */
  int32_t max_pages_per_seq; /* W >= 1: row stride of block_table                   */
  int32_t total_q;           /* rows of k_new / v_new = sum(q_lens) (append)        */
} pkv_kv_shape;

/* Bytes of device workspace for pkv_kv_append / pkv_kv_rollback with this
 * shape (0 on a bad shape): an error word, a flag and one int per window row.
 * Zero-fill it before its first use. One call at a time per workspace. */
size_t pkv_kv_workspace_bytes(const pkv_kv_shape* shape);

/*
 * Append window token i of sequence b (row sum(q_lens[0..b)) + i of k_new /
 * v_new) at position seq_lens[b] + i: slot pos % 256 of page
 * block_table[b][pos / 256], popping a free page for every table entry the
 * window grows into. Then seq_lens[b] += q_lens[b].
 * k_new, v_new bf16 [total_q, Hkv, D] (read); k_pool, v_pool bf16
 * [P, Hkv, 256, D] (written at the window's slots only); block_table int32
 * [B, W] (new entries written); seq_lens int32 [B] (in/out); q_lens int32 [B];
 * free_pages int32 [P], free_count int32 [1] (in/out).
 * Contract: 0 <= seq_len, 0 <= q_len, seq_len + q_len <= W * 256; the entry of a
 * partly filled last page that receives tokens lies in [0, P); sum(q_lens) ==
 * total_q; enough free pages, each in [0, P).
 */
int pkv_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, int32_t* block_table,
                  int32_t* seq_lens, const int32_t* q_lens, int32_t* free_pages, int32_t* free_count,
                  const pkv_kv_shape* shape, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Keep accepted[b] of the q_lens[b] window tokens that end each sequence:
 * seq_lens[b] becomes seq_lens[b] - q_lens[b] + accepted[b]; every table entry
 * wholly past the new length is pushed on the free stack and set to -1.
 * accepted is pkv_accept's out_accept (0 for a sequence it rejected).
 * Contract: 0 <= accepted <= q_len <= seq_len; ceil(seq_len / 256) <= W; the
 * stack stays within num_pages.
 */
/* pkv_kv_append into quantized pools (the Q8 and Q4 formats of pkv_q8_encode /
 * pkv_q4_encode): the same pages, table and length updates, with every window
 * row's vector encoded into its slot's codes and scale (codes int8
 * [P, Hkv, 256, D] for Q8, uint8 [P, Hkv, 256, D / 2] for Q4; scales fp32
 * [P, Hkv, 256]); the same contract and error behaviour. pkv_kv_rollback
 * serves every format (it touches no pool). */
int pkv_kv_append_q8(const void* k_new, const void* v_new, void* k_codes, float* k_scales, void* v_codes,
                     float* v_scales, int32_t* block_table, int32_t* seq_lens, const int32_t* q_lens,
                     int32_t* free_pages, int32_t* free_count, const pkv_kv_shape* shape, void* workspace,
                     size_t workspace_bytes, void* stream);
int pkv_kv_append_q4(const void* k_new, const void* v_new, void* k_codes, float* k_scales, void* v_codes,
                     float* v_scales, int32_t* block_table, int32_t* seq_lens, const int32_t* q_lens,
                     int32_t* free_pages, int32_t* free_count, const pkv_kv_shape* shape, void* workspace,
                     size_t workspace_bytes, void* stream);

int pkv_kv_rollback(int32_t* block_table, int32_t* seq_lens, const int32_t* q_lens, const int32_t* accepted,
                    int32_t* free_pages, int32_t* free_count, const pkv_kv_shape* shape, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Synchronise `stream`, copy the error word of a cache workspace into *flags
 * and clear it. */
int pkv_kv_check_errors(void* workspace, void* stream, uint32_t* flags);

/* ------------------------------------------------------------ page allocator */

/*
 * Sources: ExLlamaV2 "Dynamic Generator" page, "Continuous Batching" (a job
 * queue starts jobs while their pages fit; a finished job frees its pages; the
 * holes are filled by later jobs; unreferenced pages are defragmented when the
 * queue is empty), "Deduplication" (a new job references the K/V already cached
 * for its prompt prefix) and "Prompt caching" (the most recently used pages are
 * the last to be overwritten, so a later job sharing a prefix with a finished
 * one still finds it).
 *
 * pkv_pool is a host object (created and freed by the calls below; the only
 * memory this library allocates itself) that decides which page holds what;
 * it never touches device memory. Block tables and free stacks built from its
 * answers are the caller's to upload. Every page is FREE (holds nothing
 * reusable), CACHED (unreferenced, holds a full prompt page a later job may
 * reuse) or USED (referenced by block-table rows or free stacks the caller
 * keeps; the reference count is the number of holders).
 *
 * A full prompt page is found again by its prefix, every token id up to the
 * end of the page; the index keys it by a 64-bit FNV-1a hash chained over the
 * prompt's pages and confirms a hit against the page's own 256 tokens,
 * position and chain predecessor. New pages come from FREE pages, lowest index
 * first (filling holes), then by evicting the CACHED page released longest ago
 * (lowest index on ties), which forgets its prefix.
 * Calls on one pool must not overlap; different pools are independent.
 */
typedef struct pkv_pool pkv_pool;

/* A pool of num_pages pages (1 .. 2^23), all FREE; NULL on a bad size or when
 * host memory runs out. */
pkv_pool* pkv_pool_create(int32_t num_pages);
void pkv_pool_destroy(pkv_pool* pool);

/* out[0..2] = FREE, CACHED and USED page counts. */
int pkv_pool_stats(const pkv_pool* pool, int32_t* out);

/*
 * Pages for a job's prompt (tokens[0 .. n_tokens)): pages[0 .. *n_pages) in
 * table order, *n_pages = ceil(n_tokens / 256) <= max_pages. The prompt's full
 * pages are matched against the cache from the start until the first miss; a
 * page is matched only if at least one prompt token follows it, so the job
 * always has a token to prefill and never writes into a shared page. Matched
 * pages gain a reference (CACHED ones are revived); the rest are new USED
 * pages, and the new full ones are keyed by their prefix. *cached_tokens =
 * 256 x matched pages: the prefill starts there (its K/V is already in the
 * pages). All or nothing: PKV_ERR_SPACE when too few pages can be had.
 */
int pkv_pool_admit(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, int32_t* pages,
                   int32_t max_pages, int32_t* n_pages, int32_t* cached_tokens);

/* n new private USED pages (reference count 1, no prefix), e.g. to fill the
 * device free stack pkv_kv_append pops from. PKV_ERR_SPACE if too few. */
int pkv_pool_alloc(pkv_pool* pool, int32_t n, int32_t* pages);

/* One more reference on each USED page (a page may repeat): sharing a job's
 * pages with another holder. PKV_ERR_STATE (nothing changed) if one is not USED. */
int pkv_pool_retain(pkv_pool* pool, const int32_t* pages, int32_t n);

/* One reference fewer on each page (a page may repeat): a finished job's
 * table pages, or unused free-stack pages. At zero a keyed page becomes
 * CACHED, any other FREE. PKV_ERR_STATE (nothing changed) if a page would go
 * below zero. */
int pkv_pool_release(pkv_pool* pool, const int32_t* pages, int32_t n);

/*
 * Defragmentation plan. n_occ = pages not FREE. Movable pages (CACHED; also
 * USED when move_referenced != 0) at index >= n_occ move into the FREE pages
 * below n_occ, both in ascending order, so that every target is FREE and no
 * target is another move's source. With move_referenced every occupied page
 * ends up below n_occ. Writes remap[0 .. P) (old index -> new; identity except
 * moved pages), src/dst[0 .. *n_moves) (capacity P each), and updates the
 * pool. The caller then moves the contents (pkv_pool_copy_pages) and, for
 * moved USED pages, rewrites its block tables (pkv_table_remap) before using
 * them again. The generator does this only when its queue is empty.
 */
int pkv_pool_defrag(pkv_pool* pool, int32_t move_referenced, int32_t* remap, int32_t* src, int32_t* dst,
                    int32_t* n_moves);

/*
 * Device side of a defragmentation (or any page move): copy page src[i] of
 * both pools to page dst[i], every KV head, for i < n_moves.
 * k_pool, v_pool bf16 [P, Hkv, 256, D]; src, dst int32 device arrays [n_moves].
 * Contract: entries in [0, P); no page is both a source and a target; targets
 * distinct (pkv_pool_defrag's plans are). Moves with an entry outside [0, P)
 * are skipped and set PKV_EFLAG_PAGE in *err (a caller-owned device word,
 * may be NULL).
 */
int pkv_pool_copy_pages(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int32_t n_moves,
                        int32_t num_pages, int32_t num_kv_heads, int32_t head_dim, uint32_t* err, void* stream);

/* pkv_pool_copy_pages for pools of any page size: copy page src[i] of both
 * pool_a and pool_b (device buffers of num_pages pages of page_bytes bytes
 * each) to page dst[i], for i < n_moves; same contract and error word. A
 * quantized cache moves its code pools (page_bytes = Hkv * 256 * D for Q8,
 * Hkv * 256 * D / 2 for Q4) and then its scale pools (Hkv * 256 * 4).
 * page_bytes: a positive multiple of 16, else PKV_ERR_SHAPE. */
int pkv_pool_copy_page_bytes(void* pool_a, void* pool_b, const int32_t* src, const int32_t* dst, int32_t n_moves,
                             int32_t num_pages, int64_t page_bytes, uint32_t* err, void* stream);

/* Rewrite block_table[rows, width] in place: every entry t in [0, num_pages)
 * becomes remap[t] (remap: device int32 [num_pages], entries in [0,
 * num_pages)); negative entries stay; entries >= num_pages stay and set
 * PKV_EFLAG_PAGE in *err (device word, may be NULL). */
int pkv_table_remap(int32_t* block_table, int32_t rows, int32_t width, const int32_t* remap,
                    int32_t num_pages, uint32_t* err, void* stream);

/* ---------------------------------------------------------------------- misc */

const char* pkv_status_string(int status);
int pkv_version(void); /* major * 10000 + minor * 100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
