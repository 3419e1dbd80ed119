/*
 * sss.h -- C ABI of the sparse self-speculative decode attention library
 * (libsss.so, HIP for AMD MI355X / gfx950).
 *
 * The method (SparseSpec, "Accelerating Large-Scale Reasoning Model
 * Inference: Self-Speculative Decoding with Sparse Attention", §4.1 PillarAttn
 * and Fig. 7; SpecAttn, "SpecAttn: Co-Designing Sparse Attention with
 * Self-Speculative Decoding", technical framework): one model drafts k tokens
 * with attention restricted to a few critical KV blocks and verifies them with
 * full attention.  The verification pass already computes the softmax
 * probability of every cached token; its per-block mass, aggregated over the
 * verify rows of one GQA group, picks the blocks the next k drafts read.
 *
 * Entry points:
 *   sss_verify_attn  full causal attention of n_q = k+1 query tokens per
 *                    request over the whole paged cache, plus per-block
 *                    probability mass;
 *   sss_block_topk   per (request, KV head) Top-N block list;
 *   sss_draft_attn   single-query attention over the selected blocks plus a
 *                    recent window;
 *   sss_merge        log-sum-exp merge of split-KV partials;
 *   sss_fused_step   all of the above for a (mixed or chained) batch in one
 *                    work-list launch (or, for a chained step of whole
 *                    units, one persistent launch, or a verify launch and a
 *                    select-and-draft launch);
 *   sss_sparse_verify_attn  verify rows over a block layout per query
 *                    position, the union of a request's layouts loaded once;
 *   sss_kv_write     K/V of new token positions into the paged cache;
 *   sss_kv_commit    lengths after acceptance (drops rejected positions).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument except `kv` itself and the host structs points to
 *   DEVICE memory owned by the caller.  Inputs are read only; outputs must
 *   not alias inputs or each other.  The library allocates nothing: callers
 *   size the workspace with the matching *_workspace_size query.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *   enqueued asynchronously on it; the library never synchronises.
 * - Arguments are validated on the host before anything is launched.  A
 *   violated precondition returns SSS_ERR_INVALID_ARGUMENT or
 *   SSS_ERR_UNSUPPORTED and launches nothing; sss_last_error() then holds a
 *   message naming the argument.  SSS_ERR_HIP reports a failed launch.
 *   Faults during execution surface at the caller's next synchronisation.
 * - Device-resident values (seq_lens, budgets, selections) cannot be checked
 *   on the host.  Kernels clamp every index they derive from them to the
 *   buffers' stated sizes; a request whose seq_len exceeds
 *   kv->max_seq_len, kv->max_pages_per_req * page_size, or falls below the
 *   entry point's minimum gets NaN in its floating outputs.
 * - Results are bitwise reproducible for equal arguments on one GPU.
 * - Entry points only enqueue kernels (no allocation, memset or
 *   synchronisation), so they can be captured in a HIP graph.
 * - Query head hq reads KV head hq / G with G = num_q_heads / num_kv_heads.
 * - LSE values are natural-log log-sum-exp of the scaled logits.
 */
#ifndef SSS_H_
#define SSS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSS_OK = 0,
  SSS_ERR_INVALID_ARGUMENT = 1,
  SSS_ERR_UNSUPPORTED = 2,
  SSS_ERR_WORKSPACE_TOO_SMALL = 3,
  SSS_ERR_HIP = 4
} sss_status;

typedef enum { SSS_F32 = 0, SSS_BF16 = 1 } sss_dtype;

/*
 * Paged KV cache (SparseSpec §4.2: the paged cache of PagedAttention).
 *
 * k, v        [num_pages][num_kv_heads][page_size][head_dim], dense, in
 *             `dtype`; 16-byte aligned.  One (page, head) is a contiguous run
 *             of page_size * head_dim elements.
 * page_table  [batch][max_pages_per_req] int32: token t of request b lives in
 *             page page_table[b][t / page_size], slot t % page_size.  Entries
 *             past ceil(seq_lens[b] / page_size) are never read.
 * seq_lens    [batch] int32: KV length of each request.  For verify it
 *             counts the n_q new tokens, which occupy the last n_q positions.
 * max_seq_len host-side upper bound of seq_lens, used to size grids.
 *
 * Supported: dtype F32 or BF16; head_dim 64 or 128; page_size >= 1;
 * num_pages >= 1; max_pages_per_req >= ceil(max_seq_len / page_size);
 * num_pages * num_kv_heads * page_size < 2^31 token rows per tensor (else
 * SSS_ERR_UNSUPPORTED).
 */
typedef struct {
  const void* k;
  const void* v;
  int32_t dtype;
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_pages_per_req;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t max_seq_len;
} sss_paged_kv;

/*
 * Verify attention with block importance.
 *
 * Definition (SparseSpec §4.1 and Fig. 7; SpecAttn technical framework):
 * for request b, KV head h, query position i in [0, n_q) and group head g,
 * row r = i*G + g at position pos = L_b - n_q + i attends to tokens
 * t <= pos with logits s = sm_scale * <q, k_t>:
 *     lse[b][i][hq] = log sum_{t<=pos} exp(s_t),
 *     o[b][i][hq]   = sum_{t<=pos} exp(s_t - lse) v_t.
 * The per-block importance is the probability mass the scored rows put on
 * each block of `block_size` tokens, summed over the rows
 * r >= score_row_start * G of the unit:
 *     block_scores[b][h][j] = sum_r sum_{t in block j, t<=pos_r} exp(s_rt - lse_r).
 * With score_row_start = 1 only the k draft positions are scored (the
 * bonus row is skipped); 0 scores all k+1.  Blocks j >= ceil(L_b/block_size)
 * (up to max_blocks) are written as 0.
 *
 * q     [batch][n_q][num_q_heads][head_dim] in kv->dtype, 16-byte aligned.
 * o     same shape and dtype as q.
 * lse   [batch][n_q][num_q_heads] float.
 * block_scores [batch][num_kv_heads][max_blocks] float.
 * num_splits  number of KV chunks for the longest request (0 = chosen by
 *             the library); shorter requests use proportionally fewer.
 * workspace   device scratch of at least sss_verify_workspace_size() bytes,
 *             256-byte aligned; its contents on entry are irrelevant.
 *
 * Preconditions (host-checked): batch >= 0; 1 <= n_q <= 32;
 * num_q_heads % num_kv_heads == 0; n_q * G <= 128; block_size >= 1;
 * 0 <= score_row_start < n_q; max_blocks >= ceil(max_seq_len / block_size);
 * max_seq_len >= n_q; num_splits >= 0.  Device-side:
 * n_q <= seq_lens[b] <= max_seq_len.
 * Path: BF16 caches with page_size a multiple of 16 and block_size 16, a
 * multiple of 32, or 1 (single tokens, the page-size-1 selection of
 * SparseSpec §4.1) run the matrix-core (MFMA) kernel; every other supported
 * case runs the vector-ALU kernel.  Both compute in fp32 and round o once
 * to kv->dtype.
 */
sss_status sss_verify_attn(const sss_paged_kv* kv, const void* q, int32_t batch, int32_t n_q,
                           int32_t num_q_heads, float sm_scale, int32_t block_size,
                           int32_t score_row_start, int32_t num_splits, void* o, float* lse,
                           float* block_scores, int32_t max_blocks, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Workspace bytes sss_verify_attn needs for these arguments (0 on invalid
 * arguments; call sss_last_error() to see why). */
size_t sss_verify_workspace_size(const sss_paged_kv* kv, int32_t batch, int32_t n_q,
                                 int32_t num_q_heads, int32_t block_size, int32_t max_blocks,
                                 int32_t num_splits);

/* Bytes of the library's static device scratch (per GPU). */
#define SSS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * sss_verify_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and host
 * checks as sss_verify_attn (the same kernels and plan run, so outputs are
 * bitwise equal); the split partials and block log masses live in a static
 * device array of SSS_NOALLOC_SCRATCH_BYTES (32 MiB) that every GPU the
 * library runs on holds until the process ends.
 *
 * Nothing is allocated: no hipMalloc / hipFree, no allocating library call.
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, with the device current) and keeps its address.
 * Arguments whose workspace (sss_verify_workspace_size) exceeds
 * SSS_NOALLOC_SCRATCH_BYTES return SSS_ERR_WORKSPACE_TOO_SMALL and launch
 * nothing.  The scratch holds the last call's contents; nothing in it needs
 * to start at zero.  All calls on one GPU share the one array: calls that
 * overlap on that GPU (other streams, other host threads) race and give
 * wrong results -- serialise them.
 */
sss_status sss_verify_attn_noalloc(const sss_paged_kv* kv, const void* q, int32_t batch,
                                   int32_t n_q, int32_t num_q_heads, float sm_scale,
                                   int32_t block_size, int32_t score_row_start, int32_t num_splits,
                                   void* o, float* lse, float* block_scores, int32_t max_blocks,
                                   void* stream);

/*
 * Top-N block selection (SparseSpec §4.1: Top-K over the aggregated scores).
 *
 * For request b and KV head h with L = seq_lens[b] and window start
 * ws = max(0, L - window) (ws = L when window == 0), the candidates are the
 * blocks j < ceil(L/block_size) with j*block_size < ws.  The selection keeps
 * N = min(budget[b], #candidates, max_sel) candidates, ranked by larger
 * score first and lower index first among equal scores (-0.0 equals +0.0),
 * and writes them in ascending order:
 *     sel[b][h][0..N) ascending, sel[b][h][N..max_sel) = -1, sel_count[b][h] = N.
 * Scores must not be NaN.
 *
 * block_scores [batch][num_kv_heads][max_blocks] float (fp32 compared
 * exactly, so equal inputs give bit-identical selections);
 * seq_lens [batch], budget [batch] int32 (budget < 0 counts as 0);
 * sel [batch][num_kv_heads][max_sel] int32; sel_count [batch][num_kv_heads].
 * Preconditions: block_size >= 1; window >= 0; max_sel >= 1;
 * max_blocks >= 1.  Device-side: ceil(seq_lens[b]/block_size) <= max_blocks
 * (blocks past max_blocks are ignored).
 */
sss_status sss_block_topk(const float* block_scores, int32_t batch, int32_t num_kv_heads,
                          int32_t max_blocks, const int32_t* seq_lens, int32_t block_size,
                          const int32_t* budget, int32_t window, int32_t* sel,
                          int32_t* sel_count, int32_t max_sel, void* stream);

/*
 * Sparse draft attention (SpecAttn technical framework: drafting loads only
 * the critical KV entries; SparseSpec §4.1/§4.2).
 *
 * One query per (request, query head) at position L-1 attends to
 *     S = { t in block j : j in sel[b][h][0..sel_count), t < ws }  U  [ws, L)
 * with ws = max(0, L - window) (ws = L when window == 0):
 *     lse = log sum_{t in S} exp(s_t),  o = sum_{t in S} exp(s_t - lse) v_t.
 * An empty S gives o = 0 and lse = -inf.  Entries of sel that are negative
 * or past the sequence contribute no tokens; the listed entries must be
 * distinct.  Their order does not matter.
 *
 * q, o [batch][1][num_q_heads][head_dim] in kv->dtype; lse [batch][1][num_q_heads].
 * sel  [batch][num_kv_heads][max_sel] int32; sel_count [batch][num_kv_heads]
 * (clamped to [0, max_sel]).
 * num_splits number of chunks each unit's token list is cut into (0 = chosen
 * by the library).
 * Preconditions: num_q_heads % num_kv_heads == 0; G <= 128;
 * block_size >= 1; window >= 0; max_sel >= 1; num_splits >= 0.
 * Device-side: 1 <= seq_lens[b] <= max_seq_len.  Path: BF16 caches with
 * page_size and block_size multiples of 16 run the matrix-core kernel over
 * 16-token page runs; BF16 caches with block_size == 1 and G <= 32 run it
 * over single tokens gathered from the list; every other case runs the
 * vector-ALU kernel.
 */
sss_status sss_draft_attn(const sss_paged_kv* kv, const void* q, int32_t batch,
                          int32_t num_q_heads, float sm_scale, int32_t block_size,
                          const int32_t* sel, const int32_t* sel_count, int32_t max_sel,
                          int32_t window, int32_t num_splits, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

size_t sss_draft_workspace_size(const sss_paged_kv* kv, int32_t batch, int32_t num_q_heads,
                                int32_t block_size, int32_t max_sel, int32_t window,
                                int32_t num_splits);

/*
 * Sparse verification with a layout per query position (SpecSA, 核心创新 /
 * 重叠感知分组查询执行 and 技术细节与实现挑战 / 稀疏布局的动态管理: each query of
 * a verify step has its own sparse layout, and queries whose layouts
 * overlap run as one group that shares the KV blocks they have in common).
 *
 * Definition: for request b, KV head h and query position i in [0, n_q)
 * (row r = i*G + g, position pos = L_b - n_q + i), the query heads of the
 * group attend to
 *     S_i = ({ t in block j : j in row_sel[b][h][i][0..row_sel_count[b][h][i]),
 *              t < ws }  U  [ws, L_b))  restricted to t <= pos,
 * with ws = max(0, L_b - window) (ws = L_b when window == 0):
 *     lse[b][i][hq] = log sum_{t in S_i} exp(s_t),
 *     o[b][i][hq]   = sum_{t in S_i} exp(s_t - lse) v_t.
 * An empty S_i gives o = 0 and lse = -inf.  Layout entries that are
 * negative or name a block at or past the window start add nothing;
 * repeated entries and their order do not matter.
 *
 * Execution: each workgroup (one chunk of one request and KV head) builds the union of
 * the n_q layouts in LDS, loads each block of the union once for all the
 * unit's rows, and masks each row to its own position's blocks; a row wave
 * whose positions hold none of a tile's blocks skips that tile.
 *
 * q, o     [batch][n_q][num_q_heads][head_dim] BF16, 16-byte aligned.
 * lse      [batch][n_q][num_q_heads] float.
 * row_sel  [batch][num_kv_heads][n_q][max_sel] int32 block indices.
 * row_sel_count [batch][num_kv_heads][n_q] int32 (clamped to [0, max_sel]).
 * num_splits  chunks the longest possible union list is cut into (0 =
 *             chosen by the library).
 * workspace   device scratch of at least sss_sparse_verify_workspace_size()
 *             bytes, 256-byte aligned (0 bytes when nothing is split).
 *
 * Preconditions (host-checked): batch >= 0; 1 <= n_q <= 32;
 * num_q_heads % num_kv_heads == 0; n_q * G <= 128; max_sel >= 1;
 * window >= 0; num_splits >= 0; max_seq_len >= n_q; a BF16 cache with
 * page_size and block_size multiples of 16 (else SSS_ERR_UNSUPPORTED);
 * a 4-byte mask per block of the longest request, ceil(max_seq_len /
 * block_size), fits in the workgroup's K/V tile area while the union is
 * built (16880 blocks for up to 32 rows at head_dim 128, fewer for more rows
 * or head_dim 64), else SSS_ERR_UNSUPPORTED.  Device-side: n_q <= seq_lens[b] <= max_seq_len (else that unit's
 * outputs are NaN).  Caller owns every buffer; nothing is allocated.
 */
sss_status sss_sparse_verify_attn(const sss_paged_kv* kv, const void* q, int32_t batch,
                                  int32_t n_q, int32_t num_q_heads, float sm_scale,
                                  int32_t block_size, const int32_t* row_sel,
                                  const int32_t* row_sel_count, int32_t max_sel, int32_t window,
                                  int32_t num_splits, void* o, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Workspace bytes sss_sparse_verify_attn needs (0 when nothing is split or
 * on invalid arguments; call sss_last_error() to tell them apart). */
size_t sss_sparse_verify_workspace_size(const sss_paged_kv* kv, int32_t batch, int32_t n_q,
                                        int32_t num_q_heads, int32_t block_size, int32_t max_sel,
                                        int32_t window, int32_t num_splits);

/*
 * Log-sum-exp merge of attention partials over disjoint KV subsets (the
 * verification kernel keeps the log-sum-exp of the logits, SparseSpec §4.1,
 * which is what makes partial results combinable):
 *     lse[r] = log sum_s exp(lse_parts[s][r]),
 *     o[r]   = sum_s exp(lse_parts[s][r] - lse[r]) * o_parts[s][r].
 * Partials with lse -inf carry no weight; if every partial of a row is
 * -inf, o = 0 and lse = -inf.
 *
 * o_parts [num_parts][rows][head_dim] float; lse_parts [num_parts][rows] float;
 * o [rows][head_dim] in o_dtype (SSS_F32 or SSS_BF16); lse [rows] float (may
 * be NULL).  Preconditions: num_parts >= 1; rows >= 0; 1 <= head_dim <= 1024.
 */
sss_status sss_merge(const float* o_parts, const float* lse_parts, int32_t num_parts, int32_t rows,
                     int32_t head_dim, void* o, int32_t o_dtype, float* lse, void* stream);

/*
 * Fused decode step: verify, block scores, Top-N and sparse draft in one
 * work-list launch (SparseSpec §4.2, unified batch scheduler and fused
 * sparse/full attention: drafting and verifying requests share one
 * balanced launch instead of running as separate kernels).
 *
 * The verify half computes exactly what sss_verify_attn does for its
 * requests (o, lse, block_scores) and, when `sel` is non-NULL, what
 * sss_block_topk does on those scores (sel, sel_count, with `budget`,
 * `window`, `max_sel`).  The draft half computes what sss_draft_attn does
 * for its requests.  Either half may be NULL or have batch 0.
 *
 * chained == 0: the halves are independent request sets (a mixed batch in
 *   which some requests verify and the others draft).  Draft selections
 *   are inputs and must not alias the verify half's outputs.
 * chained != 0: the draft half drafts the verify half's own requests right
 *   after their selection: draft->kv must describe the same cache, page
 *   table and lengths as verify->kv, draft->batch == verify->batch,
 *   draft->block_size == verify->block_size, draft->max_sel ==
 *   verify->max_sel, and draft->sel / draft->sel_count must be
 *   verify->sel / verify->sel_count (written by this call, then read).
 *
 * Work decomposition: one launch with a slot per possible chunk -- every
 * verify unit (request, KV head) has ceil(max_seq_len / C) slots, every
 * unchained draft unit ceil(longest list / C') -- verify slots first, so
 * the small draft items fill the tail; slots past a unit's actual length
 * exit at once.  A unit that fits in one chunk is finished inside the
 * launch (outputs, scores, selection and, when chained, its draft).  Split
 * units are finished by follow-up launches on the same stream (merge and
 * scoring, selection, draft), which touch only those units.  A chained step
 * whose verify units all fit in one chunk, with no separate draft half,
 * runs as two launches instead: the one-launch verify kernel, then one
 * workgroup per unit that selects and drafts over the selection held in
 * LDS -- with 1024 or more units of at most 1024 candidates and draft lists
 * in one chunk, one wave per unit (the draft the separate entry point runs
 * for that many units); with 1024 or more units otherwise, the Top-N and
 * draft kernels of the separate entry points.  A chained step of split
 * units of 65 to 96 rows whose verify runs as load-wave workgroups (fewer
 * than 1024 units) takes no work list either: the verify and merge
 * launches of sss_verify_attn, one launch with a workgroup per draft chunk
 * that selects its unit's Top-N and drafts the chunk, then the draft merge
 * of sss_draft_attn (SSS_FUSED_ROWS_SPLIT below).
 *
 * Requirements beyond those of the separate entry points: both halves use
 * the matrix-core path (BF16 cache, page_size a multiple of 16, block_size
 * a multiple of 16 and, for a verify half, 16 or a multiple of 32) and the
 * same head_dim; the draft group size G <= 32; otherwise
 * SSS_ERR_UNSUPPORTED.  workspace: at least sss_fused_workspace_size()
 * bytes (0 when no unit can be split: NULL is then allowed), 256-byte
 * aligned, contents irrelevant on entry.  Results equal the separate entry
 * points' up to fp32 summation order: both run the same attention routine,
 * but a unit may be split into a different number of token groups or
 * chunks (the separate verify runs whole one-row-tile units as two token
 * groups when that lets two workgroups share a compute unit, the separate
 * draft runs one wave per unit when there are 1024 or more units), which
 * changes the rounding.  A chained step whose verify units all fit in one
 * chunk uses the separate verify kernel itself, so its verify outputs,
 * scores and selection are bitwise those of sss_verify_attn followed by
 * sss_block_topk (and, with 1024 or more units, its draft bitwise that of
 * sss_draft_attn over that selection); a step in the rows-split form
 * equals all three entry points bitwise.
 */
typedef struct {
  sss_paged_kv kv;
  const void* q;          /* [batch][n_q][num_q_heads][head_dim] */
  int32_t batch, n_q, num_q_heads;
  float sm_scale;
  int32_t block_size, score_row_start, max_blocks;
  void* o;                /* like q */
  float* lse;             /* [batch][n_q][num_q_heads] */
  float* block_scores;    /* [batch][num_kv_heads][max_blocks] */
  /* Top-N of the scores (sel == NULL: none) */
  const int32_t* budget;  /* [batch] */
  int32_t window;
  int32_t* sel;           /* [batch][num_kv_heads][max_sel] */
  int32_t* sel_count;     /* [batch][num_kv_heads] */
  int32_t max_sel;
} sss_verify_step;

typedef struct {
  sss_paged_kv kv;
  const void* q;          /* [batch][1][num_q_heads][head_dim] */
  int32_t batch, num_q_heads;
  float sm_scale;
  int32_t block_size;
  const int32_t* sel;     /* [batch][num_kv_heads][max_sel] */
  const int32_t* sel_count;
  int32_t max_sel, window;
  void* o;                /* like q */
  float* lse;             /* [batch][1][num_q_heads] */
} sss_draft_step;

sss_status sss_fused_step(const sss_verify_step* verify, const sss_draft_step* draft,
                          int32_t chained, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sss_fused_step that also records the caller's HIP event `verify_done`
 * (a hipEvent_t passed as void*; NULL: none) on `stream` right after the
 * launch that produces the verify outputs: in the two-launch form after the
 * verify kernel, in the persistent form after its one launch, in the
 * rows-split form after the verify's merge launch, in the
 * work-list form after the work-list launch (before the launches that
 * finish split units).  Events recorded around the call then time the
 * verify kernel inside a step.  The record is a stream barrier like any
 * event record; an event created without hipEventDisableSystemFence also
 * writes back the caches when it completes.  Same arguments, results and
 * errors as sss_fused_step, plus SSS_ERR_HIP if the record fails.  Not a
 * step of the method: a measurement hook.
 */
sss_status sss_fused_step_marked(const sss_verify_step* verify, const sss_draft_step* draft,
                                 int32_t chained, void* workspace, size_t workspace_bytes,
                                 void* stream, void* verify_done);

/* Workspace bytes sss_fused_step needs (0 on invalid arguments). */
size_t sss_fused_workspace_size(const sss_verify_step* verify, const sss_draft_step* draft,
                                int32_t chained);

/*
 * Which launch form sss_fused_step takes for these arguments (host query; no
 * device memory is read and nothing is launched):
 *   SSS_FUSED_PERSISTENT  a chained step of at least two units per compute
 *                         unit (512) whose verify units fit one workgroup
 *                         each, unless the two-launch form selects and
 *                         drafts with one wave per unit (1024 or more units
 *                         of at most 1024 candidates, which is faster):
 *                         one persistent launch whose workgroups loop
 *                         over units, drafting the unit each verified before
 *                         while the other workgroup on the compute unit
 *                         streams (SparseSpec §4.2, persistent-style fused
 *                         attention).  Verify outputs, scores and selections
 *                         are bitwise those of sss_verify_attn +
 *                         sss_block_topk; the draft splits its list over two
 *                         token groups and equals sss_draft_attn up to
 *                         summation order;
 *   SSS_FUSED_TWO_LAUNCH  other chained steps of whole units: the unsplit
 *                         verify launch, then selection and draft launches
 *                         (one launch of one wave per unit for 1024 or more
 *                         units of at most 1024 candidates);
 *   SSS_FUSED_ROWS_SPLIT  a chained step of split units of 65 to 96 rows
 *                         (k+1 positions x G heads) whose verify chunks run
 *                         as load-wave workgroups, with fewer than 1024
 *                         units and a draft of at most 32 heads per KV
 *                         head: the verify and merge launches of
 *                         sss_verify_attn, one launch in which each draft
 *                         chunk's workgroup selects its unit's Top-N and
 *                         drafts the chunk over it, and the draft merge of
 *                         sss_draft_attn.  Every output, score and
 *                         selection is bitwise that of sss_verify_attn +
 *                         sss_block_topk + sss_draft_attn with their
 *                         default splits;
 *   SSS_FUSED_WORK_LIST   everything else: the work-list launch plus the
 *                         merge / selection / draft launches of split units.
 * Returns -1 when sss_fused_step would reject the arguments (and 0 when
 * both halves are empty).
 */
enum {
  SSS_FUSED_NOTHING = 0,
  SSS_FUSED_PERSISTENT = 1,
  SSS_FUSED_TWO_LAUNCH = 2,
  SSS_FUSED_WORK_LIST = 3,
  SSS_FUSED_ROWS_SPLIT = 4
};
int32_t sss_fused_step_form(const sss_verify_step* verify, const sss_draft_step* draft,
                            int32_t chained);

/*
 * KV write for new token positions (SpecSA, 核心创新 / 刷新/复用NSA内核融合:
 * the KV of the speculative positions is written before verification and
 * refreshed -- overwritten -- when it is recomputed; the KV of accepted
 * tokens is then reused by later queries).
 *
 * For request b and i in [0, n_new), token t = pos0[b] + i gets
 *     k[page_table[b][t / page_size]][h][t % page_size][:] = k_new[b][i][h][:]
 * (and likewise v) for every KV head h.  Rows whose position lies outside
 * [0, max_pages_per_req * page_size) or whose page id lies outside
 * [0, num_pages) are skipped (nothing is written for them).  kv->seq_lens is
 * not read; the caller owns the lengths (see sss_kv_commit).
 *
 * k_new, v_new [batch][n_new][num_kv_heads][head_dim] in kv->dtype, 16-byte
 * aligned; pos0 [batch] int32.  THE CACHE PAGES kv->k / kv->v ARE WRITTEN
 * (the one exception to "inputs are read only").  Two rows of one call
 * must not map to the same slot.  Preconditions: batch >= 0, n_new >= 0.
 */
sss_status sss_kv_write(const sss_paged_kv* kv, const void* k_new, const void* v_new,
                        int32_t batch, int32_t n_new, const int32_t* pos0, void* stream);

/*
 * Commit after acceptance (SpecSA, 刷新/复用: rejected speculative positions
 * are dropped).  The last n_q positions of each request were speculative;
 * the first keep[b] of them (clamped to [0, n_q]) stay:
 *     new_seq_lens[b] = max(0, seq_lens[b] - n_q + clamp(keep[b], 0, n_q)).
 * Dropped positions are not touched in the cache: a position at or past a
 * request's length is never read, and the next sss_kv_write overwrites it.
 * seq_lens, keep, new_seq_lens [batch] int32; new_seq_lens may equal
 * seq_lens (in place).  Preconditions: batch >= 0, n_q >= 1.
 */
sss_status sss_kv_commit(const int32_t* seq_lens, const int32_t* keep, int32_t batch, int32_t n_q,
                         int32_t* new_seq_lens, void* stream);

/* Static description of a status code. */
const char* sss_status_string(sss_status status);

/* Message of the last failed call on this thread ("" if none). */
const char* sss_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t sss_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSS_H_ */
