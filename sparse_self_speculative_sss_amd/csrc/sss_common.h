// Internal definitions shared by the HIP sources of libsss (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sss.h"

namespace sss {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSeg = 16;  // tokens per segment of the matrix-core path
// dynamic LDS a workgroup may request: the 160 KiB of a gfx950 compute unit
// minus a reserve for the kernels' static LDS (barrier reductions)
constexpr size_t kMaxLds = 159 * 1024;

// LDS bytes of one matrix-core workgroup (attn_mfma.hip).
size_t mfma_smem_bytes(int head_dim, int nwr, int nwt, long long ell_floats, bool qreg = false);

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Workgroup barrier that orders LDS accesses only: each wave's LDS
// operations complete before it meets the others, but global loads and
// stores in flight are not waited for (the workgroup-scope fence of
// __syncthreads waits for all of them, which makes every barrier of a
// latency-bound phase cost a memory round trip).  For exchanges through LDS
// only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders LDS accesses among the lanes of one wave (LDS operations of a wave
// complete in issue order; the fences keep the compiler from moving them
// across this point).  No instruction is emitted.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float qnan() { return __builtin_nanf(""); }

// Window start: first token of the recent window; L when there is no window.
__host__ __device__ __forceinline__ int window_start(int L, int window) {
  if (window <= 0) return L;
  return L - window > 0 ? L - window : 0;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Everything an attention launch needs.  One "unit" is a (request, KV head)
// pair; its rows are the n_q * G query rows that share the KV head
// (row r = i * G + g).  Logits are kept in the log2 domain internally
// (scale_log2 = sm_scale * log2(e)); outputs use natural logs.
struct AttnParams {
  // paged cache
  const void* k;
  const void* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t num_pages, page_size, num_kv_heads, head_dim, max_pages, max_seq_len;
  // queries / rows
  const void* q;  // [B][n_q][Hq][d]
  int32_t batch, n_q, num_q_heads, group, rows;
  float scale_log2;
  // split-KV: `num_chunks` chunks per unit (grid dimension); verify chunks
  // hold `chunk_tokens` tokens, draft chunks `chunk_items` list entries
  int32_t num_chunks, chunk_tokens, chunk_items;
  float* o_part;    // [U][num_chunks][rows][d] normalised partial O
  float* lse_part;  // [U][num_chunks][rows]   log2-domain partial LSE
  // final outputs (written directly when num_chunks == 1)
  void* o;
  float* lse;
  // verify: block importance partials, log2 domain, [U][max_blocks][rows];
  // when num_chunks == 1 the matrix-core kernel also writes block_scores
  int32_t block_size, max_blocks, score_row_start;
  float* ell;
  float* block_scores;
  int32_t ell_in_lds;      // LDS holds the log masses of a unit that fits in one chunk
  int32_t ell_lds_floats;  // their count (blocks of a chunk x rows)
  // draft
  const int32_t* sel;
  const int32_t* sel_count;
  int32_t max_sel, window;
  // >= 0: units whose request length is <= skip_len were finished by the
  // fused step kernel and are skipped; -1: none
  int32_t skip_len;
  // sparse verify: sel / sel_count hold a layout per query position,
  // [U][n_q][max_sel] / [U][n_q]; chunk 0 of each unit writes the length of
  // its segment list here (for the split merge)
  int32_t* list_len;
};

// Finalize a verify or draft launch: merge split partials (if any) and, for
// verify, turn the per-(block, row) partial log-masses into block scores.
struct FinalizeParams {
  int32_t batch, num_kv_heads, n_q, group, rows, head_dim;
  int32_t num_chunks, chunk_tokens, chunk_items;  // as in AttnParams
  int32_t dtype;  // sss_dtype of o
  const int32_t* seq_lens;
  int32_t max_seq_len, max_pages, page_size;
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  // verify only (ell == nullptr for draft)
  const float* ell;
  float* block_scores;
  int32_t block_size, max_blocks, score_row_start;
  // draft only: list length per unit is needed to know the chunk count
  const int32_t* sel_count;
  int32_t max_sel, window, draft;
  int32_t simple_list;  // draft list enumerated token by token (vector-ALU path)
  int32_t single_done;  // units that fit in one chunk were finished by the attention kernel
  int32_t skip_len;     // as in AttnParams
  const int32_t* list_len;  // sparse verify: segment list length per unit
};

// Fused step (fused.hip): work-list shape and in-kernel selection state.  The
// verify and draft halves use their own AttnParams; unit indices are
// (request, KV head) of each half.  Split units keep the partial layout of
// the one-launch-per-stage path ([unit][maxch][rows]...), so the same merge
// and selection kernels finish them.
struct FusedParams {
  int32_t nv_units;    // verify units (0: no verify half)
  int32_t nd_units;    // draft units run as separate items (0: none / chained)
  int32_t chunk_v, maxch_v;  // tokens per verify chunk; chunks of the longest unit
  int32_t chunk_d, maxch_d;  // list entries per draft chunk; chunks of the longest list
  // Top-N of the verify units (topk == 0: scores only)
  int32_t topk, topk_window, max_sel, chained;
  const int32_t* budget;
  int32_t* sel;
  int32_t* sel_count;
  // LDS byte offsets: block log masses of a verify chunk, the selection
  int32_t off_ell, off_sel;
  // finish kernel of split verify units: LDS offset and capacity of the
  // parked Top-N keys, offset of the selection its chained draft reads, and
  // whether it drafts the unit (chained steps with short draft lists)
  int32_t fin_off_keys, fin_keys_cap, fin_off_sel, fin_draft;
};

struct FusedPlanIn {
  int32_t head_dim;
  int32_t rows_v;        // n_q * G of the verify half (0: none)
  long long nv;          // verify units
  int32_t max_len_v, block_size_v;
  long long nd;          // draft units run as items
  int32_t list_max_d;    // longest draft list (16-token entries)
  int32_t chained, max_sel;
};

struct FusedPlan {
  int32_t nwr, nwt;
  int32_t chunk_v, maxch_v, chunk_d, maxch_d;
  int32_t off_ell, off_sel;
  size_t lds_bytes;
  long long max_items;
};

void fused_plan(const FusedPlanIn& in, FusedPlan& pl);

// KV write (kv_update.hip): rows [batch][n_new][num_kv_heads][head_dim] of
// k_new / v_new go to token pos0[b] + i of each request's paged cache.
struct KvWriteParams {
  void* k;
  void* v;
  const void* k_new;
  const void* v_new;
  const int32_t* page_table;
  const int32_t* pos0;
  int32_t num_pages, page_size, num_kv_heads, head_dim, max_pages, elem_bytes;
  int32_t batch, n_new;
};

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t s);
hipError_t launch_kv_commit(const int32_t* seq_lens, const int32_t* keep, int batch, int n_q,
                            int32_t* out, hipStream_t s);

// Host-side launchers (each returns hipGetLastError() of its launches).
hipError_t launch_fused(const FusedParams& f, const AttnParams& pv, const AttnParams& pd,
                        const FusedPlan& pl, int head_dim, hipStream_t s);
// Selection and chained draft of whole verify units after an unsplit verify
// launch, one workgroup per unit.  select_draft_lds gives the LDS bytes and
// the offsets of the selection and of the parked keys (FusedParams::off_sel,
// ::off_ell).
size_t select_draft_lds(int head_dim, int max_sel, int max_blocks, int32_t& off_sel,
                        int32_t& off_keys);
hipError_t launch_select_draft(const FusedParams& f, const AttnParams& pv, const AttnParams& pd,
                               int head_dim, hipStream_t s);
// The same, one wave per unit (units of at most 1024 candidates whose
// drafts run one wave per unit): select_draft_wave_lds gives the LDS bytes
// and the selection's offset (FusedParams::off_sel).
size_t select_draft_wave_lds(int head_dim, int max_sel, int32_t& off_sel);
hipError_t launch_select_draft_wave(const FusedParams& f, const AttnParams& pv,
                                    const AttnParams& pd, int head_dim, hipStream_t s);
// Selection and chained draft of split verify units after their merge
// launch, one workgroup per draft chunk (pd.num_chunks per unit), each
// selecting the unit itself: select_draft_split_lds gives the LDS bytes,
// the selection's offset (FusedParams::off_sel) and the parked keys'
// capacity (FusedParams::fin_keys_cap).
size_t select_draft_split_lds(int head_dim, int max_sel, int max_blocks, int32_t& off_sel,
                              int32_t& keys_cap);
hipError_t launch_select_draft_split(const FusedParams& f, const AttnParams& pv,
                                     const AttnParams& pd, int head_dim, hipStream_t s);
// One workgroup per split verify unit: merge, scores, selection and, with
// f.fin_draft, the chained draft.  finish_lds sets the fin_* LDS fields of f
// and returns the workgroup's LDS bytes.
size_t finish_lds(FusedParams& f, int head_dim, int max_blocks, bool draft);
hipError_t launch_fused_finish(const FusedParams& f, const AttnParams& pv, const AttnParams& pd,
                               int head_dim, size_t lds_bytes, hipStream_t s);
hipError_t launch_verify_mfma(const AttnParams& p, hipStream_t s);
// Verify of units with three 32-row tiles: three compute waves and a load
// wave per workgroup (verify_rows.hip), when a chunk's block log masses fit
// in LDS with two workgroups per compute unit (verify_rows_fits).
bool verify_rows_fits(const AttnParams& p);
bool verify_rows_fits_shape(int head_dim, int rows, int block_size, int page_size,
                            int chunk_tokens);
constexpr int kVerifyRowsWaves = 4;  // waves of a verify_rows workgroup
hipError_t launch_verify_rows(const AttnParams& p, hipStream_t s);
// Persistent chained step (persist.hip): LDS bytes and offsets of its
// workgroup (0: the step does not fit), and the launch over `grid`
// workgroups that loop over the units.
size_t persist_lds(int head_dim, int rows, int group, int max_blocks, int max_sel,
                   int32_t* offs /* [5] */);
hipError_t launch_persist_step(const AttnParams& pv, const AttnParams& pd, int max_sel,
                               int topk_window, const int32_t* budget, int32_t* sel,
                               int32_t* sel_count, int grid, hipStream_t s);
// Sparse verify (a layout per query position): LDS bytes beyond the tiles,
// and the launch.
size_t sparse_union_lds_bytes(int max_blocks, int n_q, int max_sel);
// whether the per-block masks of a request of max_blocks blocks fit in the
// tile area of the configuration for nwr row tiles
bool sparse_union_fits(int head_dim, int nwr, int max_blocks);
hipError_t launch_sparse_verify_mfma(const AttnParams& p, hipStream_t s);
hipError_t launch_draft_mfma(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_simple(const AttnParams& p, int dtype, bool draft, hipStream_t s);
hipError_t launch_finalize(const FinalizeParams& p, hipStream_t s);
// skip_len >= 0: units whose request length is <= skip_len are left alone
// (the fused step kernel finished them); -1: every unit.
hipError_t launch_topk(const float* scores, int batch, int hkv, int max_blocks,
                       const int32_t* seq_lens, int block_size, const int32_t* budget,
                       int window, int32_t* sel, int32_t* sel_count, int max_sel, int skip_len,
                       hipStream_t s);
hipError_t launch_merge(const float* o_parts, const float* lse_parts, int num_parts, int rows,
                        int head_dim, void* o, int o_dtype, float* lse, hipStream_t s);

// Number of list entries (tokens) of a draft unit's attention list as the
// vector-ALU path enumerates it: selected blocks block by block, then the
// window.  Shared definition for kernels and finalize.
__host__ __device__ __forceinline__ int draft_list_len_simple(int nsel, int block_size, int L,
                                                              int ws) {
  return nsel * block_size + (L - ws);
}

// Matrix-core path: the list is made of 16-token segments.
__host__ __device__ __forceinline__ int draft_list_len_mfma(int nsel, int block_size, int L,
                                                            int ws) {
  const int spb = block_size / kSeg;
  const int w0 = (ws / kSeg) * kSeg;
  return nsel * spb + (ws < L ? ceil_div(L - w0, kSeg) : 0);
}

}  // namespace sss
