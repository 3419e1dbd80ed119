// Fused decode step: verify (with block scores and Top-N) and sparse draft
// in one launch driven by a device-built work list (SparseSpec §4.2: the
// unified batch scheduler mixes drafting and verifying requests in every
// step, and a single fused kernel serves both the sparse and the full
// attention; §5.5 / Fig. 15 compare it with launching the two in sequence).
//
// Workgroup i of fused_kernel owns one slot of a fixed work list: first the
// chunk slots of the verify units (chunk index maxch_v - 1 down to 0, every
// unit for each), then the chunk slots of every draft unit.  A slot past its unit's actual chunk
// count (known only on the device, from the lengths) exits at once.  The
// dispatcher hands out workgroups in index order as slots free up, so the
// large verify chunks start first and the small draft items fill the tail:
//   - a verify unit that fits in one chunk is finished in place: outputs,
//     block scores from the LDS-resident block masses, its Top-N selection
//     and, for a chained step, its draft over that fresh selection -- all
//     inside one workgroup, so only workgroup-scope ordering is needed;
//   - a chunk of a split verify unit, or of a split draft list, leaves a
//     normalised partial (and block log masses); the host then launches the
//     split-merge / scoring, selection and draft kernels for those units
//     only (kernel boundaries order them; no workgroup waits for another
//     and no device-scope fence is needed).
#include <algorithm>

#include "attn_item.h"
#include "topk_dev.h"

namespace sss {
namespace {

constexpr int kVerifyKind = 0, kDraftKind = 1;

__device__ __forceinline__ bool unit_valid(const AttnParams& p, int L, int min_len) {
  return L >= min_len && L <= p.max_seq_len && (long long)L <= (long long)p.max_pages * p.page_size;
}

// Number of chunks of unit u and the cost (tokens) of chunk c.
__device__ __forceinline__ int verify_chunks(const AttnParams& pv, int u, int chunk) {
  const int L = pv.seq_lens[u / pv.num_kv_heads];
  return unit_valid(pv, L, pv.n_q) ? ceil_div(L, chunk) : 1;
}
__device__ __forceinline__ int draft_segments(const AttnParams& pd, int u, int& valid) {
  const int b = u / pd.num_kv_heads;
  const int L = pd.seq_lens[b];
  valid = unit_valid(pd, L, 1);
  if (!valid) return 0;
  int nsel = pd.sel_count[u];
  nsel = nsel < 0 ? 0 : (nsel > pd.max_sel ? pd.max_sel : nsel);
  return draft_list_len_mfma(nsel, pd.block_size, L, window_start(L, pd.window));
}

// Top-N selection of verify unit u from its block scores (written by this
// workgroup before a workgroup barrier, or by an earlier launch) and, for a
// chained step, the draft of the same unit over that selection, read from
// an LDS copy at f.off_sel.  `keys` (LDS room for keys_cap words, or null)
// parks the selection's keys.  All NT = 64 * NWTD threads call it.
template <int D, int NWTD>
__device__ void select_then_draft(const FusedParams& f, const AttnParams& pv,
                                  const AttnParams& pd, int u, char* smem, uint32_t* keys,
                                  int keys_cap) {
  constexpr int NT = 64 * NWTD;
  const int b = u / pv.num_kv_heads;
  const int L = pv.seq_lens[b];
  int ncand, n;
  topk_bounds(L, pv.block_size, f.topk_window, pv.max_blocks, f.budget[b], f.max_sel, ncand, n);
  if (threadIdx.x == 0) f.sel_count[u] = n;
  int32_t* sel_s = reinterpret_cast<int32_t*>(smem + f.off_sel);
  static_assert(kTopkLdsWords * 4 <= Geo<D>::GROUP_BYTES,
                "selection scratch must fit in the tile area");
  topk_select<NT>(pv.block_scores + (long long)u * pv.max_blocks, ncand, n,
                  f.sel + (long long)u * f.max_sel, f.max_sel, f.chained ? sel_s : nullptr,
                  reinterpret_cast<int*>(smem), keys, keys_cap);
  if (!f.chained) return;
  // draft of the same unit over the selection just made
  const int Ld = pd.seq_lens[b];
  const int nseg = unit_valid(pd, Ld, 1)
                       ? draft_list_len_mfma(n, pd.block_size, Ld, window_start(Ld, pd.window))
                       : 0;
  Item dt;
  dt.u = u;
  dt.c = 0;
  dt.chunk = max(2 * NWTD, (nseg + 2 * NWTD - 1) / (2 * NWTD) * (2 * NWTD));
  dt.single = 1;
  dt.part_row0 = 0;
  dt.ell_off = 0;
  dt.sel_off = f.off_sel;
  dt.nsel_s = n;
  dt.list_off = 0;
  attn_item<D, 1, NWTD, true, false>(pd, dt, smem);
}

// One workgroup per work-list slot.  NWR row waves x NWT token groups for
// verify items; draft items (one row tile) use all NWR * NWT waves as token
// groups.
template <int D, int NWR, int NWT>
__global__ void __launch_bounds__(64 * NWR * NWT, 2)
    fused_kernel(FusedParams f, AttnParams pv, AttnParams pd) {
  constexpr int NT = 64 * NWR * NWT;
  constexpr int NWTD = NWR * NWT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const long long vslots = (long long)f.nv_units * f.maxch_v;
  int kind, u, c;
  if ((long long)blockIdx.x < vslots) {
    // last chunk index first: the long units' full chunks start first and
    // the units that fit in one chunk come last among the verify slots
    kind = kVerifyKind;
    c = f.maxch_v - 1 - (int)(blockIdx.x / f.nv_units);
    u = blockIdx.x % f.nv_units;
    // within a layer of slots, all KV heads of request r on XCD r % 8 (slot
    // b runs on XCD b % 8) with the requests dealt round-robin, as in the
    // one-item kernels, when the verify batch is a multiple of 8 (16
    // requests x 4K, interleaved A/B: 0.0891 -> 0.0882 ms per step)
    if ((pv.batch & 7) == 0 && (f.nv_units & 7) == 0) {
      const int H = pv.num_kv_heads, k = u >> 3;
      u = ((u & 7) + 8 * (k / H)) * H + k % H;
    }
    if (c >= verify_chunks(pv, u, f.chunk_v)) return;
  } else {
    kind = kDraftKind;
    const int i = (int)(blockIdx.x - vslots);
    u = i / f.maxch_d;
    c = i % f.maxch_d;
    if (c > 0) {
      int valid;
      const int nseg = draft_segments(pd, u, valid);
      if (!valid || c >= ceil_div(nseg, f.chunk_d)) return;
    }
  }

  if (kind == kVerifyKind) {
    const int b = u / pv.num_kv_heads;
    Item it;
    it.u = u;
    it.c = c;
    it.chunk = f.chunk_v;
    it.single = 0;
    it.part_row0 = (long long)u * f.maxch_v * pv.rows;
    it.ell_off = f.off_ell;
    it.sel_off = -1;
    it.nsel_s = 0;
    // a split unit's chunk leaves its partial; the follow-up launches finish it
    if (attn_item<D, NWR, NWT, false, true>(pv, it, smem) != kItemFinal || !f.topk) return;
    // this workgroup wrote the unit's block scores: order them before its
    // own reads, then select (and draft)
    __threadfence_block();
    __syncthreads();
    select_then_draft<D, NWTD>(f, pv, pd, u, smem, nullptr, 0);
  } else {
    Item it;
    it.u = u;
    it.c = c;
    it.chunk = f.chunk_d;
    it.single = 0;
    it.part_row0 = (long long)u * f.maxch_d * pd.rows;
    it.ell_off = 0;
    it.sel_off = -1;
    it.nsel_s = 0;
    attn_item<D, 1, NWTD, true, false>(pd, it, smem);
  }
}

// Selection and chained draft of whole verify units whose scores an
// unsplit verify launch wrote: one workgroup (one row tile of draft rows,
// kDraftWaves token groups) per unit.  LDS: the draft item's area, the
// selection at f.off_sel, then the unit's Top-N keys (f.off_ell) when
// max_blocks <= kSelectMaxKeys.
constexpr int kDraftWaves = 4;
constexpr int kSelectMaxKeys = 4096;

template <int D>
__global__ void __launch_bounds__(64 * kDraftWaves, 2)
    select_draft_kernel(FusedParams f, AttnParams pv, AttnParams pd) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const bool park = pv.max_blocks <= kSelectMaxKeys;
  select_then_draft<D, kDraftWaves>(f, pv, pd, blockIdx.x, smem,
                                    park ? reinterpret_cast<uint32_t*>(smem + f.off_ell) : nullptr,
                                    park ? pv.max_blocks : 0);
}

// Selection and chained draft of split verify units whose block scores a
// merge launch wrote, one workgroup per draft chunk (the chunking of
// sss_draft_attn: one row tile of draft rows, kDraftWaves token groups,
// partials merged by the merge launch that follows): every workgroup of a
// unit selects the unit's Top-N itself -- the same selection, held in LDS
// -- and chunk 0 writes it out; then each drafts its chunk of the list.
// The selection costs each workgroup one read of the unit's scores and the
// radix passes, in place of a Top-N launch between the merge and the draft
// (8 units of 2046 candidates: 10-11 us plus a 4-5 us gap).
template <int D>
__global__ void __launch_bounds__(64 * kDraftWaves, 2)
    select_draft_split_kernel(FusedParams f, AttnParams pv, AttnParams pd) {
  constexpr int NT = 64 * kDraftWaves;
  constexpr int kTopkBytes = (kTopkLdsWords * 4 + 127) / 128 * 128;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int u = (int)(blockIdx.x / (unsigned)pd.num_chunks);
  const int c = (int)(blockIdx.x % (unsigned)pd.num_chunks);
  const int b = u / pv.num_kv_heads;
  const int L = pv.seq_lens[b];
  int ncand, n;
  topk_bounds(L, pv.block_size, f.topk_window, pv.max_blocks, f.budget[b], f.max_sel, ncand, n);
  // chunks past the unit's draft list have nothing to do (as in attn_item;
  // chunk 0 always runs: it owns the unit's outputs and its selection)
  const int Ld = pd.seq_lens[b];
  const int nseg = unit_valid(pd, Ld, 1)
                       ? draft_list_len_mfma(n, pd.block_size, Ld, window_start(Ld, pd.window))
                       : 0;
  if (c > 0 && c * pd.chunk_items >= nseg) return;
  if (c == 0 && threadIdx.x == 0) f.sel_count[u] = n;
  int32_t* const sel_s = reinterpret_cast<int32_t*>(smem + f.off_sel);
  // the radix scratch and the parked keys borrow the draft's tile area
  const bool park = ncand <= f.fin_keys_cap;
  const float* const sc = pv.block_scores + (long long)u * pv.max_blocks;
  uint32_t* const keys = park ? reinterpret_cast<uint32_t*>(smem + kTopkBytes) : nullptr;
  const int cap = park ? f.fin_keys_cap : 0;
  if (c == 0)
    topk_select<NT>(sc, ncand, n, f.sel + (long long)u * f.max_sel, f.max_sel, sel_s,
                    reinterpret_cast<int*>(smem), keys, cap);
  else
    topk_select<NT, false>(sc, ncand, n, nullptr, f.max_sel, sel_s, reinterpret_cast<int*>(smem),
                           keys, cap);
  Item it;
  it.u = u;
  it.c = c;
  it.chunk = pd.chunk_items;
  it.single = pd.num_chunks == 1;
  it.part_row0 = (long long)u * pd.num_chunks * pd.rows;
  it.ell_off = 0;
  it.sel_off = f.off_sel;
  it.nsel_s = n;
  it.list_off = (int)item_lds_bytes(D, 1, kDraftWaves);
  attn_item<D, 1, kDraftWaves, true, false>(pd, it, smem);
}

// Selection and chained draft of whole verify units, one wave per unit, for
// batches whose drafts run one wave per unit anyway (at least four units
// per compute unit) and units of at most 64 * KPL candidates: the wave
// selects with topk_wave (no workgroup barrier; the histogram borrows the
// tile area, which the draft overwrites afterwards), keeps the selection in
// LDS and drafts over it.  This replaces the Top-N launch and the draft
// launch of such steps by one launch.  Units are taken in the XCD-aware
// order of the one-item kernels (all heads of request r on XCD r % 8 when
// the batch is a multiple of 8), so each wave reads the scores its unit's
// verify wrote on the same XCD.
template <int D, int KPL>
__global__ void __launch_bounds__(64, 2)
    select_draft_wave_kernel(FusedParams f, AttnParams pv, AttnParams pd) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int u = blockIdx.x;
  if ((pv.batch & 7) == 0) {
    const int H = pv.num_kv_heads, k = u >> 3;
    u = ((u & 7) + 8 * (k / H)) * H + k % H;
  }
  const int b = u / pv.num_kv_heads;
  int ncand, n;
  topk_bounds(pv.seq_lens[b], pv.block_size, f.topk_window, pv.max_blocks, f.budget[b], f.max_sel,
              ncand, n);
  if (threadIdx.x == 0) f.sel_count[u] = n;
  int32_t* sel_s = reinterpret_cast<int32_t*>(smem + f.off_sel);
  static_assert(kTopkBins * 4 <= Geo<D>::GROUP_BYTES, "histogram must fit in the tile area");
  topk_wave<KPL>(ScoreSrc{pv.block_scores + (long long)u * pv.max_blocks}, ncand, n,
                 f.sel + (long long)u * f.max_sel, f.max_sel, sel_s, reinterpret_cast<int*>(smem));
  const int Ld = pd.seq_lens[b];
  const int nseg =
      unit_valid(pd, Ld, 1) ? draft_list_len_mfma(n, pd.block_size, Ld, window_start(Ld, pd.window))
                            : 0;
  Item dt;
  dt.u = u;
  dt.c = 0;
  dt.chunk = max(2, (nseg + 1) / 2 * 2);
  dt.single = 1;
  dt.part_row0 = 0;
  dt.ell_off = 0;
  dt.sel_off = f.off_sel;
  dt.nsel_s = n;
  dt.list_off = 0;
  attn_item<D, 1, 1, true, false>(pd, dt, smem);
}

// Finishes the split verify units of a fused step, one workgroup per unit
// (eight waves, or four when it also drafts: the draft's token groups): merges the chunk partials into o / lse, turns the block
// log masses into block scores (keys parked in LDS), selects and, with
// f.fin_draft, drafts the unit over that selection (held in LDS).  Every
// phase issues its loads together: the partial LSEs with one batched copy,
// each thread's merge elements with all their partials at once, each
// block's rows at once; the selection reads the keys from LDS instead of
// the scores back from memory.  (One thread per output looping over
// dependent loads, the scores re-read for the selection, and the chained
// draft as a separate launch took 15.3 + 14.8 us for 16 requests x 8 KV
// heads of 4K tokens in 4 chunks.)
// waves of a finishing workgroup: eight, or four (the draft's token groups)
// when it drafts -- the 16-request chained step took 31.6 us with an
// eight-group draft against 25.4 us with four; the 96-request mixed batch's
// finish 20.9 us with eight waves against 30.9 us with four
template <bool DRAFT>
constexpr int finish_waves() { return DRAFT ? 4 : 8; }
constexpr int kFinishStage = 4096;  // partial LSEs staged in LDS (S * rows)
constexpr int kFinishLoads = 16;    // 16-byte loads a thread keeps in flight

__host__ __device__ constexpr int fin_off_stage_host() {
  return 512 + (int)((kTopkLdsWords * 4 + 15) / 16 * 16);
}
__device__ __forceinline__ int fin_off_stage() { return fin_off_stage_host(); }

// o = sum_s w_s o_s for elements e4 (float4 of row r = e4 / (D/4)) of the
// unit, EB elements per thread and SB partials of each loaded at once.
template <int NT, int D, int SB, int EB>
__device__ void finish_merge(const AttnParams& p, const f32x4* __restrict__ op, int S,
                             const float* lse2, const float* lpart, long long orow0, int b, int h) {
  constexpr int d4 = D / 4;
  const int R = p.rows, G = p.group;
  const int n4 = R * d4;
  bf16* o = reinterpret_cast<bf16*>(p.o);
  for (int e0 = 0; e0 < n4; e0 += EB * NT) {
    f32x4 acc[EB];
#pragma unroll
    for (int k = 0; k < EB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += SB) {
      f32x4 v[EB][SB];
#pragma unroll
      for (int k = 0; k < EB; ++k) {
        const int e4 = min(e0 + k * NT + (int)threadIdx.x, n4 - 1);
#pragma unroll
        for (int j = 0; j < SB; ++j)
          v[k][j] = op[(long long)min(s0 + j, S - 1) * n4 + e4];
      }
#pragma unroll
      for (int k = 0; k < EB; ++k) {
        const int e4 = min(e0 + k * NT + (int)threadIdx.x, n4 - 1);
        const int r = e4 / d4;
        const float tot = lse2[r];
        const bool live = tot == tot && tot != neg_inf();
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          const int s1 = s0 + j;
          const float w = (live && s1 < S) ? fast_exp2(lpart[s1 * R + r] - tot) : 0.f;
          acc[k][0] += w * v[k][j][0];
          acc[k][1] += w * v[k][j][1];
          acc[k][2] += w * v[k][j][2];
          acc[k][3] += w * v[k][j][3];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < EB; ++k) {
      const int e4 = e0 + k * NT + (int)threadIdx.x;
      if (e4 < n4) {
        const int r = e4 / d4;
        const float tot = lse2[r];
        const long long orow = orow0 + ((long long)(r / G)) * p.num_q_heads + h * G + r % G;
        bf16x4 w4;
#pragma unroll
        for (int c = 0; c < 4; ++c) w4[c] = from_f32<bf16>(tot != tot ? qnan() : acc[k][c]);
        *reinterpret_cast<bf16x4*>(o + orow * D + 4 * (e4 % d4)) = w4;
      }
    }
  }
}

// Block scores sum_r 2^(ell[j][r] - lse2[r]) over rows r0 .. r0 + 4 nq4 - 1
// (float4s), BB blocks per thread and batch with all their loads issued
// together; written to sc_out (0 past nblk) and, when parked, as Top-N keys.
template <int NT, int BB, int QMAX>
__device__ void finish_scores(const AttnParams& p, const float* ell, const float* lse2, int r0,
                              int nq4, int nblk, int ncand, bool park, float* sc_out,
                              uint32_t* keys) {
  const int R = p.rows;
  const int tid = threadIdx.x;
  for (int j0 = 0; j0 < p.max_blocks; j0 += BB * NT) {
    f32x4 x[BB][QMAX];
#pragma unroll
    for (int jb = 0; jb < BB; ++jb) {
      const int j = min(j0 + jb * NT + tid, max(nblk - 1, 0));
      const f32x4* e = reinterpret_cast<const f32x4*>(ell + (long long)j * R + r0);
#pragma unroll
      for (int q = 0; q < QMAX; ++q)
        if (q < nq4) x[jb][q] = e[q];
    }
#pragma unroll
    for (int jb = 0; jb < BB; ++jb) {
      const int j = j0 + jb * NT + tid;
      float sc = 0.f;
#pragma unroll
      for (int q = 0; q < QMAX; ++q)
        if (q < nq4) {
          const float* l2 = lse2 + r0 + 4 * q;
          sc += fast_exp2(x[jb][q][0] - l2[0]) + fast_exp2(x[jb][q][1] - l2[1]) +
                fast_exp2(x[jb][q][2] - l2[2]) + fast_exp2(x[jb][q][3] - l2[3]);
        }
      if (j < p.max_blocks) {
        if (j >= nblk) sc = 0.f;
        sc_out[j] = sc;
        if (park && j < ncand) keys[j] = score_key(sc);
      }
    }
  }
}

template <int D, bool DRAFT>
__global__ void __launch_bounds__(64 * finish_waves<DRAFT>(), 2)
    finish_kernel(FusedParams f, AttnParams p, AttnParams pd) {
  constexpr int kFinishWaves = finish_waves<DRAFT>();
  constexpr int kFinishThreads = 64 * kFinishWaves;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
  const int L = p.seq_lens[b];
  // units that fit in one chunk, and invalid ones, were finished in place
  if (!unit_valid(p, L, p.n_q) || L <= f.chunk_v) return;
  const int R = p.rows;
  const int S = ceil_div(L, f.chunk_v);
  float* lse2 = reinterpret_cast<float*>(smem);
  int* topk_lds = reinterpret_cast<int*>(smem + 512);
  float* lst = reinterpret_cast<float*>(smem + fin_off_stage());
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem + f.fin_off_keys);
  const float* lp = p.lse_part + (long long)u * f.maxch_v * R;
  const long long orow0 = (long long)b * p.n_q * p.num_q_heads;

  // When a thread's merge elements (all partials of each) or its blocks
  // (all rows of each) make one batch, their loads are issued here, before
  // the partial LSEs are reduced, so that the unit's partials arrive in one
  // memory round trip instead of three.  Only in the drafting (four-wave)
  // form: the registers would halve the eight-wave form's occupancy.
  constexpr int PEB = 4, PSB = 4;  // merge: elements per thread, partials
  constexpr int PBB = 2, PQ = 8;   // scores: blocks per thread, float4 rows
  const f32x4* op = reinterpret_cast<const f32x4*>(p.o_part) + (long long)u * f.maxch_v * R * (D / 4);
  const int n4 = R * (D / 4);
  const bool merge_pre = DRAFT && S <= PSB && n4 <= PEB * kFinishThreads;
  f32x4 mv[PEB][PSB];
  if (DRAFT && merge_pre) {
#pragma unroll
    for (int k = 0; k < PEB; ++k) {
      const int e4 = min(k * kFinishThreads + tid, n4 - 1);
#pragma unroll
      for (int j = 0; j < PSB; ++j) mv[k][j] = op[(long long)min(j, S - 1) * n4 + e4];
    }
  }
  const int nblk = ceil_div(L, p.block_size);
  const float* ell = p.ell + (long long)u * p.max_blocks * R;
  const int r0 = p.score_row_start * p.group;
  const bool vec = (R % 4) == 0 && (r0 % 4) == 0;
  const int nr = R - r0;
  const bool score_pre = DRAFT && vec && nr <= 4 * PQ && p.max_blocks <= PBB * kFinishThreads;
  f32x4 sx[PBB][PQ];
  if (DRAFT && score_pre) {
#pragma unroll
    for (int jb = 0; jb < PBB; ++jb) {
      const int j = min(jb * kFinishThreads + tid, max(nblk - 1, 0));
      const f32x4* e = reinterpret_cast<const f32x4*>(ell + (long long)j * R + r0);
#pragma unroll
      for (int q = 0; q < PQ; ++q)
        if (q < nr / 4) sx[jb][q] = e[q];
    }
  }

  // partial LSEs -> LDS, then each row's LSE over `lpr` lanes
  const bool staged = S * R <= kFinishStage;
  if (staged) {
    for (int i0 = 0; i0 < S * R; i0 += kFinishLoads * kFinishThreads) {
      float x[kFinishLoads];
#pragma unroll
      for (int k = 0; k < kFinishLoads; ++k) x[k] = lp[min(i0 + k * kFinishThreads + tid, S * R - 1)];
#pragma unroll
      for (int k = 0; k < kFinishLoads; ++k)
        if (i0 + k * kFinishThreads + tid < S * R) lst[i0 + k * kFinishThreads + tid] = x[k];
    }
  }
  lds_barrier();
  const float* lpart = staged ? lst : lp;
  {
    int lpr = 1;
    while (lpr < 16 && 2 * lpr * R <= kFinishThreads) lpr *= 2;
    const int q = tid % lpr;
    for (int rb = 0; rb < R; rb += kFinishThreads / lpr) {
      const int r = rb + tid / lpr;
      const bool live = r < R;
      float m = neg_inf();
      bool nan = false;
      if (live)
        for (int s0 = q; s0 < S; s0 += lpr) {
          const float x = lpart[s0 * R + r];
          nan |= (x != x);
          m = fmaxf(m, x);
        }
      for (int o = 1; o < lpr; o <<= 1) {
        m = fmaxf(m, __shfl_xor(m, o));
        nan |= __shfl_xor((int)nan, o) != 0;
      }
      float sum = 0.f;
      if (live && !nan && m != neg_inf())
        for (int s0 = q; s0 < S; s0 += lpr) sum += fast_exp2(lpart[s0 * R + r] - m);
      for (int o = 1; o < lpr; o <<= 1) sum += __shfl_xor(sum, o);
      if (live && q == 0) {
        const float tot = nan ? qnan() : (m == neg_inf() ? neg_inf() : m + fast_log2(sum));
        lse2[r] = tot;
        const int G = p.group;
        p.lse[orow0 + (long long)(r / G) * p.num_q_heads + h * G + r % G] = tot * kLn2;
      }
    }
  }
  lds_barrier();

  // merge: EB elements per thread, SB partials each, in flight together
  if (DRAFT && merge_pre) {
    bf16* o = reinterpret_cast<bf16*>(p.o);
    const int G = p.group;
#pragma unroll
    for (int k = 0; k < PEB; ++k) {
      const int e4 = k * kFinishThreads + tid;
      if (e4 < n4) {
        const int r = e4 / (D / 4);
        const float tot = lse2[r];
        const bool live = tot == tot && tot != neg_inf();
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < PSB; ++j) {
          const float w = (live && j < S) ? fast_exp2(lpart[j * R + r] - tot) : 0.f;
          acc[0] += w * mv[k][j][0];
          acc[1] += w * mv[k][j][1];
          acc[2] += w * mv[k][j][2];
          acc[3] += w * mv[k][j][3];
        }
        const long long orow = orow0 + ((long long)(r / G)) * p.num_q_heads + h * G + r % G;
        bf16x4 w4;
#pragma unroll
        for (int c = 0; c < 4; ++c) w4[c] = from_f32<bf16>(tot != tot ? qnan() : acc[c]);
        *reinterpret_cast<bf16x4*>(o + orow * D + 4 * (e4 % (D / 4))) = w4;
      }
    }
  } else if (S <= 2)
    finish_merge<kFinishThreads, D, 2, kFinishLoads / 2>(p, op, S, lse2, lpart, orow0, b, h);
  else if (S <= 4)
    finish_merge<kFinishThreads, D, 4, kFinishLoads / 4>(p, op, S, lse2, lpart, orow0, b, h);
  else
    finish_merge<kFinishThreads, D, 8, kFinishLoads / 8>(p, op, S, lse2, lpart, orow0, b, h);

  // block scores (every row of a block loaded at once), keys parked in LDS
  int ncand, n;
  topk_bounds(L, p.block_size, f.topk_window, p.max_blocks, f.topk ? f.budget[b] : 0, f.max_sel,
              ncand, n);
  const bool park = f.topk && ncand <= f.fin_keys_cap;
  float* sc_out = p.block_scores + (long long)u * p.max_blocks;
  // a thread scores BB blocks per batch with the float4s of all their rows
  // loaded together; scalar rows (counts not a multiple of 4) one block at
  // a time
  if (DRAFT && score_pre) {
#pragma unroll
    for (int jb = 0; jb < PBB; ++jb) {
      const int j = jb * kFinishThreads + tid;
      float sc = 0.f;
#pragma unroll
      for (int q = 0; q < PQ; ++q)
        if (q < nr / 4) {
          const float* l2 = lse2 + r0 + 4 * q;
          sc += fast_exp2(sx[jb][q][0] - l2[0]) + fast_exp2(sx[jb][q][1] - l2[1]) +
                fast_exp2(sx[jb][q][2] - l2[2]) + fast_exp2(sx[jb][q][3] - l2[3]);
        }
      if (j < p.max_blocks) {
        if (j >= nblk) sc = 0.f;
        sc_out[j] = sc;
        if (park && j < ncand) keys[j] = score_key(sc);
      }
    }
  } else if (vec && nr <= 4 * 4)
    finish_scores<kFinishThreads, 4, 4>(p, ell, lse2, r0, nr / 4, nblk, ncand, park, sc_out, keys);
  else if (vec && nr <= 4 * 8)
    finish_scores<kFinishThreads, 2, 8>(p, ell, lse2, r0, nr / 4, nblk, ncand, park, sc_out, keys);
  else if (vec && nr <= 4 * 16)
    finish_scores<kFinishThreads, 1, 16>(p, ell, lse2, r0, nr / 4, nblk, ncand, park, sc_out, keys);
  else
    for (int j = tid; j < p.max_blocks; j += kFinishThreads) {
      float sc = 0.f;
      if (j < nblk) {
        const float* e = ell + (long long)j * R + r0;
        for (int k0 = 0; k0 < nr; k0 += kFinishLoads) {
          float x[kFinishLoads];
#pragma unroll
          for (int k = 0; k < kFinishLoads; ++k) x[k] = e[min(k0 + k, nr - 1)];
#pragma unroll
          for (int k = 0; k < kFinishLoads; ++k)
            if (k0 + k < nr) sc += fast_exp2(x[k] - lse2[r0 + k0 + k]);
        }
      }
      sc_out[j] = sc;
      if (park && j < ncand) keys[j] = score_key(sc);
    }
  if (!f.topk) return;
  if (tid == 0) f.sel_count[u] = n;
  int32_t* sel_s = DRAFT ? reinterpret_cast<int32_t*>(smem + f.fin_off_sel) : nullptr;
  int32_t* const sel_out = f.sel + (long long)u * f.max_sel;
  if (park) {
    // the keys of every block, parked above, before any read; up to 1024
    // candidates one wave selects (no workgroup barrier in the selection)
    lds_barrier();
    if (ncand <= 64 * 16) {
      if (tid < 64) {
        if (ncand <= 64 * 8)
          topk_wave<8>(KeySrc{keys}, ncand, n, sel_out, f.max_sel, sel_s, topk_lds);
        else
          topk_wave<16>(KeySrc{keys}, ncand, n, sel_out, f.max_sel, sel_s, topk_lds);
      }
      lds_barrier();
    } else {
      topk_select_parked<kFinishThreads>(keys, ncand, n, sel_out, f.max_sel, sel_s, topk_lds);
    }
  } else {
    // the scores of every block, written to memory above, before any read
    __threadfence_block();
    __syncthreads();
    topk_select<kFinishThreads>(sc_out, ncand, n, sel_out, f.max_sel, sel_s, topk_lds);
  }
  if constexpr (DRAFT) {
    // the chained draft of this unit over the selection in LDS (the LDS
    // above is dead: the selection ended with a barrier)
    const int Ld = pd.seq_lens[b];
    const int nseg = unit_valid(pd, Ld, 1)
                         ? draft_list_len_mfma(n, pd.block_size, Ld, window_start(Ld, pd.window))
                         : 0;
    constexpr int A = 2 * kFinishWaves;
    Item dt;
    dt.u = u;
    dt.c = 0;
    dt.chunk = max(A, (nseg + A - 1) / A * A);
    dt.single = 1;
    dt.part_row0 = 0;
    dt.ell_off = 0;
    dt.sel_off = f.fin_off_sel;
    dt.nsel_s = n;
    dt.list_off = 0;
    attn_item<D, 1, kFinishWaves, true, false>(pd, dt, smem);
  }
}

template <int D, int NWR, int NWT>
hipError_t launch_cfg(const FusedParams& f, const AttnParams& pv, const AttnParams& pd,
                      const FusedPlan& pl, hipStream_t s) {
  auto kern = fused_kernel<D, NWR, NWT>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kMaxLds);
  if (attr != hipSuccess) return attr;
  // one workgroup per slot; those past their unit's chunk count exit
  hipLaunchKernelGGL(kern, dim3((unsigned)pl.max_items), dim3(64 * NWR * NWT), pl.lds_bytes, s,
                     f, pv, pd);
  return hipGetLastError();
}

}  // namespace

namespace {

long long lcm_of(long long a, long long b) {
  long long x = a, y = b;
  while (y) {
    const long long t = x % y;
    x = y;
    y = t;
  }
  return a / x * b;
}

// LDS layout and chunking for one choice of token groups.
void plan_with(const FusedPlanIn& in, int nwr, int nwt, size_t lds_cap, FusedPlan& pl) {
  pl.nwr = nwr;
  pl.nwt = nwt;
  const int nwtd = nwr * nwt;
  const int D = in.head_dim;
  const size_t area = std::max(item_lds_bytes(D, nwr, nwt), item_lds_bytes(D, 1, nwtd));
  const size_t sel_bytes = in.chained ? align_up((size_t)in.max_sel * 4, 16) : 0;
  const size_t fixed = align_up(area, 16) + sel_bytes;
  pl.chunk_v = 0;
  pl.maxch_v = 0;
  size_t ell_bytes = 0;
  if (in.nv > 0 && lds_cap > fixed) {
    // whole token-group shares of whole blocks
    const long long align = lcm_of(32LL * nwt, (long long)in.block_size_v * nwt);
    const long long room_blocks = (long long)(lds_cap - fixed) / (4LL * in.rows_v);
    const long long hi = room_blocks * in.block_size_v / align * align;
    // about 512 slots in all, counting every unit as long as the longest
    // (mixed batch of 96 requests, 1K-32K tokens, on MI355X: 0.434 ms with
    // 1024 slots, 0.402 ms with 512, equal within noise at 384 and 768; the
    // LDS room for block masses caps the chunk near 512 there anyway)
    long long want = ((long long)in.nv * in.max_len_v + 511) / 512;
    want = std::max(align, (want + align - 1) / align * align);
    const long long whole = ((long long)in.max_len_v + align - 1) / align * align;
    want = std::min(want, whole);
    if (hi >= align) {
      pl.chunk_v = (int)std::min(want, hi);
      pl.maxch_v = ceil_div(in.max_len_v, pl.chunk_v);
      ell_bytes = align_up((size_t)(pl.chunk_v / in.block_size_v) * in.rows_v * 4, 16);
    }
  }
  // draft chunks: about the token count of a verify chunk, whole tiles of
  // every token group
  pl.chunk_d = 0;
  pl.maxch_d = 0;
  if (in.nd > 0) {
    const int align = 2 * nwtd;
    int want = std::max(64, pl.chunk_v / kSeg);
    want = (want + align - 1) / align * align;
    pl.chunk_d = want;
    pl.maxch_d = std::max(1, ceil_div(std::max(in.list_max_d, 1), pl.chunk_d));
  }
  pl.off_ell = (int)align_up(area, 16);
  pl.off_sel = pl.off_ell + (int)ell_bytes;
  pl.lds_bytes = (size_t)pl.off_sel + sel_bytes;
  pl.max_items = (long long)in.nv * std::max(pl.maxch_v, 1) + (long long)in.nd * pl.maxch_d;
}

}  // namespace

// Chunk sizes, LDS layout and work-list bound of a fused step (host only,
// no device calls: the workspace query and the launch agree).  Two shapes:
//   - every verify unit whole (enough units to fill the GPU a few times
//     over): the widest workgroup, block masses of a whole unit in LDS, one
//     workgroup per compute unit;
//   - units split into chunks: half as many token groups per workgroup and
//     chunks small enough that two workgroups share a compute unit, so one
//     streams while the other starts or finishes an item.
void fused_plan(const FusedPlanIn& in, FusedPlan& pl) {
  const int nwr = in.rows_v > 0 ? ceil_div(in.rows_v, 32) : 1;
  const int nwt = token_groups_for(nwr);
  plan_with(in, nwr, nwt, kMaxLds, pl);
  if (in.nv > 0 && pl.chunk_v > 0 && pl.maxch_v <= 1) return;  // whole units
  if (nwt >= 2) {
    FusedPlan half;
    plan_with(in, nwr, nwt / 2, kMaxLds / 2 - 512, half);
    if (in.nv == 0 || half.chunk_v > 0) pl = half;
  }
}

size_t select_draft_lds(int head_dim, int max_sel, int max_blocks, int32_t& off_sel,
                        int32_t& off_keys) {
  off_sel = (int32_t)align_up(item_lds_bytes(head_dim, 1, kDraftWaves), 16);
  off_keys = off_sel + (int32_t)align_up((size_t)max_sel * 4, 16);
  return (size_t)off_keys + (max_blocks <= kSelectMaxKeys ? (size_t)max_blocks * 4 : 0);
}

hipError_t launch_select_draft(const FusedParams& f, const AttnParams& pv, const AttnParams& pd,
                               int head_dim, hipStream_t s) {
  if (f.nv_units == 0) return hipSuccess;
  int32_t off_sel, off_keys;
  const size_t smem = select_draft_lds(head_dim, f.max_sel, pv.max_blocks, off_sel, off_keys);
  if (smem > kMaxLds || off_sel != f.off_sel || off_keys != f.off_ell) return hipErrorInvalidValue;
  auto go = [&](auto kern) -> hipError_t {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3((unsigned)f.nv_units), dim3(64 * kDraftWaves), smem, s, f, pv,
                       pd);
    return hipGetLastError();
  };
  if (head_dim == 128) return go(select_draft_kernel<128>);
  if (head_dim == 64) return go(select_draft_kernel<64>);
  return hipErrorInvalidValue;
}

size_t select_draft_split_lds(int head_dim, int max_sel, int max_blocks, int32_t& off_sel,
                              int32_t& keys_cap) {
  const size_t area = item_lds_bytes(head_dim, 1, kDraftWaves);
  off_sel = (int32_t)align_up(area, 16);
  const size_t topk = (size_t)(kTopkLdsWords * 4 + 127) / 128 * 128;
  keys_cap = (int32_t)std::min<size_t>((size_t)max_blocks, (area - topk) / 4);
  return (size_t)off_sel + align_up((size_t)max_sel * 4, 16);
}

hipError_t launch_select_draft_split(const FusedParams& f, const AttnParams& pv,
                                     const AttnParams& pd, int head_dim, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)f.nv_units * pd.num_chunks);
  if (grid == 0) return hipSuccess;
  int32_t off_sel, cap;
  const size_t smem = select_draft_split_lds(head_dim, f.max_sel, pv.max_blocks, off_sel, cap);
  if (smem > kMaxLds || off_sel != f.off_sel || cap != f.fin_keys_cap) return hipErrorInvalidValue;
  auto go = [&](auto kern) -> hipError_t {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kDraftWaves), smem, s, f, pv, pd);
    return hipGetLastError();
  };
  if (head_dim == 128) return go(select_draft_split_kernel<128>);
  if (head_dim == 64) return go(select_draft_split_kernel<64>);
  return hipErrorInvalidValue;
}

size_t select_draft_wave_lds(int head_dim, int max_sel, int32_t& off_sel) {
  off_sel = (int32_t)align_up(item_lds_bytes(head_dim, 1, 1), 16);
  return (size_t)off_sel + align_up((size_t)max_sel * 4, 16);
}

hipError_t launch_select_draft_wave(const FusedParams& f, const AttnParams& pv,
                                    const AttnParams& pd, int head_dim, hipStream_t s) {
  if (f.nv_units == 0) return hipSuccess;
  int32_t off_sel;
  const size_t smem = select_draft_wave_lds(head_dim, f.max_sel, off_sel);
  if (smem > kMaxLds || off_sel != f.off_sel || pv.max_blocks > 1024) return hipErrorInvalidValue;
  auto go = [&](auto kern) -> hipError_t {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3((unsigned)f.nv_units), dim3(64), smem, s, f, pv, pd);
    return hipGetLastError();
  };
  const bool small = pv.max_blocks <= 512;
  if (head_dim == 128)
    return small ? go(select_draft_wave_kernel<128, 8>) : go(select_draft_wave_kernel<128, 16>);
  if (head_dim == 64)
    return small ? go(select_draft_wave_kernel<64, 8>) : go(select_draft_wave_kernel<64, 16>);
  return hipErrorInvalidValue;
}

size_t finish_lds(FusedParams& f, int head_dim, int max_blocks, bool draft) {
  const size_t keys_at = (size_t)fin_off_stage_host() + (size_t)kFinishStage * 4;
  size_t cap = (size_t)max_blocks;
  const size_t draft_area = align_up(item_lds_bytes(head_dim, 1, finish_waves<true>()), 16);
  const size_t sel_bytes = draft ? align_up((size_t)f.max_sel * 4, 16) : 0;
  // keys beyond the LDS room are read back from memory by the selection
  if (keys_at + cap * 4 + sel_bytes > kMaxLds) cap = 0;
  f.fin_off_keys = (int32_t)keys_at;
  f.fin_keys_cap = (int32_t)cap;
  f.fin_draft = draft ? 1 : 0;
  const size_t end_keys = align_up(keys_at + cap * 4, 16);
  f.fin_off_sel = (int32_t)(draft ? std::max(draft_area, end_keys) : end_keys);
  return (size_t)f.fin_off_sel + sel_bytes;
}

hipError_t launch_fused_finish(const FusedParams& f, const AttnParams& pv, const AttnParams& pd,
                               int head_dim, size_t lds_bytes, hipStream_t s) {
  if (f.nv_units == 0) return hipSuccess;
  if (lds_bytes > kMaxLds) return hipErrorInvalidValue;
  auto go = [&](auto kern, int waves) -> hipError_t {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3((unsigned)f.nv_units), dim3(64 * waves), lds_bytes, s, f, pv,
                       pd);
    return hipGetLastError();
  };
  const int w = f.fin_draft ? finish_waves<true>() : finish_waves<false>();
  if (head_dim == 128)
    return f.fin_draft ? go(finish_kernel<128, true>, w) : go(finish_kernel<128, false>, w);
  if (head_dim == 64)
    return f.fin_draft ? go(finish_kernel<64, true>, w) : go(finish_kernel<64, false>, w);
  return hipErrorInvalidValue;
}

hipError_t launch_fused(const FusedParams& f, const AttnParams& pv, const AttnParams& pd,
                        const FusedPlan& pl, int head_dim, hipStream_t s) {
  if (pl.max_items == 0) return hipSuccess;
  if (pl.lds_bytes > kMaxLds) return hipErrorInvalidValue;
  const int cfg = pl.nwr * 8 + pl.nwt;
  if (head_dim == 128) {
    switch (cfg) {
      case 1 * 8 + 4: return launch_cfg<128, 1, 4>(f, pv, pd, pl, s);
      case 1 * 8 + 2: return launch_cfg<128, 1, 2>(f, pv, pd, pl, s);
      case 2 * 8 + 2: return launch_cfg<128, 2, 2>(f, pv, pd, pl, s);
      case 2 * 8 + 1: return launch_cfg<128, 2, 1>(f, pv, pd, pl, s);
      case 3 * 8 + 1: return launch_cfg<128, 3, 1>(f, pv, pd, pl, s);
      case 4 * 8 + 1: return launch_cfg<128, 4, 1>(f, pv, pd, pl, s);
    }
  } else if (head_dim == 64) {
    switch (cfg) {
      case 1 * 8 + 4: return launch_cfg<64, 1, 4>(f, pv, pd, pl, s);
      case 1 * 8 + 2: return launch_cfg<64, 1, 2>(f, pv, pd, pl, s);
      case 2 * 8 + 2: return launch_cfg<64, 2, 2>(f, pv, pd, pl, s);
      case 2 * 8 + 1: return launch_cfg<64, 2, 1>(f, pv, pd, pl, s);
      case 3 * 8 + 1: return launch_cfg<64, 3, 1>(f, pv, pd, pl, s);
      case 4 * 8 + 1: return launch_cfg<64, 4, 1>(f, pv, pd, pl, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sss
