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

// Finishes the split verify units of a fused step, one workgroup per unit:
// merges the chunk partials into o / lse, turns the block log masses into
// block scores, then selects (the one-launch merge and selection kernels
// spread this over more launches; here a unit's partials are small).
constexpr int kFinishThreads = 1024;
constexpr int kFinishWeights = 8192;

__global__ void __launch_bounds__(kFinishThreads) finish_kernel(FusedParams f, AttnParams p) {
  __shared__ float lse2[128];
  __shared__ float wts[kFinishWeights];
  __shared__ int topk_lds[kTopkLdsWords];
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
  const int L = p.seq_lens[b];
  // units that fit in one chunk, and invalid ones, were finished in place
  if (!unit_valid(p, L, p.n_q) || L <= f.chunk_v) return;
  const int R = p.rows, D = p.head_dim, G = p.group;
  const int S = ceil_div(L, f.chunk_v);
  const float* lp = p.lse_part + (long long)u * f.maxch_v * R;
  const float* op = p.o_part + (long long)u * f.maxch_v * R * D;
  auto out_row = [&](int r) -> long long {
    return ((long long)b * p.n_q + r / G) * p.num_q_heads + h * G + r % G;
  };
  for (int r = tid; r < R; r += kFinishThreads) {
    float m = neg_inf();
    bool nan = false;
    for (int s = 0; s < S; ++s) {
      const float x = lp[s * R + r];
      nan |= (x != x);
      m = fmaxf(m, x);
    }
    float sum = 0.f;
    if (!nan && m != neg_inf())
      for (int s = 0; s < S; ++s) sum += fast_exp2(lp[s * R + r] - m);
    const float tot = nan ? qnan() : (m == neg_inf() ? neg_inf() : m + fast_log2(sum));
    lse2[r] = tot;
    p.lse[out_row(r)] = tot * kLn2;
  }
  __syncthreads();
  const bool wfit = S * R <= kFinishWeights;
  if (wfit)
    for (int i = tid; i < S * R; i += kFinishThreads) {
      const float tot = lse2[i % R];
      wts[i] = (tot == neg_inf() || tot != tot) ? 0.f : fast_exp2(lp[i] - tot);
    }
  __syncthreads();
  bf16* o = reinterpret_cast<bf16*>(p.o);
  for (int idx = tid; idx < R * D; idx += kFinishThreads) {
    const int r = idx / D, d = idx % D;
    const float tot = lse2[r];
    float acc = 0.f;
    if (tot != neg_inf())
      for (int s = 0; s < S; ++s) {
        const float w = wfit ? wts[s * R + r] : fast_exp2(lp[s * R + r] - tot);
        acc += w * op[((long long)s * R + r) * D + d];
      }
    if (tot != tot) acc = qnan();
    o[out_row(r) * D + d] = from_f32<bf16>(acc);
  }
  const int nblk = ceil_div(L, p.block_size);
  const float* ell = p.ell + (long long)u * p.max_blocks * R;
  const int r0 = p.score_row_start * G;
  float* sc_out = p.block_scores + (long long)u * p.max_blocks;
  // rows in groups of 4 with 16-byte loads when the row count allows
  const bool vec = (R % 4) == 0 && (r0 % 4) == 0;
  for (int j = tid; j < p.max_blocks; j += kFinishThreads) {
    float sc = 0.f;
    if (j < nblk) {
      const float* e = ell + (long long)j * R;
      if (vec) {
        for (int r = r0; r < R; r += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(e + r);
          sc += fast_exp2(x[0] - lse2[r]) + fast_exp2(x[1] - lse2[r + 1]) +
                fast_exp2(x[2] - lse2[r + 2]) + fast_exp2(x[3] - lse2[r + 3]);
        }
      } else {
        for (int r = r0; r < R; ++r) sc += fast_exp2(e[r] - lse2[r]);
      }
    }
    sc_out[j] = sc;
  }
  if (!f.topk) return;
  __threadfence_block();
  __syncthreads();
  int ncand, n;
  topk_bounds(L, p.block_size, f.topk_window, p.max_blocks, f.budget[b], f.max_sel, ncand, n);
  if (tid == 0) f.sel_count[u] = n;
  // the merge weights are dead: their LDS parks the selection's keys
  topk_select<kFinishThreads>(sc_out, ncand, n, f.sel + (long long)u * f.max_sel, f.max_sel,
                              nullptr, topk_lds, reinterpret_cast<uint32_t*>(wts),
                              kFinishWeights);
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

hipError_t launch_fused_finish(const FusedParams& f, const AttnParams& pv, hipStream_t s) {
  if (f.nv_units == 0) return hipSuccess;
  hipLaunchKernelGGL(finish_kernel, dim3((unsigned)f.nv_units), dim3(kFinishThreads), 0, s, f, pv);
  return hipGetLastError();
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
