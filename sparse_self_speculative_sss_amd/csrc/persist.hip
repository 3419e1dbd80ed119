// Persistent decode step (SparseSpec §4.2: one persistent-style fused kernel
// serves the full attention of the verifying requests and the sparse
// attention of the drafting ones; §4.1 PillarAttn: the verify pass yields
// the block scores whose Top-K is the pattern the following draft steps
// use; SpecAttn, technical framework: the critical KV entries are a
// by-product of verification and the draft loads only those).
//
// One launch runs, for every (request, KV head) unit of a chained step:
// the verify (k+1 positions x G heads over the whole paged cache, block log
// masses kept in LDS), the block scores, the Top-N selection and the draft
// over that selection.  A workgroup is two waves (two token groups that
// split each unit's tokens) and two workgroups share a compute unit.
// Workgroup w loops over the units w, w + grid, w + 2 grid, ... (in the
// XCD-aware order of the one-item kernels).  For each unit it first drafts
// the unit it verified before -- that unit's selection and draft query are
// still in its LDS -- and then verifies the new unit.  The short, latency-bound dependent chain
// of draft tiles therefore runs while the other workgroup on the compute
// unit keeps streaming the cache, instead of in launches after the whole
// verify.  The next unit's Q and page ids are loaded during the selection,
// so they arrive while it runs.  Only the last unit of each workgroup is drafted at the
// end.  No workgroup waits for another: every dependency (block masses ->
// scores -> selection -> draft) stays inside one workgroup.
//
// The verify arithmetic is that of the one-item kernel with two token
// groups (attn_item with Q in registers): the same tile partition, order
// and merge, so outputs, scores and selections are bitwise equal to
// sss_verify_attn + sss_block_topk on the same inputs.  The draft splits
// its list over the two token groups (the stand-alone draft of this many
// units runs one wave per unit), so it agrees with sss_draft_attn up to
// summation order.
#include <algorithm>

#include "attn_item.h"
#include "attn_tile.h"
#include "topk_dev.h"

namespace sss {
namespace {

constexpr int kPersistWaves = 2;  // token groups (waves) per workgroup
constexpr int kPersistThreads = 64 * kPersistWaves;
constexpr int kTopkLdsBytes = (kTopkLdsWords * 4 + 127) / 128 * 128;
constexpr int kWaveTopkKeys = 16;  // keys per lane of the one-wave selection (1024 candidates)

// Everything the persistent step reads: one paged cache serves both halves
// (a chained step drafts the requests it verifies), so the draft half adds
// only its query, outputs, scale and window.  Field names follow
// AttnParams where they mean the same (the segment helpers take either).
struct PersistParams {
  const bf16* k;
  const bf16* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t num_pages, page_size, num_kv_heads, head_dim, max_pages, max_seq_len;
  int32_t block_size, max_blocks, score_row_start;
  // verify: q [B][n_q][Hq][d], o like q, lse [B][n_q][Hq], block_scores
  // [B][Hkv][max_blocks]; rows = n_q * group per unit
  const bf16* q;
  bf16* o;
  float* lse;
  float* block_scores;
  int32_t batch, n_q, num_q_heads, group, rows;
  float scale_log2;
  // selection: budget [B], sel [B][Hkv][max_sel], sel_count [B][Hkv]
  int32_t max_sel, topk_window;
  const int32_t* budget;
  int32_t* sel;
  int32_t* sel_count;
  // draft: q [B][1][Hq][d], o like it, lse [B][1][Hq]
  const bf16* dq;
  bf16* dout;
  float* dlse;
  float dscale_log2;
  int32_t window;
  int32_t units;  // batch x KV heads
  // LDS byte offsets: the unit's block log masses (or the next unit's Q
  // rows parked there), the row log2-LSEs, two flags, the selection the
  // next draft reads and its draft query rows
  int32_t off_ell, off_lse, off_flags, off_sel, off_dq;
};

// Unit run by the i-th workgroup slot: all KV heads of request r on XCD r % 8
// when the batch is a multiple of 8 (slot i runs on XCD i % 8 as long as the
// grid is a multiple of 8), the requests dealt round-robin over the XCDs.
__device__ __forceinline__ int persist_unit(int i, int batch, int H) {
  if ((batch & 7) != 0) return i;
  const int k = i >> 3;
  return ((i & 7) + 8 * (k / H)) * H + k % H;
}

// Combines the two token groups' (m, l, O) of one row tile through LDS at
// `red` (tg 1 writes, tg 0 reads after the barrier; rows < nrows) and
// leaves the result in token group 0's `a`.  Same arithmetic and order as
// attn_item's token-group merge.  All threads call it; it has one (LDS-only)
// barrier.
template <int D>
__device__ __forceinline__ void merge_groups(Acc<D>& a, float* red, int tg, int rl, int hl,
                                             int nrows) {
  float* ml = red + 32 * D;  // [2][32] max, then [2][32] sum
  if (hl == 0) {
    ml[tg * 32 + rl] = a.m;
    ml[2 * 32 + tg * 32 + rl] = a.l;
  }
  if (tg == 1 && rl < nrows) {
    float* dst = red + rl * D;
#pragma unroll
    for (int mt = 0; mt < Geo<D>::MT; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = a.o[mt][4 * q4 + e];
        *reinterpret_cast<f32x4*>(dst + 32 * mt + 8 * q4 + 4 * hl) = v4;
      }
  }
  lds_barrier();
  if (tg == 0) {
    float mg = fmaxf(a.m, ml[32 + rl]);
    const float mu = (mg == neg_inf()) ? 0.f : mg;
    const float a0 = fast_exp2(a.m - mu);
    float lsum = a.l * a0;
#pragma unroll
    for (int mt = 0; mt < Geo<D>::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) a.o[mt][i] *= a0;
    const float ag = fast_exp2(ml[32 + rl] - mu);
    lsum += ag * ml[2 * 32 + 32 + rl];
    if (rl < nrows) {
      const float* src = red + rl * D;
#pragma unroll
      for (int mt = 0; mt < Geo<D>::MT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + 32 * mt + 8 * q4 + 4 * hl);
#pragma unroll
          for (int e = 0; e < 4; ++e) a.o[mt][4 * q4 + e] += ag * v4[e];
        }
    }
    a.m = mg;
    a.l = lsum;
  }
}

// OR of v over the workgroup's two waves through LDS slots `flags` (two
// ints), at an LDS-only barrier.
__device__ __forceinline__ int lds_barrier_or(int v, int* flags) {
  const bool any = __builtin_amdgcn_ballot_w64(v != 0) != 0;
  if ((threadIdx.x & 63) == 0) flags[threadIdx.x >> 6] = any ? 1 : 0;
  lds_barrier();
  return flags[0] | flags[1];
}

// The draft of unit du (request bd, head hd) over its selection sel_s[0, nsel)
// (LDS) plus the window, with the draft query rows staged at dq; the list's
// segments are split over the two token groups (at most 64 each).  On
// return the outputs are written.  When `vnext` is set, the last tile
// prefetches the first verify tile (segments vs0, vs1) into `regs`.
template <int D>
__device__ __forceinline__ void run_draft(const PersistParams& pd, int du, const int32_t* sel_s,
                                          int nsel, const char* dq, char* smem, int* flags,
                                          TileRegs<D, 1>& regs, bool vnext, const Seg& vs0,
                                          const Seg& vs1, const FastDiv& pdiv) {
  typedef Geo<D> G;
  const int lane = threadIdx.x & 63;
  const int tg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, rl = lane & 31;
  const int Gd = pd.group;
  const int bd = du / pd.num_kv_heads, hd = du % pd.num_kv_heads;
  const bf16* __restrict__ kc = pd.k;
  const bf16* __restrict__ vc = pd.v;
  char* const grp = smem + tg * G::GROUP_BYTES;

  const int L = pd.seq_lens[bd];
  const bool valid =
      L >= 1 && L <= pd.max_seq_len && (long long)L <= (long long)pd.max_pages * pd.page_size;
  int bad = valid ? 0 : 1;
  const int ws = valid ? window_start(L, pd.window) : 0;
  const int nseg = valid ? draft_list_len_mfma(nsel, pd.block_size, L, ws) : 0;
  const int per_group = ceil_div(ceil_div(nseg, kPersistWaves), 2) * 2;
  const int g_lo = min(tg * per_group, nseg), g_hi = min(g_lo + per_group, nseg);
  const int n_tiles = ceil_div(min(per_group, nseg), 2);
  const int pos_r = L - 1;
  const float scl = fmaxf(fabsf(pd.dscale_log2), 1e-30f);

  SegLane dl = seg_lane<true>(pd, sel_s, bd, hd, g_lo + lane, g_hi, nsel, L, ws);
  seg_resolve(pd, pdiv, hd, dl, bad);

  Acc<D> a;
  acc_init(a);
  float dummy = 0.f;
  Seg sa = {}, sb = {};
  if (n_tiles > 0) {
    sa = seg_of(pd, dl, dl, false, 0);
    sb = seg_of(pd, dl, dl, false, 1);
    load_tile<D, 1>(regs, kc, vc, sa, sb, lane);
  } else if (vnext) {
    load_tile<D, 1>(regs, kc, vc, vs0, vs1, lane);
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int rel0 = 2 * t;
    const bool live = g_lo + rel0 < g_hi;
    const Seg ca = sa, cb = sb;
    const bool full = seg_full(ca) && seg_full(cb);
    store_tile<D, 1>(regs, grp, lane, ca, cb, full);
    group_sync<1>();
    if (t + 1 < n_tiles) {
      sa = seg_of(pd, dl, dl, false, rel0 + 2);
      sb = seg_of(pd, dl, dl, false, rel0 + 3);
      load_tile<D, 1>(regs, kc, vc, sa, sb, lane);
    } else if (vnext) {
      load_tile<D, 1>(regs, kc, vc, vs0, vs1, lane);
    }
    if (live) {
      const f32x16 sacc = qk_tile_lds<D>(grp, dq, Gd, rl, hl);
      float s[16], pr[16], psum;
      const bool interior = full && cb.t0 + kSeg - 1 <= pos_r;
      const float mx = mask_logits(sacc, s, ca, cb, interior, pos_r, hl);
      softmax_pv<D>(a, s, mx, scl, grp + G::K_BYTES, pr, psum, dummy, rl, hl);
    }
    group_sync<1>();
  }
  a.l += __shfl_xor(a.l, 32);
  bad = lds_barrier_or(bad, flags);  // both groups are done with their tile buffers
  merge_groups<D>(a, reinterpret_cast<float*>(smem), tg, rl, hl, Gd);
  if (tg == 0 && rl < Gd) {
    const long long orow = (long long)bd * pd.num_q_heads + hd * Gd + rl;
    write_row<D>(a, pd.dout, pd.dlse, orow, bad != 0, hl);
  }
  // token group 0 reads the merge scratch (its own tile buffer) before it
  // stores its next tile there: program order within the wave suffices
}

// Segments [g_lo, g_hi) of token group tg for a verify unit of L tokens, and
// the tile count of the loop (group 0's share), as attn_item splits them.
__device__ __forceinline__ void verify_range(int L, int bs, int tg, int& g_lo, int& g_hi,
                                             int& n_tiles) {
  const int seg_hi = ceil_div(L, kSeg);
  const int galign = bs < 2 * kSeg ? 2 : bs / kSeg;
  const int per_group = ceil_div(ceil_div(seg_hi, kPersistWaves), galign) * galign;
  g_lo = min(tg * per_group, seg_hi);
  g_hi = min(g_lo + per_group, seg_hi);
  n_tiles = ceil_div(min(per_group, seg_hi), 2);
}

__device__ __forceinline__ bool verify_unit_ok(const PersistParams& p, int L) {
  return L >= p.n_q && L <= p.max_seq_len && (long long)L <= (long long)p.max_pages * p.page_size;
}

// The first two descriptor batches of unit u's token group (page ids in
// flight).
__device__ __forceinline__ void verify_segs(const PersistParams& p, int u, int tg, SegLane& cur,
                                            SegLane& nxt) {
  const int lane = threadIdx.x & 63;
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
  const int L = p.seq_lens[b];
  int g_lo = 0, g_hi = 0, nt = 0;
  if (verify_unit_ok(p, L)) verify_range(L, p.block_size, tg, g_lo, g_hi, nt);
  cur = seg_lane<false>(p, nullptr, b, h, g_lo + lane, g_hi, 0, L, L);
  nxt = seg_lane<false>(p, nullptr, b, h, g_lo + 64 + lane, g_hi, 0, L, L);
}

// Unit u's Q rows as 16-byte chunks, chunk e = row * CPT + column for
// e = threadIdx.x + 128 j (rows < 32), loaded unconditionally (a row past
// the unit's reads row 0; it is zeroed when parked).  The loads are left in
// flight: park_q_chunks consumes them later.
template <int D, int NQ>
__device__ __forceinline__ void verify_q_chunks(const PersistParams& p, int u, uint4 (&qc)[NQ]) {
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int e = (int)threadIdx.x + kPersistThreads * j;
    const int row0 = e / Geo<D>::CPT, cc = e % Geo<D>::CPT;
    const int row = row0 < p.rows ? row0 : 0;
    const int iq = row / p.group, hq = h * p.group + row % p.group;
    qc[j] = *reinterpret_cast<const uint4*>(p.q + (((long long)b * p.n_q + iq) * p.num_q_heads + hq) * D +
                                            8 * cc);
  }
}

// The chunks of verify_q_chunks into LDS at qpark (row stride K_STRIDE):
// rows past the unit's zeroed, a negative scale folded in (exact sign flip).
template <int D, int NQ>
__device__ __forceinline__ void park_q_chunks(const PersistParams& p, const uint4 (&qc)[NQ],
                                              char* qpark) {
  const uint32_t flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int e = (int)threadIdx.x + kPersistThreads * j;
    const int row = e / Geo<D>::CPT, cc = e % Geo<D>::CPT;
    if (row < 32) {
      uint4 v = qc[j];
      v.x ^= flip;
      v.y ^= flip;
      v.z ^= flip;
      v.w ^= flip;
      if (row >= p.rows) v = uint4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4*>(qpark + row * Geo<D>::K_STRIDE + 16 * cc) = v;
    }
  }
}

// Block scores of a unit from its block log masses: sc_j = sum over rows
// r0 <= r < R of 2^(ell[j][r] - lse2[r]), rows summed in order (as attn_item
// does, so the scores are bitwise equal); written to `scores` (0 past nblk,
// NaN if bad) and, for j < ncand, parked as Top-N keys.  Rows are read as
// float4 when they allow it, all of a block's at once.
__device__ __forceinline__ void unit_scores(const float* ell, const float* lse2, int R, int r0,
                                            int nblk, int max_blocks, bool bad, int ncand,
                                            float* scores, uint32_t* keys) {
  const int tid = threadIdx.x;
  if ((R & 3) == 0 && (r0 & 3) == 0 && R - r0 <= 32) {
    const int nq4 = (R - r0) >> 2;
    for (int j = tid; j < max_blocks; j += kPersistThreads) {
      float sc = 0.f;
      if (j < nblk) {
        const f32x4* e = reinterpret_cast<const f32x4*>(ell + (long long)j * R + r0);
        f32x4 x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q < nq4) x[q] = e[q];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q < nq4) {
            const float* l2 = lse2 + r0 + 4 * q;
            sc += fast_exp2(x[q][0] - l2[0]);
            sc += fast_exp2(x[q][1] - l2[1]);
            sc += fast_exp2(x[q][2] - l2[2]);
            sc += fast_exp2(x[q][3] - l2[3]);
          }
      }
      sc = bad ? qnan() : sc;
      scores[j] = sc;
      if (j < ncand) keys[j] = score_key(sc);
    }
  } else {
    for (int j = tid; j < max_blocks; j += kPersistThreads) {
      float sc = 0.f;
      if (j < nblk) {
        const float* e = ell + (long long)j * R;
        for (int rr = r0; rr < R; ++rr) sc += fast_exp2(e[rr] - lse2[rr]);
      }
      sc = bad ? qnan() : sc;
      scores[j] = sc;
      if (j < ncand) keys[j] = score_key(sc);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(kPersistThreads, 1) persist_step_kernel(PersistParams p) {
  typedef Geo<D> G;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int tg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, rl = lane & 31;
  const int r = rl;
  const bool row_ok = r < p.rows;
  char* const grp = smem + tg * G::GROUP_BYTES;
  int* const flags = reinterpret_cast<int*>(smem + p.off_flags);
  const int grid = gridDim.x;
  const int nmine = p.units > (int)blockIdx.x ? (p.units - (int)blockIdx.x + grid - 1) / grid : 0;
  // the next unit's Q rows: loaded into qpre before an epilogue, parked in
  // the dead block-mass area at its end, read into the Q^T operand after
  // the next draft (no Q registers are held across the draft's tiles)
  constexpr int kQChunks = (32 * G::CPT + kPersistThreads - 1) / kPersistThreads;
  uint4 qpre[kQChunks];
  bf16x8 qreg[G::KS];
  SegLane vcur = {}, vnxt = {};
  const FastDiv pdiv(p.page_size);

  int du = -1, dn = 0;  // the unit verified last (its draft is pending), its selection's length
  if (nmine > 0) {
    const int u0 = persist_unit(blockIdx.x, p.batch, p.num_kv_heads);
    const int b0 = u0 / p.num_kv_heads, h0 = u0 % p.num_kv_heads;
    const bf16* row = nullptr;
    if (row_ok)
      row = p.q + (((long long)b0 * p.n_q + r / p.group) * p.num_q_heads + h0 * p.group + r % p.group) * D;
    load_qreg<D>(qreg, row, p.scale_log2 < 0.f);
    verify_segs(p, u0, tg, vcur, vnxt);
  }

  for (int k = 0; k < nmine; ++k) {
    const int u = persist_unit(blockIdx.x + k * grid, p.batch, p.num_kv_heads);
    const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
    const int L = p.seq_lens[b];
    const bool unit_ok = verify_unit_ok(p, L);
    const int budget = p.budget[b];
    int g_lo = 0, g_hi = 0, n_tiles = 0;
    if (unit_ok) verify_range(L, p.block_size, tg, g_lo, g_hi, n_tiles);
    int bad = unit_ok ? 0 : 1;
    // the first two descriptor batches (page ids fetched before the last
    // epilogue): cache rows
    seg_resolve(p, pdiv, h, vcur, bad);
    seg_resolve(p, pdiv, h, vnxt, bad);
    Seg sa = {}, sb = {};
    if (n_tiles > 0) {
      sa = seg_of(p, vcur, vnxt, false, 0);
      sb = seg_of(p, vcur, vnxt, false, 1);
    }
    TileRegs<D, 1> regs;
    if (du >= 0) {
      // the last unit's draft (handing its last tile's prefetch over to this
      // verify keeps the verify's first segments live through the draft, and
      // the two then overflow the register file)
      const Seg z = {};
      run_draft<D>(p, du, reinterpret_cast<const int32_t*>(smem + p.off_sel), dn, smem + p.off_dq,
                   smem, flags, regs, false, z, z, pdiv);
    }
    if (n_tiles > 0) {
      load_tile<D, 1>(regs, p.k, p.v, sa, sb, lane);
    }
    if (k > 0) {
      // this unit's Q operand from where the last epilogue parked it; every
      // wave holds it before any block mass overwrites it
      const char* qpark = smem + p.off_ell;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        const bf16x8 z = {};
        qreg[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qpark + rl * G::K_STRIDE + 32 * ks + 16 * hl)
                          : z;
      }
      lds_barrier();
    }

    // ---- verify of unit u: this token group's tiles ----
    {
      float* const ell_s = reinterpret_cast<float*>(smem + p.off_ell);
      const FastDiv bdiv(p.block_size);
      const int bs = p.block_size;
      const int R = p.rows;
      const float scl = fmaxf(fabsf(p.scale_log2), 1e-30f);
      const int pos_r = L - p.n_q + (row_ok ? r / p.group : 0);
      const int pos_min = L - p.n_q;
      Acc<D> a;
      acc_init(a);
      float blk_run = 0.f;
      int cur_batch = 0;
      for (int t = 0; t < n_tiles; ++t) {
        const int rel0 = 2 * t;
        const bool tile_live = g_lo + rel0 < g_hi;
        const Seg ca = sa, cb = sb;
        const bool full = seg_full(ca) && seg_full(cb);
        store_tile<D, 1>(regs, grp, lane, ca, cb, full);
        if (rel0 > 0 && (rel0 & 63) == 0) {
          vcur = vnxt;
          ++cur_batch;
          vnxt = seg_lane<false>(p, nullptr, b, h, g_lo + 64 * (cur_batch + 1) + lane, g_hi, 0, L, L);
        }
        if ((rel0 & 63) == 32) seg_resolve(p, pdiv, h, vnxt, bad);
        group_sync<1>();
        if (t + 1 < n_tiles) {
          const int ra = rel0 + 2, rb = ra + 1;
          sa = seg_of(p, vcur, vnxt, (ra >> 6) != cur_batch, ra & 63);
          sb = seg_of(p, vcur, vnxt, (rb >> 6) != cur_batch, rb & 63);
          load_tile<D, 1>(regs, p.k, p.v, sa, sb, lane);
        }
        if (tile_live) {
          const f32x16 sacc = qk_tile<D>(grp, qreg, rl, hl);
          float s[16], pr[16], psum;
          const bool interior = full && cb.t0 + kSeg - 1 <= pos_min;
          const float mx = mask_logits(sacc, s, ca, cb, interior, pos_r, hl);
          const float m_use = softmax_pv<D>(a, s, mx, scl, grp + G::K_BYTES, pr, psum, blk_run, rl, hl);
          // per-block log mass of this row, frame m_use
          if (bs == kSeg) {
            float x = 0.f, y = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) x += pr[i];
#pragma unroll
            for (int i = 8; i < 16; ++i) y += pr[i];
            x += __shfl_xor(x, 32);
            y += __shfl_xor(y, 32);
            const Seg& mine = hl ? cb : ca;
            if (row_ok && mine.lo < mine.hi)
              ell_s[(mine.t0 / kSeg) * R + r] = m_use + fast_log2(hl ? y : x);
          } else {
            blk_run += psum;
            const bool last = (bdiv.mod(ca.t0 + 2 * kSeg) == 0) || (g_lo + rel0 + 2 >= g_hi);
            if (last) {
              const float tot = blk_run + __shfl_xor(blk_run, 32);
              if (row_ok && hl == 0) ell_s[bdiv.div(ca.t0) * R + r] = m_use + fast_log2(tot);
              blk_run = 0.f;
            }
          }
        }
        group_sync<1>();
      }

      const bool more = k + 1 < nmine;

      // ---- epilogue: token groups merged, outputs, block scores, selection
      // (every exchange through LDS, so the barriers wait for no memory
      // operation in flight) ----
      float* const lse2s = reinterpret_cast<float*>(smem + p.off_lse);
      a.l += __shfl_xor(a.l, 32);
      bad = lds_barrier_or(bad, flags);
      merge_groups<D>(a, reinterpret_cast<float*>(smem), tg, rl, hl, 32);
      if (tg == 0 && row_ok) {
        const long long orow =
            ((long long)b * p.n_q + r / p.group) * p.num_q_heads + h * p.group + r % p.group;
        const float lse2 = write_row<D>(a, p.o, p.lse, orow, bad != 0, hl);
        if (hl == 0) lse2s[r] = lse2;
      }
      lds_barrier();
      uint32_t* const keys = reinterpret_cast<uint32_t*>(smem);
      int ncand, n;
      topk_bounds(L, bs, p.topk_window, p.max_blocks, budget, p.max_sel, ncand, n);
      unit_scores(ell_s, lse2s, R, p.score_row_start * p.group, unit_ok ? ceil_div(L, bs) : 0,
                  p.max_blocks, bad != 0, ncand, p.block_scores + (long long)u * p.max_blocks, keys);
      if (tid == 0) p.sel_count[u] = n;
      lds_barrier();
      // in flight during the selection: the next unit's Q rows and page ids,
      // this unit's draft query rows (consumed after it, so no load is waited
      // for inside the latency-bound phases)
      if (more) {
        const int un = persist_unit(blockIdx.x + (k + 1) * grid, p.batch, p.num_kv_heads);
        verify_q_chunks<D>(p, un, qpre);
        verify_segs(p, un, tg, vcur, vnxt);
      }
      const int Gd = p.group;
      const bool dq_mine = tid < Gd * G::CPT;  // group <= 32: at most 512 chunks
      uint4 dqc[kQChunks];
#pragma unroll
      for (int j = 0; j < kQChunks; ++j) {
        const int e = min(tid + kPersistThreads * j, Gd * G::CPT - 1);
        dqc[j] = *reinterpret_cast<const uint4*>(
            p.dq + ((long long)b * p.num_q_heads + h * Gd + e / G::CPT) * D + 8 * (e % G::CPT));
      }
      // token group 0 selects (one-wave radix select) while group 1 parks
      // the next Q rows; larger candidate sets take the workgroup routine
      int* const topk_lds = reinterpret_cast<int*>(smem + 2 * G::GROUP_BYTES - kTopkLdsBytes);
      int32_t* const sel_out = p.sel + (long long)u * p.max_sel;
      int32_t* const sel_s = reinterpret_cast<int32_t*>(smem + p.off_sel);
      if (p.max_blocks <= 64 * kWaveTopkKeys) {
        if (tg == 0) topk_wave<kWaveTopkKeys>(KeySrc{keys}, ncand, n, sel_out, p.max_sel, sel_s, topk_lds);
      } else {
        topk_select_parked<kPersistThreads>(keys, ncand, n, sel_out, p.max_sel, sel_s, topk_lds);
      }
      // the block masses are dead: park the next unit's Q rows there; the
      // draft query rows of this unit into its slot
      if (more) park_q_chunks<D>(p, qpre, smem + p.off_ell);
      if (dq_mine) {
        const uint32_t flip = p.dscale_log2 < 0.f ? 0x80008000u : 0u;
        char* const dq = smem + p.off_dq;
#pragma unroll
        for (int j = 0; j < kQChunks; ++j) {
          const int e = tid + kPersistThreads * j;
          if (e < Gd * G::CPT) {
            uint4 v = dqc[j];
            v.x ^= flip;
            v.y ^= flip;
            v.z ^= flip;
            v.w ^= flip;
            *reinterpret_cast<uint4*>(dq + (e / G::CPT) * G::K_STRIDE + 16 * (e % G::CPT)) = v;
          }
        }
      }
      lds_barrier();
      du = u;
      dn = n;
    }
  }

  // the last unit's draft
  if (du >= 0) {
    TileRegs<D, 1> regs;
    const Seg z = {};
    run_draft<D>(p, du, reinterpret_cast<const int32_t*>(smem + p.off_sel), dn, smem + p.off_dq,
                 smem, flags, regs, false, z, z, pdiv);
  }
}

}  // namespace

// LDS layout of the persistent step workgroup: two tile buffers (also the
// token-group merge scratch, the Top-N keys and the selection scratch), the
// unit's block log masses (or the next unit's Q rows), row log2-LSEs, two
// flags, the selection the next draft reads and its draft query rows.
// Returns the bytes (0 when the keys and scratch do not fit in the tiles).
size_t persist_lds(int head_dim, int rows, int group, int max_blocks, int max_sel,
                   int32_t* offs /* [5] */) {
  const size_t group_bytes = (size_t)32 * (head_dim * 2 + 16) + (size_t)head_dim * 64;
  const size_t tiles = 2 * group_bytes;
  if ((size_t)max_blocks * 4 + kTopkLdsBytes > tiles) return 0;
  size_t off = tiles;
  auto take = [&](size_t n) {
    const int32_t at = (int32_t)off;
    off += align_up(n, 16);
    return at;
  };
  offs[0] = take(std::max((size_t)max_blocks * rows * 4, (size_t)32 * (head_dim * 2 + 16)));
  offs[1] = take((size_t)rows * 4);
  offs[2] = take(2 * 4);
  offs[3] = take((size_t)max_sel * 4);
  offs[4] = take((size_t)group * (head_dim * 2 + 16));
  return off;
}

hipError_t launch_persist_step(const AttnParams& pv, const AttnParams& pd, int max_sel,
                               int topk_window, const int32_t* budget, int32_t* sel,
                               int32_t* sel_count, int grid, hipStream_t s) {
  PersistParams p = {};
  p.k = reinterpret_cast<const bf16*>(pv.k);
  p.v = reinterpret_cast<const bf16*>(pv.v);
  p.page_table = pv.page_table;
  p.seq_lens = pv.seq_lens;
  p.num_pages = pv.num_pages;
  p.page_size = pv.page_size;
  p.num_kv_heads = pv.num_kv_heads;
  p.head_dim = pv.head_dim;
  p.max_pages = pv.max_pages;
  p.max_seq_len = pv.max_seq_len;
  p.block_size = pv.block_size;
  p.max_blocks = pv.max_blocks;
  p.score_row_start = pv.score_row_start;
  p.q = reinterpret_cast<const bf16*>(pv.q);
  p.o = reinterpret_cast<bf16*>(pv.o);
  p.lse = pv.lse;
  p.block_scores = pv.block_scores;
  p.batch = pv.batch;
  p.n_q = pv.n_q;
  p.num_q_heads = pv.num_q_heads;
  p.group = pv.group;
  p.rows = pv.rows;
  p.scale_log2 = pv.scale_log2;
  p.max_sel = max_sel;
  p.topk_window = topk_window;
  p.budget = budget;
  p.sel = sel;
  p.sel_count = sel_count;
  p.dq = reinterpret_cast<const bf16*>(pd.q);
  p.dout = reinterpret_cast<bf16*>(pd.o);
  p.dlse = pd.lse;
  p.dscale_log2 = pd.scale_log2;
  p.window = pd.window;
  p.units = pv.batch * pv.num_kv_heads;
  if (pd.rows != pv.group || pd.num_q_heads != pv.num_q_heads || pd.block_size != pv.block_size)
    return hipErrorInvalidValue;
  int32_t offs[5];
  const size_t lds = persist_lds(pv.head_dim, pv.rows, pv.group, pv.max_blocks, max_sel, offs);
  p.off_ell = offs[0];
  p.off_lse = offs[1];
  p.off_flags = offs[2];
  p.off_sel = offs[3];
  p.off_dq = offs[4];
  if (lds == 0 || lds > kMaxLds) return hipErrorInvalidValue;
  if (p.units <= 0) return hipSuccess;
  if (grid > p.units) grid = p.units;
  auto go = [&](auto kern) -> hipError_t {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kPersistThreads), lds, s, p);
    return hipGetLastError();
  };
  if (pv.head_dim == 128) return go(persist_step_kernel<128>);
  if (pv.head_dim == 64) return go(persist_step_kernel<64>);
  return hipErrorInvalidValue;
}

}  // namespace sss
