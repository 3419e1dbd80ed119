// Matrix-core (MFMA) paged attention for gfx950, as a workgroup-level device
// routine: one work item = one chunk of one (request, KV head) unit, verify
// (causal, k+1 query positions x GQA group rows, per-block probability mass)
// or sparse draft (one query over selected blocks plus the recent window).
// The one-item-per-workgroup kernels (attn_mfma.hip) and the persistent
// fused step kernel (fused.hip) both run items through attn_item().
//
// Work decomposition.  A unit is one (request, KV head).  Its rows are the
// n_q * G query rows sharing that KV head, padded to 32-row tiles.  A
// workgroup holds NWT token groups of NWR waves; wave (tg, rt) owns row tile
// rt of token group tg.  The waves of a token group load each 32-token KV
// tile from HBM once (16-byte coalesced loads of contiguous page runs) into
// LDS and all of them read it, so K and V are fetched once for every row of
// the unit.  Token groups cover contiguous sub-ranges of the chunk and are
// merged through LDS at the end.
//
// Per tile, with 32x32x16 bf16 MFMAs:
//   S^T = K * Q^T   (M = 32 tokens, N = 32 rows, K = head_dim)
//   O^T += V^T * P^T (M = 32 head dims, N = 32 rows, K = 16 tokens)
// Both accumulators put row (lane % 32) in lane, so the online-softmax
// rescale is lane-local and a row is shared by the lane pair (l, l ^ 32).
// V is stored transposed in LDS in the token order that makes P^T the
// lane's own softmax values (no shuffles between the two MFMAs).
//
// The routine follows SparseSpec §4.1 (PillarAttn): the verify pass keeps,
// next to the running LSE, the log of each KV block's probability mass
// (ell, log2 domain, in the frame of the row max at that time), so the exact
// per-block scores can be rematerialised once the row's final LSE is known.
#pragma once

#include "sss_common.h"
#include "topk_dev.h"

namespace sss {

template <int D>
struct Geo {
  static constexpr int KS = D / 16;             // QK MFMA k-steps
  static constexpr int MT = D / 32;             // PV M-tiles
  static constexpr int CPT = D / 8;             // 16-byte chunks per token row
  static constexpr int K_STRIDE = D * 2 + 16;   // LDS bytes per K row (padded)
  static constexpr int K_BYTES = 32 * K_STRIDE;
  static constexpr int V_BYTES = D * 64;        // V^T: D rows of 32 positions
  static constexpr int GROUP_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_CHUNKS = 32 * CPT;
  static constexpr int V_UNITS = 8 * CPT;       // 4 positions x one 16-byte chunk
  static constexpr int Q_BYTES = 32 * K_STRIDE;  // Q rows of one row tile (padded)
  static constexpr int LSE_BYTES = 128 * 4;      // final row log2-LSEs (block scores)
};

// Token groups per workgroup for a given number of 32-row tiles.
__host__ __device__ constexpr int token_groups_for(int nwr) { return nwr == 1 ? 4 : (nwr == 2 ? 2 : 1); }

// K/V tile buffers in LDS: one per token group, or two (alternating tiles)
// for a single token group of three or four row waves, so that those waves
// meet at one barrier per tile instead of two.
__host__ __device__ constexpr int tile_buffers(int nwr, int nwt) {
  return (nwt == 1 && nwr >= 3) ? 2 : nwt;
}

// LDS bytes attn_item<D, NWR, NWT, *> uses from the start of its LDS area:
// K/V tiles (or the token-group merge scratch, which reuses them), Q tiles
// (none when the Q operand is held in registers: QREG), row LSEs.
__host__ __device__ constexpr size_t item_lds_bytes(int D, int nwr, int nwt, bool qreg = false) {
  return (size_t)tile_buffers(nwr, nwt) * ((size_t)32 * (D * 2 + 16) + (size_t)D * 64) +
         (qreg ? (size_t)0 : (size_t)nwr * 32 * (D * 2 + 16)) + 128 * 4;
}

// The dispatcher deals workgroups round-robin over the eight XCDs
// (workgroup b runs on XCD b % 8), so in unit order XCD x runs KV head
// x mod Hkv of every request, and each request's page-table row is fetched
// into every XCD's L2.  For unsplit units of a batch that is a multiple of
// 8, workgroup b instead runs request 8 floor(k / Hkv) + b % 8, head
// k % Hkv, with k = floor(b / 8): all heads of request r on XCD r % 8, the
// requests still dealt round-robin over the XCDs, so that a batch of mixed
// lengths stays balanced across them (contiguous blocks of requests per XCD
// made a mixed batch of 96 requests 29% slower).  Batch 128 x 8K on
// MI355X: verify 0.675 -> 0.666 ms, draft 48 -> 47 us, step 0.745 -> 0.738
// ms; 256 x 4K verify 0.694 -> 0.689 ms; bitwise-identical outputs.  Split
// grids keep unit order.
__device__ __forceinline__ unsigned xcd_item(unsigned b, const AttnParams& p) {
  if (p.num_chunks != 1 || (p.batch & 7) != 0) return b;
  const unsigned H = (unsigned)p.num_kv_heads, k = b >> 3;
  return ((b & 7u) + 8u * (k / H)) * H + k % H;
}

// What attn_item left behind.
enum ItemStatus { kItemNone = 0, kItemFinal = 1, kItemPartial = 2 };

// One work item: chunk c of unit u.
struct Item {
  int u, c;
  int chunk;             // tokens (verify) or list entries (draft) per chunk
  int single;            // every unit is one chunk (outputs are final)
  long long part_row0;   // partial-output row of chunk 0, row 0 of the unit
  int ell_off;           // verify: LDS byte offset of the chunk's block log
                         // masses (-1: stored to p.ell as blocks complete)
  int sel_off;           // draft: LDS byte offset of the unit's selection
                         // (-1: read from p.sel / p.sel_count)
  int nsel_s;            // the selection's length when sel_off >= 0
  int list_off;          // single tokens: LDS byte offset of a draft chunk's
                         // token list (cache row per entry, -1 = none), or
                         // of a verify's logit staging slots (4 KiB per
                         // wave; used with several row tiles)
};

// Orders LDS writes before reads among the waves sharing a tile: a plain
// wave-local ordering point when a token group is a single wave (LDS
// operations of one wave complete in issue order), a workgroup barrier
// otherwise.
template <int NWR>
__device__ __forceinline__ void group_sync() {
  if (NWR == 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// Division by a runtime divisor 1 <= d <= 2^31 of a dividend 0 <= x < 2^31
// as a multiply-high, add and shift (Granlund and Montgomery's round-up
// method with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1; the
// sum cannot overflow for x < 2^31).  The tile loop divides token positions
// by the page and block sizes; a plain integer division costs ~25 scalar
// instructions each time.
struct FastDiv {
  uint32_t d, m;
  int l;
  __device__ explicit FastDiv(int divisor) {
    d = (uint32_t)divisor;
    l = d > 1u ? 32 - __builtin_clz(d - 1u) : 0;
    m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1ull);
  }
  __device__ __forceinline__ int div(int x) const {
    return (int)((__umulhi((uint32_t)x, m) + (uint32_t)x) >> l);
  }
  __device__ __forceinline__ int mod(int x) const { return x - div(x) * (int)d; }
};

struct Seg {
  long long base;  // element offset of token t0 of this (page, head) run
  int t0, lo, hi;  // 16-aligned start; valid tokens are [lo, hi)
  uint32_t pm;     // sparse verify: query positions whose layout holds it
};

// Descriptor of one 16-token segment, held by one lane: 64 consecutive
// segments of a token group live in one register set, and each tile reads
// its two descriptors with readlane, so page-table lookups are issued a whole
// batch ahead instead of once per tile.  Once the batch's page ids have
// arrived, seg_resolve turns each into the cache row of the segment's first
// token, in vector code once per batch: the tile loop then only reads the
// row (turning a page id into an address took ~25 scalar instructions per
// segment in every tile of every wave).
struct SegLane {
  int t0;
  int lohi;     // (lo - t0) | ((hi - t0) << 8)
  int pg;       // page id as loaded from the page table
  uint32_t pm;  // sparse verify: query positions whose layout holds it
  int row;      // after seg_resolve: cache row (page, head, slot) of token t0
};

// Segment k of a verify unit (16 tokens starting at 16k), or entry k of a
// list (LIST: a draft unit's selection, or the union of a sparse verify
// unit's layouts held in LDS with the query positions of each block in
// pm_s): first the segments of the listed blocks (only their tokens before
// the window start), then the window, which every position sees.
// The page id is loaded for every lane (the table index is clamped into the
// request's row) and only checked when a tile reads the descriptor, so the
// load is never waited for here.
template <bool LIST, class P>
__device__ __forceinline__ SegLane seg_lane(const P& p, const int32_t* sel_s, int b,
                                            int h, int k, int k_end, int nsel, int L, int ws,
                                            const uint32_t* pm_s = nullptr) {
  int t0 = 0, lo = 0, hi = 0;
  uint32_t pm = 0xffffffffu;
  if (k < k_end) {
    if (!LIST) {
      t0 = k * kSeg;
      lo = t0;
      hi = min(t0 + kSeg, L);
    } else {
      const int spb = p.block_size / kSeg;
      if (k < nsel * spb) {
        const int j = sel_s ? sel_s[k / spb]
                            : p.sel[((long long)b * p.num_kv_heads + h) * p.max_sel + k / spb];
        if (pm_s) pm = pm_s[k / spb];
        if (j >= 0 && j < ceil_div(ws, p.block_size)) {
          t0 = j * p.block_size + kSeg * (k % spb);
          lo = t0;
          hi = min(t0 + kSeg, ws);
        }
      } else {
        t0 = (ws / kSeg) * kSeg + kSeg * (k - nsel * spb);
        lo = max(t0, ws);
        hi = min(t0 + kSeg, L);
      }
    }
  }
  SegLane d;
  d.t0 = t0;
  d.lohi = lo < hi ? ((lo - t0) | ((hi - t0) << 8)) : 0;
  d.pg = p.page_table[(long long)b * p.max_pages + min(t0 / p.page_size, p.max_pages - 1)];
  d.pm = pm;
  return d;
}

// The cache rows of a batch of descriptors (this lane's segment), once its
// page ids have arrived.  An empty segment reads page 0; a page id outside
// [0, num_pages) also reads page 0 and sets this lane's `bad` (the unit's
// outputs become NaN once the flags are combined).
template <class P>
__device__ __forceinline__ void seg_resolve(const P& p, const FastDiv& pdiv, int h,
                                            SegLane& d, int& bad) {
  int pg = d.pg;
  if (d.lohi == 0) {
    pg = 0;
  } else if (pg < 0 || pg >= p.num_pages) {
    bad = 1;
    pg = 0;
  }
  // rows of the pool number < 2^31 (checked on the host)
  d.row = (pg * p.num_kv_heads + h) * p.page_size + pdiv.mod(d.t0);
}

// Descriptor idx of the current (or next) batch as uniform values, from
// resolved batches.  PM: also read the position mask.
template <bool PM = false, class P>
__device__ __forceinline__ Seg seg_of(const P& p, const SegLane& cur, const SegLane& nxt,
                                      bool use_nxt, int idx) {
  Seg s;
  s.pm = 0xffffffffu;
  if (PM) {
    const uint32_t pmc = __builtin_amdgcn_readlane(cur.pm, idx);
    const uint32_t pmn = __builtin_amdgcn_readlane(nxt.pm, idx);
    s.pm = use_nxt ? pmn : pmc;
  }
  const int t0c = __builtin_amdgcn_readlane(cur.t0, idx);
  const int t0n = __builtin_amdgcn_readlane(nxt.t0, idx);
  const int lhc = __builtin_amdgcn_readlane(cur.lohi, idx);
  const int lhn = __builtin_amdgcn_readlane(nxt.lohi, idx);
  const int rowc = __builtin_amdgcn_readlane(cur.row, idx);
  const int rown = __builtin_amdgcn_readlane(nxt.row, idx);
  s.t0 = use_nxt ? t0n : t0c;
  const int lh = use_nxt ? lhn : lhc;
  s.lo = s.t0 + (lh & 255);
  s.hi = s.t0 + (lh >> 8);
  s.base = (long long)(use_nxt ? rown : rowc) * p.head_dim;
  return s;
}

__device__ __forceinline__ bool seg_full(const Seg& s) { return s.lo == s.t0 && s.hi == s.t0 + kSeg; }

// Swizzle of the 16-byte quads of a V^T row and permutation of the rows,
// chosen so that the transposing writes (16 lanes: 8 positions x 2 rows
// eight apart) and the MFMA operand reads (8 lanes: 8 consecutive rows)
// both spread over the LDS banks.
__device__ __forceinline__ int vq_swz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }
__device__ __forceinline__ int vrow(int d) { return d ^ ((d >> 3) & 1); }

// Position p (0..31) of the V^T tile holds tile token tau(p): within each 16,
// positions 4..7 and 8..11 are exchanged.  This is the K-order in which a
// lane's own S^T accumulator values form the P^T operand of the PV MFMA.
__device__ __forceinline__ int tau_group(int g4) {  // group of 4 positions -> group of 4 tokens
  const int w = g4 & 3;
  return (g4 & ~3) | (w == 1 ? 2 : (w == 2 ? 1 : w));
}

template <int D, int NWR>
struct TileRegs {
  static constexpr int NL = 64 * NWR;
  static constexpr int KJ = (Geo<D>::K_CHUNKS + NL - 1) / NL;
  static constexpr int VJ = (Geo<D>::V_UNITS + NL - 1) / NL;
  static constexpr bool K_CHUNKS_EXACT = Geo<D>::K_CHUNKS % NL == 0;
  static constexpr bool V_UNITS_EXACT = Geo<D>::V_UNITS % NL == 0;
  bf16x8 k[KJ];
  bf16x8 v[VJ][4];
};

// KV bytes are read exactly once: non-temporal loads keep them from evicting
// the lines this kernel writes and re-reads (outputs, block log masses).
__device__ __forceinline__ bf16x8 stream_load(const bf16x8* ptr) {
  return __builtin_nontemporal_load(ptr);
}

// K chunk ci: token ci / CPT, 16-byte column ci % CPT.  V unit ui: 4 tokens
// (positions 4*g4 .. 4*g4+3, g4 = ui % 8) x one 16-byte column ui / 8.
// Every load is issued unconditionally: tokens outside [lo, hi) still lie in
// an allocated page slot (a segment's page is valid, or page 0 for an empty
// segment), lanes past the tile's chunk count re-read the last chunk, and
// invalid tokens are dealt with when the tile is stored (V zeroed) and
// scored (logits masked).  Conditional loads would make the compiler wait
// for them before the next tile's loads are issued.
template <int D, int NWR>
__device__ __forceinline__ void load_tile(TileRegs<D, NWR>& r, const bf16* __restrict__ kc,
                                          const bf16* __restrict__ vc, const Seg& sa,
                                          const Seg& sb, int lig) {
  typedef TileRegs<D, NWR> TR;
  typedef Geo<D> G;
#pragma unroll
  for (int j = 0; j < TR::KJ; ++j) {
    int ci = lig + TR::NL * j;
    if (!TR::K_CHUNKS_EXACT) ci = min(ci, G::K_CHUNKS - 1);
    const int m = ci / G::CPT, c = ci % G::CPT;
    const long long base = m < kSeg ? sa.base : sb.base;
    r.k[j] = stream_load(reinterpret_cast<const bf16x8*>(kc + base + (long long)(m % kSeg) * D + 8 * c));
  }
#pragma unroll
  for (int j = 0; j < TR::VJ; ++j) {
    int ui = lig + TR::NL * j;
    if (!TR::V_UNITS_EXACT) ui = min(ui, G::V_UNITS - 1);
    const int g4 = ui & 7, c = (ui >> 3) % G::CPT;
    const int tok0 = 4 * tau_group(g4);
    const long long base = (tok0 < kSeg ? sa.base : sb.base) + (long long)(tok0 % kSeg) * D + 8 * c;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r.v[j][e] = stream_load(reinterpret_cast<const bf16x8*>(vc + base + (long long)e * D));
  }
}

// Tile registers -> LDS: K rows as loaded, V transposed.  Unless both
// segments are full, V rows of tokens outside their segment's [lo, hi) are
// zeroed (their probabilities are 0, but the cache slots may hold non-finite
// values).
template <int D, int NWR>
__device__ __forceinline__ void store_tile(TileRegs<D, NWR>& r, char* grp, int lig, const Seg& sa,
                                           const Seg& sb, bool full) {
  typedef TileRegs<D, NWR> TR;
  typedef Geo<D> G;
#pragma unroll
  for (int j = 0; j < TR::KJ; ++j) {
    const int ci = lig + TR::NL * j;
    if (TR::K_CHUNKS_EXACT || ci < G::K_CHUNKS) {
      const int m = ci / G::CPT, c = ci % G::CPT;
      *reinterpret_cast<bf16x8*>(grp + m * G::K_STRIDE + 16 * c) = r.k[j];
    }
  }
  char* vt = grp + G::K_BYTES;
#pragma unroll
  for (int j = 0; j < TR::VJ; ++j) {
    const int ui = lig + TR::NL * j;
    if (TR::V_UNITS_EXACT || ui < G::V_UNITS) {
      const int g4 = ui & 7, c = (ui >> 3) % G::CPT;
      if (!full) {
        const int tok0 = 4 * tau_group(g4);
        const Seg& sg = tok0 < kSeg ? sa : sb;
        const bf16x8 zero = {};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = sg.t0 + tok0 % kSeg + e;
          if (t < sg.lo || t >= sg.hi) r.v[j][e] = zero;
        }
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int d = 8 * c + dd;
        bf16x4 w;
        w[0] = r.v[j][0][dd];
        w[1] = r.v[j][1][dd];
        w[2] = r.v[j][2][dd];
        w[3] = r.v[j][3][dd];
        *reinterpret_cast<bf16x4*>(vt + vrow(d) * 64 + 16 * ((g4 >> 1) ^ vq_swz(d)) +
                                   8 * (g4 & 1)) = w;
      }
    }
  }
}

// ---- sparse verify: the union of a unit's per-position layouts ----

// Most blocks a unit's union can hold: every entry of every layout, and no
// more than the request has blocks.
__host__ __device__ __forceinline__ int union_max(int max_blocks, int n_q, int max_sel) {
  const long long e = (long long)n_q * max_sel;
  return e < max_blocks ? (int)e : max_blocks;
}

// Builds the union of the layouts of unit (b, h): the blocks before the
// window start that at least one query position selects, ascending, each
// with the mask of the positions selecting it, compacted into blk[] and
// msk[] (union_max entries each, at `list`).  `work` holds a mask per
// candidate block and then NT / 64 ints of scan scratch; it is only used
// here (the tile area, before any tile is stored).  Returns the union's
// size; all NT threads call it, and it ends with a barrier.
template <int NT>
__device__ int layout_union(const AttnParams& p, int b, int h, int ws, char* work, char* list) {
  const int ncand = min(ceil_div(ws, p.block_size), p.max_blocks);
  uint32_t* pm = reinterpret_cast<uint32_t*>(work);
  int* scratch = reinterpret_cast<int*>(pm + p.max_blocks);
  int32_t* blk = reinterpret_cast<int32_t*>(list);
  uint32_t* msk = reinterpret_cast<uint32_t*>(blk + union_max(p.max_blocks, p.n_q, p.max_sel));
  const int tid = threadIdx.x;
  for (int j = tid; j < ncand; j += NT) pm[j] = 0u;
  __syncthreads();
  const long long unit = (long long)b * p.num_kv_heads + h;
  const int32_t* rs = p.sel + unit * p.n_q * p.max_sel;  // [n_q][max_sel]
  const int32_t* rc = p.sel_count + unit * p.n_q;        // [n_q]
  for (int e = tid; e < p.n_q * p.max_sel; e += NT) {
    const int i = e / p.max_sel, k = e - i * p.max_sel;
    const int cnt = rc[i];
    if (k < cnt) {
      const int j = rs[e];
      if (j >= 0 && j < ncand) atomicOr(&pm[j], 1u << i);
    }
  }
  __syncthreads();
  // compaction in block order: thread t owns a contiguous range of blocks
  const int per = (ncand + NT - 1) / NT;
  const int j0 = min(tid * per, ncand), j1 = min(j0 + per, ncand);
  int mine = 0;
  for (int j = j0; j < j1; ++j) mine += pm[j] != 0u;
  int total;
  int pos = wg_exclusive_sum<NT>(mine, scratch, total);
  for (int j = j0; j < j1; ++j) {
    const uint32_t m = pm[j];
    if (m != 0u) {
      blk[pos] = j;
      msk[pos] = m;
      ++pos;
    }
  }
  __syncthreads();
  return total;
}

// ---- single-token draft lists (block size 1): a tile is 32 arbitrary
// tokens, each a row (page, head, slot) of the cache, read from a list
// staged in LDS for the whole chunk ----

// Bit m of the result: tile token m (list entry rel + m) is a real token of
// this token group.  Lanes 0..31 test one entry each.
__device__ __forceinline__ uint32_t gather_mask(const int32_t* rows_s, int rel, int n_left) {
  const int lane = threadIdx.x & 63;
  const bool v = lane < 32 && lane < n_left && rows_s[rel + lane] >= 0;
  return (uint32_t)__ballot(v);
}

// Same chunk and unit assignment as load_tile; each token's row comes from
// the list, an invalid token reads row 0 (allocated memory; masked later).
template <int D, int NWR>
__device__ __forceinline__ void load_tile_gather(TileRegs<D, NWR>& r, const bf16* __restrict__ kc,
                                                 const bf16* __restrict__ vc,
                                                 const int32_t* rows_s, int rel, uint32_t vm,
                                                 int lig) {
  typedef TileRegs<D, NWR> TR;
  typedef Geo<D> G;
#pragma unroll
  for (int j = 0; j < TR::KJ; ++j) {
    int ci = lig + TR::NL * j;
    if (!TR::K_CHUNKS_EXACT) ci = min(ci, G::K_CHUNKS - 1);
    const int m = ci / G::CPT, c = ci % G::CPT;
    const int row = ((vm >> m) & 1u) ? rows_s[rel + m] : 0;
    r.k[j] = stream_load(reinterpret_cast<const bf16x8*>(kc + (long long)row * D + 8 * c));
  }
#pragma unroll
  for (int j = 0; j < TR::VJ; ++j) {
    int ui = lig + TR::NL * j;
    if (!TR::V_UNITS_EXACT) ui = min(ui, G::V_UNITS - 1);
    const int g4 = ui & 7, c = (ui >> 3) % G::CPT;
    const int tok0 = 4 * tau_group(g4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = tok0 + e;
      const int row = ((vm >> m) & 1u) ? rows_s[rel + m] : 0;
      r.v[j][e] = stream_load(reinterpret_cast<const bf16x8*>(vc + (long long)row * D + 8 * c));
    }
  }
}

// store_tile for a gathered tile: V rows of tokens outside the mask zeroed.
template <int D, int NWR>
__device__ __forceinline__ void store_tile_gather(TileRegs<D, NWR>& r, char* grp, int lig,
                                                  uint32_t vm) {
  typedef TileRegs<D, NWR> TR;
  typedef Geo<D> G;
#pragma unroll
  for (int j = 0; j < TR::KJ; ++j) {
    const int ci = lig + TR::NL * j;
    if (TR::K_CHUNKS_EXACT || ci < G::K_CHUNKS) {
      const int m = ci / G::CPT, c = ci % G::CPT;
      *reinterpret_cast<bf16x8*>(grp + m * G::K_STRIDE + 16 * c) = r.k[j];
    }
  }
  char* vt = grp + G::K_BYTES;
#pragma unroll
  for (int j = 0; j < TR::VJ; ++j) {
    const int ui = lig + TR::NL * j;
    if (TR::V_UNITS_EXACT || ui < G::V_UNITS) {
      const int g4 = ui & 7, c = (ui >> 3) % G::CPT;
      if (vm != 0xffffffffu) {
        const int tok0 = 4 * tau_group(g4);
        const bf16x8 zero = {};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!((vm >> (tok0 + e)) & 1u)) r.v[j][e] = zero;
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int d = 8 * c + dd;
        bf16x4 w;
        w[0] = r.v[j][0][dd];
        w[1] = r.v[j][1][dd];
        w[2] = r.v[j][2][dd];
        w[3] = r.v[j][3][dd];
        *reinterpret_cast<bf16x4*>(vt + vrow(d) * 64 + 16 * ((g4 >> 1) ^ vq_swz(d)) +
                                   8 * (g4 & 1)) = w;
      }
    }
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Largest lead (log2 units) of a row's logits over the softmax reference
// before the reference moves: terms stay <= 256, exact in fp32 and bf16 range.
constexpr float kRescaleSlack = 8.f;

// A single-token verify tile's logits are stored one tile later, ahead of
// the next tile's loads: stores count in the same in-order counter as loads,
// so a store issued after the loads would lengthen the wait for them.  They
// stay in the wave's LDS parking area (4 KiB, 32 tokens x 32 rows), which
// survives until then when it is a slot of its own (several row tiles); a
// single row tile parks in its K tile, which the next tile overwrites, so
// there the logits are read back token-major into registers first (REGS: 4
// chunks of 4 rows when the row count is a multiple of 4, else 16 single
// rows).  t0 = the tile's first token, -1 = nothing held (wave-uniform).
// Empty for every other kernel, whose code it leaves untouched.
template <bool ON, bool REGS>
struct TokPark {
  float v[REGS ? 16 : 1];
  int t0 = -1, n = 0;
};
template <bool REGS>
struct TokPark<false, REGS> {};

// The logits of a parked tile, the lane's share: for a row count that is a
// multiple of 4, chunk i (4 rows from 4q) of token m = lane / 8 + 8 i; else
// row rr of token m = lane / 32 + 2 i.  Indexes past the tile's tokens or the
// wave's rows repeat the last valid one (with its value), so every lane
// issues the same fixed number of stores.
__device__ __forceinline__ int tok_q(int lane, int rw) { return min(lane & 7, (rw >> 2) - 1); }
__device__ __forceinline__ int tok_m4(int lane, int i, int n) { return min((lane >> 3) + 8 * i, n - 1); }
__device__ __forceinline__ int tok_rr(int lane, int rw) { return min(lane & 31, rw - 1); }
__device__ __forceinline__ int tok_m1(int lane, int i, int n) { return min((lane >> 5) + 2 * i, n - 1); }

template <bool REGS>
__device__ __forceinline__ void tok_park(TokPark<true, REGS>& tp, const float* stage, int t0,
                                         int n, int R, int rt, int lane) {
  if constexpr (REGS) {
    const int rw = min(32, R - rt * 32);
    if ((rw & 3) == 0 && (R & 3) == 0) {
      const int q = tok_q(lane, rw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage + tok_m4(lane, i, n) * 32 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) tp.v[4 * i + e] = v[e];
      }
    } else {
      const int rr = tok_rr(lane, rw);
#pragma unroll
      for (int i = 0; i < 16; ++i) tp.v[i] = stage[tok_m1(lane, i, n) * 32 + rr];
    }
  }
  tp.t0 = t0;
  tp.n = n;
}

// Stores what tp holds: token t0 + m, row r of the unit at ell_u[(t0 + m) *
// R + r], this wave's rows rt * 32 .. rt * 32 + 31.  (Offsets stay 32-bit:
// 64-bit addresses held across the tile loop cost more registers than exist.)
template <bool REGS>
__device__ __forceinline__ void tok_flush(TokPark<true, REGS>& tp, const float* stage,
                                          float* ell_u, int R, int rt, int lane) {
  if (tp.t0 < 0) return;
  const int rw = min(32, R - rt * 32);
  float* const dst = ell_u + (long long)tp.t0 * R + rt * 32;
  if ((rw & 3) == 0 && (R & 3) == 0) {
    const int q = tok_q(lane, rw);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tok_m4(lane, i, tp.n);
      f32x4 v;
      if constexpr (REGS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = tp.v[4 * i + e];
      } else {
        v = *reinterpret_cast<const f32x4*>(stage + m * 32 + 4 * q);
      }
      *reinterpret_cast<f32x4*>(dst + (m * R + 4 * q)) = v;
    }
  } else {
    const int rr = tok_rr(lane, rw);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = tok_m1(lane, i, tp.n);
      dst[m * R + rr] = REGS ? tp.v[REGS ? i : 0] : stage[m * 32 + rr];
    }
  }
  tp.t0 = -1;
}

// Runs one item with all 64 * NWR * NWT threads of the workgroup over the
// LDS area `smem` (item_lds_bytes(D, NWR, NWT) bytes; with ELL_LDS, also
// the chunk's block log masses, chunk-blocks x rows floats at byte offset
// it.ell_off).  Final outputs (o, lse and, for
// verify, block_scores) are written when the unit fits in this chunk or
// it.single is set; otherwise the normalised partial O and log2 LSE of the
// chunk go to p.o_part / p.lse_part row it.part_row0 + c * rows, and the
// chunk's block log masses to p.ell.  Returns the ItemStatus.
//
// PD: tiles in flight per token group (register prefetch depth).  A tile
// shared by several row waves costs each of them only a fraction of its
// registers, so those configurations keep two tiles in flight.
// TOKENS: blocks of one token.  A draft then gathers its tiles token by
// token from a list (one row tile only); a verify stores each token's logit
// as its log mass.
// QREG: the Q operand is held in registers (staged once through the first
// tile buffer, before any tile is stored) instead of LDS, for block-level
// verify of one row tile; it frees the Q tile's LDS.
template <int D, int NWR, int NWT, bool DRAFT, bool ELL_LDS, bool TOKENS = false,
          bool SPARSE = false, bool QREG = false>
__device__ int attn_item(const AttnParams& p, const Item& it, char* smem) {
  static_assert(!SPARSE || (!DRAFT && !ELL_LDS && !TOKENS), "sparse verify is its own mode");
  constexpr bool GATHER = DRAFT && TOKENS;
  constexpr bool LIST = DRAFT || SPARSE;     // segments come from a block list
  constexpr bool SCORES = !DRAFT && !SPARSE;  // block importance is computed
  static_assert(!GATHER || NWR == 1, "token lists serve one-row-tile drafts");
  // tiles in flight per token group: two with several row waves, one
  // otherwise (two for the Q-in-registers verify and the one-wave draft,
  // each then one wave per SIMD, made the batch-128 x 8K step slower on
  // MI355X: 0.731 against 0.720 ms)
  constexpr int PD = NWR >= 2 ? 2 : 1;
  constexpr int NT = 64 * NWR * NWT;
  typedef Geo<D> G;

  const int u = it.u, c = it.c;
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = w % NWR, tg = w / NWR;
  const int lig = rt * 64 + lane;
  const int hl = lane >> 5;   // half of the wave: K-half of operands
  const int rl = lane & 31;   // row within the tile
  const int R = p.rows;
  const int r = rt * 32 + rl;  // unit row of this lane
  const bool row_ok = r < R;
  const int iq = row_ok ? r / p.group : 0;
  const int hq = h * p.group + (row_ok ? r % p.group : 0);
  // double-buffered K/V tiles (tile t in buffer t & 1); otherwise one
  // buffer per token group, reused by every tile
  constexpr bool DB = tile_buffers(NWR, NWT) == 2 && NWT == 1;
  constexpr int NBUF = tile_buffers(NWR, NWT);
  static_assert(!QREG || (NWR == 1 && !DRAFT && !TOKENS && !SPARSE),
                "Q in registers: block-level verify of one row tile only");
  float* lse2s =
      reinterpret_cast<float*>(smem + NBUF * G::GROUP_BYTES + (QREG ? 0 : NWR * G::Q_BYTES));

  const int L = p.seq_lens[b];
  const int minL = DRAFT ? 1 : p.n_q;
  const bool unit_ok =
      L >= minL && L <= p.max_seq_len && (long long)L <= (long long)p.max_pages * p.page_size;
  if (!unit_ok) {
    // chunk 0 owns the unit's (NaN) outputs
    if (c != 0) return kItemNone;
    if (tg == 0 && row_ok) {
      bf16* o = reinterpret_cast<bf16*>(p.o);
      const long long orow = ((long long)b * p.n_q + iq) * p.num_q_heads + hq;
      for (int d = hl; d < D; d += 2) o[orow * D + d] = from_f32<bf16>(qnan());
      if (hl == 0) p.lse[orow] = qnan();
    }
    if (SCORES)
      for (int j = threadIdx.x; j < p.max_blocks; j += NT)
        p.block_scores[(long long)u * p.max_blocks + j] = qnan();
    return kItemFinal;
  }

  // ---- this item's segment range, split among token groups ----
  int seg_lo, seg_hi, nsel = 0, ws = L, nseg = 0;
  // sparse verify: the union of the unit's layouts in LDS at it.list_off,
  // ascending block ids with the query positions holding each
  const int32_t* ublk = nullptr;
  const uint32_t* umsk = nullptr;
  if (!LIST) {
    const int t_lo = c * it.chunk;
    if (t_lo >= L) return kItemNone;  // chunk past this request's length
    const int t_hi = min(t_lo + it.chunk, L);
    seg_lo = t_lo / kSeg;
    seg_hi = ceil_div(t_hi, kSeg);
  } else {
    ws = window_start(L, p.window);
    if constexpr (SPARSE) {
      nsel = layout_union<NT>(p, b, h, ws, smem, smem + it.list_off);
      ublk = reinterpret_cast<const int32_t*>(smem + it.list_off);
      umsk = reinterpret_cast<const uint32_t*>(ublk + union_max(p.max_blocks, p.n_q, p.max_sel));
    } else {
      nsel = it.sel_off >= 0 ? it.nsel_s : p.sel_count[(long long)b * p.num_kv_heads + h];
      nsel = nsel < 0 ? 0 : (nsel > p.max_sel ? p.max_sel : nsel);
    }
    nseg = GATHER ? draft_list_len_simple(nsel, 1, L, ws)
                  : draft_list_len_mfma(nsel, p.block_size, L, ws);
    seg_lo = c * it.chunk;
    // the merge learns a sparse unit's list length from its chunk 0
    if (SPARSE && c == 0 && threadIdx.x == 0 && p.list_len) p.list_len[u] = nseg;
    if (seg_lo >= nseg && c > 0) return kItemNone;
    seg_hi = min(seg_lo + it.chunk, nseg);
  }
  // a unit that fits in its first chunk is finished here (outputs, scores)
  const bool final_out =
      it.single || (LIST ? (c == 0 && nseg <= it.chunk) : (c == 0 && L <= it.chunk));
  constexpr bool ell_lds = SCORES && ELL_LDS;
  // first block of the chunk (chunks hold whole blocks); the LDS copy of the
  // block log masses holds the chunk's blocks only and is addressed by
  // absolute block index through an offset base
  const int blk0 = LIST ? 0 : c * (it.chunk / p.block_size);
  float* const ell_s = reinterpret_cast<float*>(smem + it.ell_off) - (ptrdiff_t)blk0 * p.rows;
  const int32_t* const sel_s =
      SPARSE ? ublk
             : ((DRAFT && it.sel_off >= 0) ? reinterpret_cast<const int32_t*>(smem + it.sel_off)
                                           : nullptr);
  // the item's entries split evenly over the token groups, in whole tiles
  // (and, for block masses, whole blocks): a list or a request shorter
  // than the chunk still keeps every group busy
  const int galign = GATHER ? 32 : ((LIST || p.block_size < 2 * kSeg) ? 2 : p.block_size / kSeg);
  const int per_group = ceil_div(ceil_div(seg_hi - seg_lo, NWT), galign) * galign;
  const int g_lo = min(seg_lo + tg * per_group, seg_hi);
  const int g_hi = min(g_lo + per_group, seg_hi);
  // list entries per tile: two 16-token segments, or 32 single tokens
  constexpr int kTileEntries = GATHER ? 32 : 2;
  const int n_tiles = ceil_div(min(per_group, seg_hi - seg_lo), kTileEntries);  // group 0 has the most
  // token list of a single-token draft chunk: cache row of each entry
  int32_t* const rows_s = reinterpret_cast<int32_t*>(smem + (GATHER ? it.list_off : 0));

  const bf16* __restrict__ kc = reinterpret_cast<const bf16*>(p.k);
  const bf16* __restrict__ vc = reinterpret_cast<const bf16*>(p.v);
  char* grp = smem + tg * G::GROUP_BYTES;
  const FastDiv pdiv(p.page_size), bdiv(p.block_size);

  int bad = 0;
  // segment descriptors of the first two batches of 64
  SegLane cur = {}, nxt = {};
  if constexpr (!GATHER) {
    cur = seg_lane<LIST>(p, sel_s, b, h, g_lo + lane, g_hi, nsel, L, ws, umsk);
    nxt = seg_lane<LIST>(p, sel_s, b, h, g_lo + 64 + lane, g_hi, nsel, L, ws, umsk);
  }
  int cur_batch = 0;
  // gathered tiles: list entry of the token group's first token, relative
  // to the chunk's list, and the tokens left from there
  const int g_rel = g_lo - seg_lo, g_len = g_hi - g_lo;

  if constexpr (GATHER) {
    // the chunk's token list: selected tokens before the window, then the
    // window; entries past the list are -1
    for (int e = threadIdx.x; e < it.chunk; e += NT) {
      const int k = seg_lo + e;
      int row = -1;
      if (k < seg_hi) {
        int t = -1;
        if (k < nsel) {
          const int j = sel_s ? sel_s[k]
                              : p.sel[((long long)b * p.num_kv_heads + h) * p.max_sel + k];
          if (j >= 0 && j < ws) t = j;
        } else {
          t = ws + (k - nsel);
        }
        if (t >= 0) {
          const int pg = p.page_table[(long long)b * p.max_pages + t / p.page_size];
          if (pg < 0 || pg >= p.num_pages)
            bad = 1;
          else
            row = (pg * p.num_kv_heads + h) * p.page_size + t % p.page_size;
        }
      }
      rows_s[e] = row;
    }
  }

  // ---- Q rows of each row tile -> LDS (the Q^T operand is read from there,
  // or, with QREG, staged in the first tile buffer and read into registers) ----
  char* qtile = QREG ? smem : smem + NBUF * G::GROUP_BYTES + rt * G::Q_BYTES;
  if (tg == 0) {
#pragma unroll
    for (int j = 0; j < (32 * G::CPT) / 64; ++j) {
      const int ci = lane + 64 * j;
      const int row = ci / G::CPT, cc = ci % G::CPT;
      const int rr = rt * 32 + row;
      uint4 v = {0u, 0u, 0u, 0u};
      if (rr < R) {
        const int qi = rr / p.group, qh = h * p.group + rr % p.group;
        v = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16*>(p.q) +
                                            (((long long)b * p.n_q + qi) * p.num_q_heads + qh) * D +
                                            8 * cc);
        // a negative scale is folded into Q (an exact sign flip), so the
        // tile loop scales by |scale| and max-reduces unscaled logits
        if (p.scale_log2 < 0.f) {
          v.x ^= 0x80008000u;
          v.y ^= 0x80008000u;
          v.z ^= 0x80008000u;
          v.w ^= 0x80008000u;
        }
      }
      *reinterpret_cast<uint4*>(qtile + row * G::K_STRIDE + 16 * cc) = v;
    }
  }
  __syncthreads();
  bf16x8 qreg[QREG ? G::KS : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks)
      qreg[ks] = *reinterpret_cast<const bf16x8*>(qtile + rl * G::K_STRIDE + 32 * ks + 16 * hl);
    // every wave holds its Q before token group 0 stores its first tile there
    __syncthreads();
  }
  const int pos_r = DRAFT ? (L - 1) : (L - p.n_q + iq);
  const int pos_min = DRAFT ? (L - 1) : (L - p.n_q);  // smallest causal limit of the unit's rows
  // |scale| (log2 domain), kept positive so that a masked -inf logit times
  // it stays -inf (a zero scale becomes a negligible positive one)
  const float scl = fmaxf(fabsf(p.scale_log2), 1e-30f);
  // sparse verify: every query position of the unit, and those of this row
  // wave's rows
  const uint32_t all_pos = (uint32_t)((2ull << (p.n_q - 1)) - 1ull);
  const uint32_t wave_pos =
      (uint32_t)((2ull << ((min(rt * 32 + 32, R) - 1) / p.group)) - (1ull << ((rt * 32) / p.group)));

  f32x16 oacc[G::MT];
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mt][i] = 0.f;
  float m_run = neg_inf(), l_run = 0.f, blk_run = 0.f;
  // without LDS room the block log mass of a tile is stored one iteration
  // later, ahead of the next tile's loads: stores count in the same in-order
  // counter as loads, so a store issued after the loads would lengthen the
  // wait for them
  float ell_val = 0.f;
  long long ell_at = -1;
  float* ell_u = p.ell + (long long)u * p.max_blocks * R;

  // single-token verify: this wave's logit parking area
  float* const tok_stage = NWR == 1 ? reinterpret_cast<float*>(grp)
                                    : reinterpret_cast<float*>(smem + it.list_off) + w * 32 * 32;
  // ... and the last live tile's logits, held until the next tile's loads
  TokPark<SCORES && TOKENS, NWR == 1> tpark;

  // the first two batches' page ids, loaded while Q was staged (resolving
  // them before the Q loads made every unit wait one more round trip)
  if constexpr (!GATHER) {
    seg_resolve(p, pdiv, h, cur, bad);
    seg_resolve(p, pdiv, h, nxt, bad);
  }
  TileRegs<D, NWR> regs[PD];
  Seg sa[PD], sb[PD];
  uint32_t vm[PD];
#pragma unroll
  for (int q = 0; q < PD; ++q) {
    if constexpr (GATHER) {
      vm[q] = gather_mask(rows_s, g_rel + 32 * q, g_len - 32 * q);
      load_tile_gather<D, NWR>(regs[q], kc, vc, rows_s, g_rel + 32 * q, vm[q], lig);
    } else {
      sa[q] = seg_of<SPARSE>(p, cur, nxt, false, 2 * q);
      sb[q] = seg_of<SPARSE>(p, cur, nxt, false, 2 * q + 1);
      load_tile<D, NWR>(regs[q], kc, vc, sa[q], sb[q], lig);
    }
  }

  // With PD > 1 every trip runs all PD slots and issues each slot's next
  // loads unconditionally (past the group's tiles they read empty segments
  // of page 0): the compiler's count of the loads issued after a slot's is
  // then the same on every path.  With a break or a conditional load in the
  // trip it merged in paths on which fewer loads followed and waited for
  // the other slot's loads as well before every store, keeping one tile in
  // flight instead of PD.
  for (int t0 = 0; t0 < n_tiles; t0 += PD)
#pragma unroll
  for (int q = 0; q < PD; ++q) {
    const int t = t0 + q;
    const bool live = PD == 1 || t < n_tiles;  // uniform
    const int rel0 = kTileEntries * t;
    const bool tile_live = live && g_lo + rel0 < g_hi;
    const Seg ca = sa[q], cb = sb[q];
    char* const gt = DB ? smem + (t & 1) * G::GROUP_BYTES : grp;
    const uint32_t vmq = GATHER ? vm[q] : 0u;
    bool full = false;
    if (live) {
      if constexpr (GATHER) {
        full = vmq == 0xffffffffu;
        store_tile_gather<D, NWR>(regs[q], gt, lig, vmq);
      } else {
        full = seg_full(ca) && seg_full(cb);
        store_tile<D, NWR>(regs[q], gt, lig, ca, cb, full);
      }
    }
    if (!GATHER && rel0 > 0 && (rel0 & 63) == 0) {
      // move to the next batch of descriptors; fetch the one after it
      cur = nxt;
      ++cur_batch;
      nxt = seg_lane<LIST>(p, sel_s, b, h, g_lo + 64 * (cur_batch + 1) + lane, g_hi, nsel, L, ws,
                           umsk);
    }
    // the next batch's page ids were fetched 16 tiles ago: resolve them
    // before the first prefetch that reads that batch (its last tiles)
    if (!GATHER && (rel0 & 63) == 32) seg_resolve(p, pdiv, h, nxt, bad);
    if (live) group_sync<NWR>();
    if (SCORES && !ell_lds) {
      if (ell_at >= 0) ell_u[ell_at] = ell_val;
      ell_at = -1;
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SCORES && TOKENS) {
      tok_flush(tpark, tok_stage, ell_u, R, rt, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (PD > 1 || t + PD < n_tiles) {
      if constexpr (GATHER) {
        const int rn = rel0 + 32 * PD;
        vm[q] = gather_mask(rows_s, g_rel + rn, g_len - rn);
        load_tile_gather<D, NWR>(regs[q], kc, vc, rows_s, g_rel + rn, vm[q], lig);
      } else {
        const int ra = rel0 + 2 * PD, rb = ra + 1;
        sa[q] = seg_of<SPARSE>(p, cur, nxt, (ra >> 6) != cur_batch, ra & 63);
        sb[q] = seg_of<SPARSE>(p, cur, nxt, (rb >> 6) != cur_batch, rb & 63);
        load_tile<D, NWR>(regs[q], kc, vc, sa[q], sb[q], lig);
      }
    }
    // sparse verify: a row wave skips a tile that none of its query
    // positions selected (the window segments count for every position)
    const bool wave_live = tile_live && (!SPARSE || ((ca.pm | cb.pm) & wave_pos) != 0u);
    if (wave_live) {
      // S^T = K Q^T
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(gt + rl * G::K_STRIDE + 32 * ks + 16 * hl);
        const bf16x8 qb =
            QREG ? qreg[QREG ? ks : 0]
                 : *reinterpret_cast<const bf16x8*>(qtile + rl * G::K_STRIDE + 32 * ks + 16 * hl);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb, sacc, 0, 0, 0);
      }
      // online softmax (log2 domain; s holds unscaled logits, masked ones
      // -inf, and the scale enters with the exponent); interior tiles need
      // no mask
      float s[16];
      float mx = neg_inf();
      const bool interior = full && (GATHER || cb.t0 + kSeg - 1 <= pos_min) &&
                            (!SPARSE || (ca.pm & cb.pm & all_pos) == all_pos);
      if (interior) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = sacc[i];
          mx = fmaxf(mx, s[i]);
        }
      } else if constexpr (GATHER) {
        // every listed token precedes the query: only the mask applies
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = (i >> 2) * 8 + 4 * hl + (i & 3);
          s[i] = ((vmq >> m) & 1u) ? sacc[i] : neg_inf();
          mx = fmaxf(mx, s[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = (i >> 2) * 8 + 4 * hl + (i & 3);
          const Seg& sg = (m < kSeg) ? ca : cb;
          const int tok = sg.t0 + (m % kSeg);
          bool ok = tok >= sg.lo && tok < sg.hi && tok <= pos_r;
          if (SPARSE) ok = ok && ((sg.pm >> iq) & 1u);
          s[i] = ok ? sacc[i] : neg_inf();
          mx = fmaxf(mx, s[i]);
        }
      }
      if constexpr (!DRAFT && TOKENS) {
        // single-token blocks: the log mass of token t in row r is the
        // (masked) logit itself, whatever the frame.  The wave parks its
        // 32 tokens x 32 rows in 4 KiB of LDS of its own (one row tile: the
        // tile's K rows, which S has consumed; else a slot at it.list_off)
        // and stores them once the tile is done
#pragma unroll
        for (int i = 0; i < 16; ++i)
          tok_stage[((i >> 2) * 8 + 4 * hl + (i & 3)) * 32 + rl] = s[i] * scl;
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * scl;
      // lazy rescaling: the reference max m_run moves only when a row's max
      // exceeds it by more than kRescaleSlack (log2 units), so softmax terms
      // stay <= 2^kRescaleSlack and most tiles skip the O rescale entirely
      const float m_new = fmaxf(m_run, mx);
      const bool move = (m_run == neg_inf()) || (m_new > m_run + kRescaleSlack);
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float m_tgt = move ? m_new : m_run;
        const float alpha = (m_tgt == neg_inf()) ? 1.f : fast_exp2(m_run - m_tgt);
        l_run *= alpha;
        blk_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[mt][i] *= alpha;
        m_run = m_tgt;
      }
      const float m_use = (m_run == neg_inf()) ? 0.f : m_run;
      float pr[16];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pr[i] = fast_exp2(fmaf(s[i], scl, -m_use));
        psum += pr[i];
      }
      l_run += psum;
      // O^T += V^T P^T
      char* vt = gt + G::K_BYTES;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = static_cast<bf16>(pr[8 * kk + j]);
        const int qd = 2 * kk + hl;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
          const int d = 32 * mt + rl;
          const bf16x8 va =
              *reinterpret_cast<const bf16x8*>(vt + vrow(d) * 64 + 16 * (qd ^ vq_swz(d)));
          oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[mt], 0, 0, 0);
        }
      }
      if (SCORES) {
        // per-block log mass of this row, frame m_use
        const int bs = p.block_size;
        if constexpr (SCORES && TOKENS) {
          // the tile's logits, held for the next tile (tok_flush): token
          // ca.t0 + m, for the tokens of the request only
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          tok_park(tpark, tok_stage, ca.t0, min(32, L - ca.t0), R, rt, lane);
        } else if (bs == kSeg) {
          float a = 0.f, bb = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a += pr[i];
#pragma unroll
          for (int i = 8; i < 16; ++i) bb += pr[i];
          a += __shfl_xor(a, 32);
          bb += __shfl_xor(bb, 32);
          const Seg& mine = hl ? cb : ca;
          if (row_ok && mine.lo < mine.hi) {
            const float v = m_use + fast_log2(hl ? bb : a);
            if (ell_lds) {
              ell_s[(mine.t0 / kSeg) * R + r] = v;
            } else {
              ell_at = (long long)(mine.t0 / kSeg) * R + r;
              ell_val = v;
            }
          }
        } else {
          blk_run += psum;
          const int tile_end = ca.t0 + 2 * kSeg;
          const bool last = (bdiv.mod(tile_end) == 0) || (g_lo + rel0 + 2 >= g_hi);
          if (last) {
            const float tot = blk_run + __shfl_xor(blk_run, 32);
            if (row_ok && hl == 0) {
              const float v = m_use + fast_log2(tot);
              if (ell_lds) {
                ell_s[bdiv.div(ca.t0) * R + r] = v;
              } else {
                ell_at = (long long)bdiv.div(ca.t0) * R + r;
                ell_val = v;
              }
            }
            blk_run = 0.f;
          }
        }
      }
    }
    // a double-buffered tile needs no second barrier: the next tile goes to
    // the other buffer, and the waves meet at the next tile's barrier before
    // the buffer after it is written
    if (!DB && live) group_sync<NWR>();
  }

  if (SCORES && ell_at >= 0) ell_u[ell_at] = ell_val;
  if constexpr (SCORES && TOKENS) tok_flush(tpark, tok_stage, ell_u, R, rt, lane);

  // ---- combine the lane pair, then the token groups ----
  l_run += __shfl_xor(l_run, 32);
  bad = __syncthreads_or(bad);
  if (SCORES && ell_lds && !final_out) {
    // the chunk's block log masses -> workspace, for the split merge
    const int blk_end = ceil_div(min((c + 1) * it.chunk, L), p.block_size);
    for (int i = blk0 * R + threadIdx.x; i < blk_end * R; i += NT) ell_u[i] = ell_s[i];
  }
  if (NWT > 1) {
    float* red = reinterpret_cast<float*>(smem);  // [NWT-1][NWR][32][D]
    float* ml = red + (NWT - 1) * NWR * 32 * D;   // [NWT][NWR][32] max, then sum
    if (hl == 0) {
      ml[(tg * NWR + rt) * 32 + rl] = m_run;
      ml[NWT * NWR * 32 + (tg * NWR + rt) * 32 + rl] = l_run;
    }
    if (tg > 0) {
      float* dst = red + (((tg - 1) * NWR + rt) * 32 + rl) * D;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = oacc[mt][4 * q4 + e];
          *reinterpret_cast<f32x4*>(dst + 32 * mt + 8 * q4 + 4 * hl) = v4;
        }
    }
    __syncthreads();
    if (tg == 0) {
      float mg = m_run;
#pragma unroll
      for (int g = 1; g < NWT; ++g) mg = fmaxf(mg, ml[(g * NWR + rt) * 32 + rl]);
      const float mu = (mg == neg_inf()) ? 0.f : mg;
      const float a0 = fast_exp2(m_run - mu);
      float lsum = l_run * a0;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mt][i] *= a0;
#pragma unroll
      for (int g = 1; g < NWT; ++g) {
        const float ag = fast_exp2(ml[(g * NWR + rt) * 32 + rl] - mu);
        lsum += ag * ml[NWT * NWR * 32 + (g * NWR + rt) * 32 + rl];
        const float* src = red + (((g - 1) * NWR + rt) * 32 + rl) * D;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + 32 * mt + 8 * q4 + 4 * hl);
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[mt][4 * q4 + e] += ag * v4[e];
          }
      }
      m_run = mg;
      l_run = lsum;
    }
  }

  if (tg == 0 && row_ok) {
    const bool empty = !(l_run > 0.f);
    const float inv = empty ? 0.f : 1.f / l_run;
    const float lse2 = bad ? qnan() : (empty ? neg_inf() : m_run + fast_log2(l_run));
    const float poison = bad ? qnan() : 1.f;
    if (final_out) {
      bf16* o = reinterpret_cast<bf16*>(p.o);
      const long long orow = ((long long)b * p.n_q + iq) * p.num_q_heads + hq;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v4[e] = from_f32<bf16>(oacc[mt][4 * q4 + e] * inv * poison);
          *reinterpret_cast<bf16x4*>(o + orow * D + 32 * mt + 8 * q4 + 4 * hl) = v4;
        }
      if (hl == 0) {
        p.lse[orow] = lse2 * kLn2;
        if (SCORES) lse2s[r] = lse2;
      }
    } else {
      const long long prow = it.part_row0 + (long long)c * R + r;
      float* op = p.o_part + prow * D;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = oacc[mt][4 * q4 + e] * inv * poison;
          *reinterpret_cast<f32x4*>(op + 32 * mt + 8 * q4 + 4 * hl) = v4;
        }
      if (hl == 0) p.lse_part[prow] = lse2;
    }
  }

  if (SCORES && final_out) {
    // the whole unit ran in this item: block scores from its block log
    // masses (LDS, or read back from L2) and the final row LSEs
    __threadfence_block();
    __syncthreads();
    const int nblk = ceil_div(L, p.block_size);
    const float* ell = ell_lds ? ell_s : ell_u;
    const int r0 = p.score_row_start * p.group;
    if (TOKENS && (R & 3) == 0 && (r0 & 3) == 0) {
      // one token per thread, its rows as 16-byte loads issued 8 at a time
      // (the log masses come back from L2 / HBM, so loads are batched)
      const int nq = (R - r0) >> 2;
      for (int j = threadIdx.x; j < p.max_blocks; j += NT) {
        float sc = 0.f;
        if (j < nblk) {
          const f32x4* e = reinterpret_cast<const f32x4*>(ell + (long long)j * R + r0);
          for (int q0 = 0; q0 < nq; q0 += 8) {
            f32x4 x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (q0 + k < nq) x[k] = e[q0 + k];
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (q0 + k < nq) {
                const float* l2 = lse2s + r0 + 4 * (q0 + k);
                sc += fast_exp2(x[k][0] - l2[0]) + fast_exp2(x[k][1] - l2[1]) +
                      fast_exp2(x[k][2] - l2[2]) + fast_exp2(x[k][3] - l2[3]);
              }
          }
        }
        p.block_scores[(long long)u * p.max_blocks + j] = bad ? qnan() : sc;
      }
    } else {
      for (int j = threadIdx.x; j < p.max_blocks; j += NT) {
        float sc = 0.f;
        if (j < nblk) {
          const float* e = ell + (long long)j * R;
          for (int rr = r0; rr < R; ++rr) sc += fast_exp2(e[rr] - lse2s[rr]);
        }
        p.block_scores[(long long)u * p.max_blocks + j] = bad ? qnan() : sc;
      }
    }
  }
  return final_out ? kItemFinal : kItemPartial;
}

}  // namespace sss
