// Verify attention for units of three 32-row tiles (65 to 96 rows per
// (request, KV head): k+1 query positions x G heads, e.g. 5 x 16 = 80) with
// a load-specialised wave (SparseSpec §4.1, Fig. 7: the verify pass is full
// attention of all k+1 positions over the cache, and it also yields the
// per-block probability mass the Top-K selection reads; SparseSpec §2.1:
// verification is bound by the KV bytes it loads, so the kernel must keep
// the load stream full).
//
// A workgroup is four waves: three compute waves, one per 32-row tile, and
// one load wave.  The load wave streams the chunk's 32-token K/V tiles from
// the paged cache (three tiles in flight in its registers; the chunk's page
// ids staged in LDS first) and writes each into a ring of up to four LDS
// tile buffers (K and V rows as loaded; the compute waves read V^T with
// transposing LDS reads).  LDS counters, not
// barriers, order the ring, so the load wave runs ahead while the compute
// waves work.  The compute waves hold their Q rows in registers and only
// read LDS and issue matrix-core and softmax instructions.
//
// Measured on 8 units of 80 rows x 128K tokens in 64 chunks (MI355X): the
// one-routine form (attn_item with three row waves, each loading a third of
// every tile, Q read from LDS, 228 VGPRs, six waves on four SIMDs) took
// 122 us; this kernel with a barrier per tile 104 us (its load wave alone
// streams in 78 us, the compute waves alone need 80 us); with the counter
// ring 107 us -- the load wave still kept one tile in flight, because the
// compiler's wait counts were conservative (see the load loop) -- and with
// three tiles really in flight and no page-table reads in the loop,
// 91-101 us; with the 16-row last tile on 16x16x32 MFMAs and the wave
// roles below, 2% less again (verify call 0.113 against 0.115 ms in an
// interleaved A/B).  One workgroup per compute unit (each wave alone on its
// SIMD, five tiles in the load wave's registers) took 0.166 ms: the two
// workgroups' compute chains need to overlap.

// The arithmetic of the 32-row tiles is attn_item's for the same item (one
// token group, the same tiles in the same order, the same masking, lazy
// rescaling and block log masses); a 16-row last tile sums its rows' terms
// in another order, so it agrees with that routine up to rounding.  Split
// chunks keep their block log masses in LDS and copy them to the workspace
// in one burst at the end.
#include "attn_item.h"
#include "attn_tile.h"

namespace sss {
namespace {

constexpr int kRowWaves = 3;                     // compute waves: one 32-row tile each
constexpr int kRowsThreads = 64 * (kRowWaves + 1);
constexpr int kLoadSlots = 3;                    // tiles the load wave holds in registers
constexpr int kMaxTileBufs = 4;                  // tiles the load wave may hold in LDS
constexpr int kSpinCap = 1 << 22;                // polls before a counter wait gives up

// A tile in LDS: K rows as loaded (row stride 2 D + 16 bytes), then V rows
// as loaded (stride 2 D + 32: the transposing reads below take four rows
// of one 8-byte column group per lane quad, and this stride spreads them
// over distinct banks).  The compute waves read V^T with
// ds_read_b64_tr_b16, so the load wave stores V untransposed.
template <int D>
struct RowsTile {
  static constexpr int K_STRIDE = 2 * D + 16;
  static constexpr int V_STRIDE = 2 * D + 32;
  static constexpr int K_BYTES = 32 * K_STRIDE;
  static constexpr int BYTES = K_BYTES + 32 * V_STRIDE;
  static constexpr int CHUNKS = 32 * D / 8;  // 16-byte chunks of K (and of V)
};

// A tile's K and V, 16-byte chunk ci = lane + 64 j of each: token ci / (D / 8),
// column chunk ci % (D / 8), as loaded.
template <int D>
struct RowRegs {
  static constexpr int J = RowsTile<D>::CHUNKS / 64;
  bf16x8 k[J];
  bf16x8 v[J];
};

// Loads a tile (the two 16-token segments sa, sb); every load is issued.
template <int D>
__device__ __forceinline__ void load_rows(RowRegs<D>& r, const bf16* __restrict__ kc,
                                          const bf16* __restrict__ vc, const Seg& sa,
                                          const Seg& sb, int lane) {
  constexpr int CPT = D / 8;
#pragma unroll
  for (int j = 0; j < RowRegs<D>::J; ++j) {
    const int ci = lane + 64 * j;
    const int m = ci / CPT, c = ci % CPT;
    const long long at = (m < kSeg ? sa.base : sb.base) + (long long)(m % kSeg) * D + 8 * c;
    r.k[j] = stream_load(reinterpret_cast<const bf16x8*>(kc + at));
    r.v[j] = stream_load(reinterpret_cast<const bf16x8*>(vc + at));
  }
}

// Stores a tile to LDS at t; unless both segments are full, V rows of
// tokens outside their segment's [lo, hi) are zeroed (their probabilities
// are 0, but the cache slots may hold non-finite values).
template <int D>
__device__ __forceinline__ void store_rows(RowRegs<D>& r, char* t, const Seg& sa, const Seg& sb,
                                           bool full, int lane) {
  typedef RowsTile<D> T;
  constexpr int CPT = D / 8;
#pragma unroll
  for (int j = 0; j < RowRegs<D>::J; ++j) {
    const int ci = lane + 64 * j;
    const int m = ci / CPT, c = ci % CPT;
    *reinterpret_cast<bf16x8*>(t + m * T::K_STRIDE + 16 * c) = r.k[j];
    if (!full) {
      const Seg& sg = m < kSeg ? sa : sb;
      const int tok = sg.t0 + m % kSeg;
      if (tok < sg.lo || tok >= sg.hi) r.v[j] = bf16x8{};
    }
    *reinterpret_cast<bf16x8*>(t + T::K_BYTES + m * T::V_STRIDE + 16 * c) = r.v[j];
  }
}

// Four consecutive V rows r0 .. r0 + 3 of column c0 + (lane & 15) for every
// lane of a 16-lane group, from a V tile stored row by row: source lane j
// of the group addresses row r0 + j / 4, columns c0 + 4 (j % 4) .. + 3, and
// the transposing read hands lane i element i % 4 of source lanes
// 4 k + i / 4, k = 0 .. 3.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
template <int D>
__device__ __forceinline__ bf16x4 v_col4(const char* vbase, int r0, int c0, int lane) {
  const int j = lane & 15;
  const char* a = vbase + (r0 + (j >> 2)) * RowsTile<D>::V_STRIDE + 2 * (c0 + 4 * (j & 3));
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(a));
  return *reinterpret_cast<const bf16x4*>(&v);
}

// LDS: nb tile buffers, the final row log2-LSEs, eight counters (page-check
// flag, tiles stored, two unused, then tiles finished by each compute wave),
// the chunk's block log masses, then the chunk's page ids.
template <int D>
__host__ __device__ constexpr int rows_off_lse(int nb) { return nb * RowsTile<D>::BYTES; }
template <int D>
__host__ __device__ constexpr int rows_off_sync(int nb) { return rows_off_lse<D>(nb) + Geo<D>::LSE_BYTES; }
template <int D>
__host__ __device__ constexpr int rows_off_ell(int nb) { return rows_off_sync<D>(nb) + 32; }
enum { kSyncBad = 0, kSyncReady = 1, kSyncDone = 4 };  // kSyncDone + row tile

// Segment k of a verify item whose token range ends at segment k_end:
// tokens [16 k, min(16 k + 16, L)), empty at and past k_end (the segment
// descriptors of attn_item without the cache address, which only the load
// wave needs).
__device__ __forceinline__ Seg plain_seg(int k, int k_end, int L) {
  Seg s;
  s.base = 0;
  s.pm = 0xffffffffu;
  if (k < k_end) {
    s.t0 = k * kSeg;
    s.lo = s.t0;
    s.hi = min(s.t0 + kSeg, L);
  } else {
    s.t0 = 0;
    s.lo = 0;
    s.hi = 0;
  }
  return s;
}

// Value of lane i ^ 32 and of lane i, in some order: the two halves of the
// wave exchanged (v_permlane32_swap), for reductions over the lane pair that
// shares a row (max and sum are commutative, so the result is that of
// combining x with its partner in either order).
struct LanePair {
  float a, b;
};
__device__ __forceinline__ LanePair lane_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// The same for lane i ^ 16 (v_permlane16_swap).
__device__ __forceinline__ LanePair lane_pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Sum and max over the four lanes i, i ^ 16, i ^ 32, i ^ 48 (the lanes of
// one row in the 16-row tile); every one of them gets the same value.
__device__ __forceinline__ float quad_sum(float x) {
  const LanePair a = lane_pair16(x);
  const LanePair b = lane_pair(a.a + a.b);
  return b.a + b.b;
}
__device__ __forceinline__ float quad_max(float x) {
  const LanePair a = lane_pair16(x);
  const LanePair b = lane_pair(fmaxf(a.a, a.b));
  return fmaxf(b.a, b.b);
}

// The workgroup's counters: raised by one wave, waited on by others.
__device__ __forceinline__ int counter_peek(int* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Waits until *c >= v; false if it gave up after kSpinCap polls (a wait on
// a wave of the same workgroup, which is always resident: never expected).
__device__ __forceinline__ bool counter_wait(int* c, int v) {
  for (int n = 0; n < kSpinCap; ++n) {
    if (__builtin_amdgcn_readfirstlane(counter_peek(c)) >= v) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// HALF: the last row tile holds at most 16 rows (65 to 80 rows in all) and
// runs on 16x16x32 MFMAs (half the matrix work and softmax of a padded
// 32-row tile).  Wave roles: wave 1 loads, waves 0, 2 and 3 compute row
// tiles 0, 1 and 2.  The dispatcher puts the four waves of a workgroup on
// the four SIMDs of a compute unit and the second workgroup on the same
// SIMDs shifted by one wave (MI355X, read from the hardware ids), so SIMD
// k holds wave k of one workgroup and wave k - 1 of the other: this order
// gives each SIMD at most one full and one half row tile, or a row tile and
// a load wave (with the load wave last, two SIMDs carried two full tiles).
template <int D, bool HALF>
__global__ void __launch_bounds__(kRowsThreads, 2) verify_rows_kernel(AttnParams p, int nb) {
  typedef Geo<D> G;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const unsigned item = xcd_item(blockIdx.x, p);
  const int u = (int)(item / (unsigned)p.num_chunks), c = (int)(item % (unsigned)p.num_chunks);
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
  if (p.skip_len >= 0 && p.seq_lens[b] <= p.skip_len) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool loader = w == 1;
  const int rt = w == 0 ? 0 : (w == 2 ? 1 : 2);  // row tile of a compute wave
  const bool half = HALF && rt == 2;
  const int hl = lane >> 5, rl = lane & 31;
  const int R = p.rows;
  // this lane's row: two lanes per row in a 32-row tile (hl), four in the
  // 16-row tile (lane >> 4)
  const int r = half ? 64 + (lane & 15) : rt * 32 + rl;
  const int rsub = half ? (lane >> 4) : hl, rstep = half ? 4 : 2;
  const bool row_ok = !loader && r < R;
  const int iq = row_ok ? r / p.group : 0;
  const int hq = h * p.group + (row_ok ? r % p.group : 0);
  const int chunk = p.chunk_tokens;

  const int L = p.seq_lens[b];
  const bool unit_ok =
      L >= p.n_q && L <= p.max_seq_len && (long long)L <= (long long)p.max_pages * p.page_size;
  if (!unit_ok) {
    // chunk 0 owns the unit's (NaN) outputs
    if (c != 0) return;
    if (row_ok) {
      bf16* o = reinterpret_cast<bf16*>(p.o);
      const long long orow = ((long long)b * p.n_q + iq) * p.num_q_heads + hq;
      for (int d = rsub; d < D; d += rstep) o[orow * D + d] = from_f32<bf16>(qnan());
      if (rsub == 0) p.lse[orow] = qnan();
    }
    for (int j = threadIdx.x; j < p.max_blocks; j += kRowsThreads)
      p.block_scores[(long long)u * p.max_blocks + j] = qnan();
    return;
  }
  const int t_lo = c * chunk;
  if (t_lo >= L) return;  // chunk past this request's length
  const int t_hi = min(t_lo + chunk, L);
  const int seg_lo = t_lo / kSeg, seg_hi = ceil_div(t_hi, kSeg);
  const int n_tiles = ceil_div(seg_hi - seg_lo, 2);
  // a unit that fits in its first chunk is finished here (outputs, scores)
  const bool final_out = p.num_chunks == 1 || (c == 0 && L <= chunk);
  const int blk0 = c * (chunk / p.block_size);
  float* const lse2s = reinterpret_cast<float*>(smem + rows_off_lse<D>(nb));
  int* const sync = reinterpret_cast<int*>(smem + rows_off_sync<D>(nb));
  // the chunk's block log masses, addressed by absolute block index
  float* const ell_s = reinterpret_cast<float*>(smem + rows_off_ell<D>(nb)) - (ptrdiff_t)blk0 * R;
  int* const pages_s = reinterpret_cast<int*>(
      smem + rows_off_ell<D>(nb) + ((chunk / p.block_size) * R * 4 + 15) / 16 * 16);
  if (threadIdx.x < 8) sync[threadIdx.x] = 0;
  __syncthreads();

  // Tile j goes through LDS buffer j % nb.  The load wave stores it once
  // every compute wave has finished tile j - nb (each wave counts its own
  // finished tiles: the waves run at different speeds, and a shared count
  // would let two waves that are ahead stand in for one still reading the
  // buffer) and then raises kSyncReady to j + 1; a compute wave starts tile
  // j once kSyncReady > j and raises its counter when its LDS reads of the
  // tile are complete.  The load wave thus runs up to nb tiles ahead of the
  // slowest compute wave (plus the kLoadSlots tiles in its registers), and
  // no wave waits at a per-tile barrier for the others.
  int fail = 0;
  bool bad = false;
  if (loader) {
    const bf16* __restrict__ kc = reinterpret_cast<const bf16*>(p.k);
    const bf16* __restrict__ vc = reinterpret_cast<const bf16*>(p.v);
    const FastDiv pdiv(p.page_size);
    int bad = 0;
    // the chunk's page ids, staged in LDS once: the tile loop then issues
    // no vector memory reads but the tiles' (a page-id load in the loop
    // made the compiler wait for every outstanding tile load where the id
    // was used)
    const int pg0 = t_lo / p.page_size;
    const int npg = (t_hi - 1) / p.page_size - pg0 + 1;
    for (int i = lane; i < npg; i += 64)
      pages_s[i] = p.page_table[(long long)b * p.max_pages + pg0 + i];
    wave_lds_sync();
    // descriptor of segment k (one per lane, as seg_lane + seg_resolve): an
    // empty segment reads page 0; a page id outside [0, num_pages) also
    // reads page 0 and sets `bad`
    auto lane_seg = [&](int k) {
      SegLane d;
      d.pm = 0xffffffffu;
      int t0 = 0, lo = 0, hi = 0;
      if (k < seg_hi) {
        t0 = k * kSeg;
        lo = t0;
        hi = min(t0 + kSeg, L);
      }
      d.t0 = t0;
      d.lohi = lo < hi ? ((lo - t0) | ((hi - t0) << 8)) : 0;
      int pg = 0;
      if (d.lohi != 0) {
        pg = pages_s[pdiv.div(t0) - pg0];
        if (pg < 0 || pg >= p.num_pages) {
          bad = 1;
          pg = 0;
        }
      }
      d.pg = pg;
      d.row = (pg * p.num_kv_heads + h) * p.page_size + pdiv.mod(t0);
      return d;
    };
    SegLane cur = lane_seg(seg_lo + lane);
    SegLane nxt = lane_seg(seg_lo + 64 + lane);
    int cur_batch = 0;
    RowRegs<D> regs[kLoadSlots];
    Seg sa[kLoadSlots], sb[kLoadSlots];
    // tile j in register slot j % kLoadSlots; empty segments past the item
    // read page 0 (every load is issued)
#pragma unroll
    for (int q = 0; q < kLoadSlots; ++q) {
      sa[q] = seg_of(p, cur, nxt, false, 2 * q);
      sb[q] = seg_of(p, cur, nxt, false, 2 * q + 1);
      load_rows<D>(regs[q], kc, vc, sa[q], sb[q], lane);
    }
    // Every trip handles all kLoadSlots slots, and each slot's next loads are
    // issued unconditionally (past the item they read an empty segment of
    // page 0, which stays cached): the compiler's count of the loads issued
    // after a slot's is then the same on every path.  With a break or a
    // conditional load in the trip it merged in paths on which fewer loads
    // followed and waited for all but one tile's loads before every store:
    // one tile in flight instead of three.
    int buf = 0;
    for (int t0 = 0; t0 < n_tiles; t0 += kLoadSlots)
#pragma unroll
      for (int q = 0; q < kLoadSlots; ++q) {
        const int j = t0 + q;
        const int rel0 = 2 * j;
        if (rel0 > 0 && (rel0 & 63) == 0) {
          // move to the next batch of descriptors; make the one after it
          cur = nxt;
          ++cur_batch;
          nxt = lane_seg(seg_lo + 64 * (cur_batch + 1) + lane);
        }
        if (j < n_tiles) {
          // tile j - 1, stored an iteration ago, is complete in LDS by now:
          // publish it (waiting for the writes right after issuing them kept
          // this wave at the fence for most of each tile)
          if (j > 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            if (lane == 0)
              __hip_atomic_store(&sync[kSyncReady], j, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          if (j >= nb) {
#pragma unroll
            for (int k = 0; k < kRowWaves; ++k)
              if (!counter_wait(&sync[kSyncDone + k], j - nb + 1)) fail = 1;
          }
          store_rows<D>(regs[q], smem + buf * RowsTile<D>::BYTES, sa[q], sb[q],
                        seg_full(sa[q]) && seg_full(sb[q]), lane);
          buf = buf + 1 == nb ? 0 : buf + 1;
        }
        const int ra = 2 * (j + kLoadSlots), rb = ra + 1;
        sa[q] = seg_of(p, cur, nxt, (ra >> 6) != cur_batch, ra & 63);
        sb[q] = seg_of(p, cur, nxt, (rb >> 6) != cur_batch, rb & 63);
        load_rows<D>(regs[q], kc, vc, sa[q], sb[q], lane);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0)
      __hip_atomic_store(&sync[kSyncReady], n_tiles, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // every page id of the item has been checked (the vote over all lanes
    // first: a ballot inside the lane-0 branch would see lane 0 only)
    const bool any_bad = __builtin_amdgcn_ballot_w64(bad != 0) != 0ull;
    if (lane == 0 && any_bad) sync[kSyncBad] = 1;
    // (the compute waves' matching barrier follows their tile loop)
    fail = __syncthreads_or(fail);
  } else if (half) {
    // ---- the 16-row tile (rows 64 .. R - 1), 16x16x32 MFMAs: lane group
    // g = lane >> 4 holds tokens 4g .. 4g + 3 of each 16-token segment of
    // row 64 + (lane & 15) in S^T, and d rows 4g .. 4g + 3 of each 16-row
    // tile of O^T ----
    const int g = lane >> 4, jr = lane & 15;
    constexpr int KS2 = D / 32;  // k-steps of S^T = K Q^T
    constexpr int DT = D / 16;   // 16-row tiles of O^T
    // Q^T operand: row jr, d [32 ks + 8 g, 32 ks + 8 g + 8); a negative
    // scale is folded in as an exact sign flip
    bf16x8 q16[KS2];
    {
      const bf16* qrow = row_ok ? reinterpret_cast<const bf16*>(p.q) +
                                      (((long long)b * p.n_q + iq) * p.num_q_heads + hq) * D
                                : nullptr;
      const bool neg = p.scale_log2 < 0.f;
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) {
        uint4 v = {0u, 0u, 0u, 0u};
        if (qrow) v = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
        if (neg) {
          v.x ^= 0x80008000u;
          v.y ^= 0x80008000u;
          v.z ^= 0x80008000u;
          v.w ^= 0x80008000u;
        }
        q16[ks] = *reinterpret_cast<const bf16x8*>(&v);
      }
    }
    const int pos_r = L - p.n_q + iq;
    const int pos_min = L - p.n_q;
    const float scl = fmaxf(fabsf(p.scale_log2), 1e-30f);
    const FastDiv bdiv(p.block_size);
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = neg_inf(), l_run = 0.f, blk_run = 0.f;
    int buf = 0;
    for (int t = 0; t < n_tiles; ++t) {
      if (!counter_wait(&sync[kSyncReady], t + 1)) fail = 1;
      const char* gt = smem + buf * RowsTile<D>::BYTES;
      buf = buf + 1 == nb ? 0 : buf + 1;
      const int ka = seg_lo + 2 * t;
      const Seg ca = plain_seg(ka, seg_hi, L), cb = plain_seg(ka + 1, seg_hi, L);
      const bool interior = seg_full(ca) && seg_full(cb) && cb.t0 + kSeg - 1 <= pos_min;
      // S^T of the tile's two 16-token segments
      bf16x8 kf[2][KS2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int ks = 0; ks < KS2; ++ks)
          kf[hh][ks] = *reinterpret_cast<const bf16x8*>(gt + (16 * hh + jr) * G::K_STRIDE +
                                                         64 * ks + 16 * g);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 sv[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        sv[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS2; ++ks)
          sv[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[hh][ks], q16[ks], sv[hh], 0, 0, 0);
      }
      if (!interior) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const Seg& sg = hh ? cb : ca;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = sg.t0 + 4 * g + e;
            if (!(tok >= sg.lo && tok < sg.hi && tok <= pos_r)) sv[hh][e] = neg_inf();
          }
        }
      }
      float mx = neg_inf();
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sv[hh][e]);
      mx = quad_max(mx) * scl;
      const float m_new = fmaxf(m_run, mx);
      const bool move = (m_run == neg_inf()) || (m_new > m_run + kRescaleSlack);
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float m_tgt = move ? m_new : m_run;
        const float alpha = (m_tgt == neg_inf()) ? 1.f : fast_exp2(m_run - m_tgt);
        l_run *= alpha;
        blk_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[dt][e] *= alpha;
        m_run = m_tgt;
      }
      const float m_use = (m_run == neg_inf()) ? 0.f : m_run;
      // V^T operand of O^T tile dt: d row 16 dt + jr, tokens 4g .. 4g + 3 and
      // 16 + 4g .. 16 + 4g + 3 (the k order of this lane's probabilities)
      const char* vt = gt + RowsTile<D>::K_BYTES;
      bf16x8 vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x4 lo4 = v_col4<D>(vt, 4 * g, 16 * dt, lane);
        const bf16x4 hi4 = v_col4<D>(vt, 16 + 4 * g, 16 * dt, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[dt][e] = lo4[e];
          vf[dt][4 + e] = hi4[e];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      float pr[8];
      float psum = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[4 * hh + e] = fast_exp2(fmaf(sv[hh][e], scl, -m_use));
          psum += pr[4 * hh + e];
        }
      l_run += psum;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = static_cast<bf16>(pr[e]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pb, o[dt], 0, 0, 0);
      // the tile's LDS reads are complete: its buffer may be refilled
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0)
        __hip_atomic_fetch_add(&sync[kSyncDone + rt], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // per-block log mass of this row, frame m_use
      if (p.block_size == kSeg) {
        const float sa0 = quad_sum(pr[0] + pr[1] + pr[2] + pr[3]);
        const float sb0 = quad_sum(pr[4] + pr[5] + pr[6] + pr[7]);
        if (row_ok && g == 0 && ca.lo < ca.hi)
          ell_s[(ca.t0 / kSeg) * R + r] = m_use + fast_log2(sa0);
        if (row_ok && g == 1 && cb.lo < cb.hi)
          ell_s[(cb.t0 / kSeg) * R + r] = m_use + fast_log2(sb0);
      } else {
        blk_run += psum;
        const int tile_end = ca.t0 + 2 * kSeg;
        if (bdiv.mod(tile_end) == 0 || ka + 2 >= seg_hi) {
          const float tot = quad_sum(blk_run);
          if (row_ok && g == 0) ell_s[bdiv.div(ca.t0) * R + r] = m_use + fast_log2(tot);
          blk_run = 0.f;
        }
      }
    }
    l_run = quad_sum(l_run);
    // (the load wave's matching barrier follows its tile loop)
    fail = __syncthreads_or(fail);
    bad = fail || sync[kSyncBad] != 0;
    if (row_ok) {
      const bool empty = !(l_run > 0.f);
      const float inv = empty ? 0.f : 1.f / l_run;
      const float lse2 = bad ? qnan() : (empty ? neg_inf() : m_run + fast_log2(l_run));
      const float poison = bad ? qnan() : 1.f;
      if (final_out) {
        const long long orow = ((long long)b * p.n_q + iq) * p.num_q_heads + hq;
        bf16* out = reinterpret_cast<bf16*>(p.o) + orow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = from_f32<bf16>(o[dt][e] * inv * poison);
          *reinterpret_cast<bf16x4*>(out + 16 * dt + 4 * g) = v4;
        }
        if (g == 0) {
          p.lse[orow] = lse2 * kLn2;
          lse2s[r] = lse2;
        }
      } else {
        const long long prow = (long long)u * p.num_chunks * R + (long long)c * R + r;
        float* op = p.o_part + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o[dt][e] * inv * poison;
          *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = v4;
        }
        if (g == 0) p.lse_part[prow] = lse2;
      }
    }
  } else {
    // ---- compute waves of 32-row tiles: row tile rt, Q rows in registers ----
    bf16x8 qreg[G::KS];
    load_qreg<D>(qreg,
                 row_ok ? reinterpret_cast<const bf16*>(p.q) +
                              (((long long)b * p.n_q + iq) * p.num_q_heads + hq) * D
                        : nullptr,
                 p.scale_log2 < 0.f);
    const int pos_r = L - p.n_q + iq;
    const int pos_min = L - p.n_q;  // smallest causal limit of the unit's rows
    const float scl = fmaxf(fabsf(p.scale_log2), 1e-30f);
    const FastDiv bdiv(p.block_size);
    Acc<D> a;
    acc_init(a);
    float blk_run = 0.f;
    int buf = 0;
    for (int t = 0; t < n_tiles; ++t) {
      if (!counter_wait(&sync[kSyncReady], t + 1)) fail = 1;
      const char* gt = smem + buf * RowsTile<D>::BYTES;
      buf = buf + 1 == nb ? 0 : buf + 1;
      const int ka = seg_lo + 2 * t;
      const Seg ca = plain_seg(ka, seg_hi, L), cb = plain_seg(ka + 1, seg_hi, L);
      const bool interior = seg_full(ca) && seg_full(cb) && cb.t0 + kSeg - 1 <= pos_min;
      // S^T = K Q^T, the tile's K fragments read before the MFMAs
      bf16x8 kf[G::KS];
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8*>(gt + rl * G::K_STRIDE + 32 * ks + 16 * hl);
      // (the scheduler would otherwise sink each read to its MFMA: one LDS
      // round trip per k-step)
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qreg[ks], sacc, 0, 0, 0);
      // masked logits in place (interior tiles need no mask), row max
      float mx = neg_inf();
      if (!interior) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = (i >> 2) * 8 + 4 * hl + (i & 3);
          const Seg& sg = (m < kSeg) ? ca : cb;
          const int tok = sg.t0 + (m % kSeg);
          if (!(tok >= sg.lo && tok < sg.hi && tok <= pos_r)) sacc[i] = neg_inf();
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      // online softmax, log2 domain, lazy rescaling (as attn_item)
      const LanePair mp = lane_pair(mx);
      mx = fmaxf(mp.a, mp.b) * scl;
      const float m_new = fmaxf(a.m, mx);
      const bool move = (a.m == neg_inf()) || (m_new > a.m + kRescaleSlack);
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float m_tgt = move ? m_new : a.m;
        const float alpha = (m_tgt == neg_inf()) ? 1.f : fast_exp2(a.m - m_tgt);
        a.l *= alpha;
        blk_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) a.o[mt][i] *= alpha;
        a.m = m_tgt;
      }
      const float m_use = (a.m == neg_inf()) ? 0.f : a.m;
      // the tile's V^T fragments read before the PV MFMAs
      // (lane (rl, hl), k-step kk: d row 32 mt + rl, tokens 16 kk + 4 hl ..
      // + 3 and 16 kk + 8 + 4 hl .. + 3, the k order of pr[8 kk ..])
      const char* vt = gt + RowsTile<D>::K_BYTES;
      bf16x8 vf[2][G::MT];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
          const int c0 = 32 * mt + 16 * ((lane >> 4) & 1);
          const bf16x4 lo4 = v_col4<D>(vt, 16 * kk + 4 * hl, c0, lane);
          const bf16x4 hi4 = v_col4<D>(vt, 16 * kk + 8 + 4 * hl, c0, lane);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vf[kk][mt][e] = lo4[e];
            vf[kk][mt][4 + e] = hi4[e];
          }
        }
      __builtin_amdgcn_sched_barrier(0);
      float pr[16];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pr[i] = fast_exp2(fmaf(sacc[i], scl, -m_use));
        psum += pr[i];
      }
      a.l += psum;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pb;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pb[jj] = static_cast<bf16>(pr[8 * kk + jj]);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
          a.o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk][mt], pb, a.o[mt], 0, 0, 0);
      }
      // the tile's LDS reads are complete: its buffer may be refilled
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0)
        __hip_atomic_fetch_add(&sync[kSyncDone + rt], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // per-block log mass of this row, frame m_use
      if (p.block_size == kSeg) {
        float sa0 = 0.f, sb0 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sa0 += pr[i];
#pragma unroll
        for (int i = 8; i < 16; ++i) sb0 += pr[i];
        const LanePair pa = lane_pair(sa0), pb2 = lane_pair(sb0);
        const Seg& mine = hl ? cb : ca;
        if (row_ok && mine.lo < mine.hi)
          ell_s[(mine.t0 / kSeg) * R + r] = m_use + fast_log2(hl ? pb2.a + pb2.b : pa.a + pa.b);
      } else {
        blk_run += psum;
        const int tile_end = ca.t0 + 2 * kSeg;
        if (bdiv.mod(tile_end) == 0 || ka + 2 >= seg_hi) {
          const LanePair bp = lane_pair(blk_run);
          if (row_ok && hl == 0) ell_s[bdiv.div(ca.t0) * R + r] = m_use + fast_log2(bp.a + bp.b);
          blk_run = 0.f;
        }
      }
    }
    const LanePair lp = lane_pair(a.l);
    a.l = lp.a + lp.b;
    // (the load wave's matching barrier follows its tile loop)
    fail = __syncthreads_or(fail);
    // a failed wait (never expected) poisons the unit like a bad page id
    bad = fail || sync[kSyncBad] != 0;
    if (row_ok) {
    if (final_out) {
      const long long orow = ((long long)b * p.n_q + iq) * p.num_q_heads + hq;
      const float lse2 = write_row<D>(a, reinterpret_cast<bf16*>(p.o), p.lse, orow, bad, hl);
      if (hl == 0) lse2s[r] = lse2;
    } else {
      const bool empty = !(a.l > 0.f);
      const float inv = empty ? 0.f : 1.f / a.l;
      const float lse2 = bad ? qnan() : (empty ? neg_inf() : a.m + fast_log2(a.l));
      const float poison = bad ? qnan() : 1.f;
      const long long prow = (long long)u * p.num_chunks * R + (long long)c * R + r;
      float* op = p.o_part + prow * D;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = a.o[mt][4 * q4 + e] * inv * poison;
          *reinterpret_cast<f32x4*>(op + 32 * mt + 8 * q4 + 4 * hl) = v4;
        }
      if (hl == 0) p.lse_part[prow] = lse2;
    }
    }
  }
  bad = fail || sync[kSyncBad] != 0;

  // ---- every wave: block scores of a whole unit, or the chunk's block log
  // masses to the workspace for the split merge ----
  if (final_out) {
    __syncthreads();
    const int nblk = ceil_div(L, p.block_size);
    const int r0 = p.score_row_start * p.group;
    for (int j = threadIdx.x; j < p.max_blocks; j += kRowsThreads) {
      float sc = 0.f;
      if (j < nblk) {
        const float* e = ell_s + (long long)j * R;
        for (int rr = r0; rr < R; ++rr) sc += fast_exp2(e[rr] - lse2s[rr]);
      }
      p.block_scores[(long long)u * p.max_blocks + j] = bad ? qnan() : sc;
    }
  } else {
    float* const ell_u = p.ell + (long long)u * p.max_blocks * R;
    const int blk_end = ceil_div(min((c + 1) * chunk, L), p.block_size);
    for (int i = blk0 * R + threadIdx.x; i < blk_end * R; i += kRowsThreads) ell_u[i] = ell_s[i];
  }
}

}  // namespace

// LDS bytes after the tile buffers' part: block log masses and page ids of
// a chunk
size_t rows_tail_bytes(long long ell_floats, int chunk_tokens, int page_size) {
  return (size_t)(ell_floats * 4 + 15) / 16 * 16 + ((size_t)chunk_tokens / page_size + 2) * 4;
}
// LDS tile buffers of a workgroup: as many as fit (up to kMaxTileBufs) with
// two workgroups per compute unit; 0 when not even two fit.
int verify_rows_bufs(int head_dim, long long ell_floats, int chunk_tokens, int page_size) {
  for (int nb = kMaxTileBufs; nb >= 2; --nb) {
    const size_t off = head_dim == 64 ? (size_t)rows_off_ell<64>(nb) : (size_t)rows_off_ell<128>(nb);
    if (off + rows_tail_bytes(ell_floats, chunk_tokens, page_size) <= kMaxLds / 2) return nb;
  }
  return 0;
}

bool verify_rows_fits_shape(int head_dim, int rows, int block_size, int page_size,
                            int chunk_tokens) {
  if (ceil_div(rows, 32) != kRowWaves || page_size < 1) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  if (block_size < kSeg || (block_size != kSeg && block_size % (2 * kSeg) != 0)) return false;
  if (chunk_tokens <= 0 || chunk_tokens % (2 * kSeg) != 0 || chunk_tokens % block_size != 0)
    return false;
  const long long ellf = (long long)(chunk_tokens / block_size) * rows;
  return verify_rows_bufs(head_dim, ellf, chunk_tokens, page_size) > 0;
}

bool verify_rows_fits(const AttnParams& p) {
  return verify_rows_fits_shape(p.head_dim, p.rows, p.block_size, p.page_size, p.chunk_tokens);
}

hipError_t launch_verify_rows(const AttnParams& p, hipStream_t s) {
  if (!verify_rows_fits(p)) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((long long)p.batch * p.num_kv_heads * p.num_chunks);
  if (grid == 0) return hipSuccess;
  const long long ellf = (long long)(p.chunk_tokens / p.block_size) * p.rows;
  const int nb = verify_rows_bufs(p.head_dim, ellf, p.chunk_tokens, p.page_size);
  const size_t smem =
      (p.head_dim == 64 ? (size_t)rows_off_ell<64>(nb) : (size_t)rows_off_ell<128>(nb)) +
      rows_tail_bytes(ellf, p.chunk_tokens, p.page_size);
  auto go = [&](auto kern) -> hipError_t {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kRowsThreads), smem, s, p, nb);
    return hipGetLastError();
  };
  // at most 16 rows in the last row tile: the 16x16x32 form of that tile
  if (p.rows <= 2 * 32 + 16)
    return p.head_dim == 128 ? go(verify_rows_kernel<128, true>) : go(verify_rows_kernel<64, true>);
  return p.head_dim == 128 ? go(verify_rows_kernel<128, false>) : go(verify_rows_kernel<64, false>);
}

}  // namespace sss
