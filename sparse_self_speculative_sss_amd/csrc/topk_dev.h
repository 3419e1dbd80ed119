// Top-N block selection of one (request, KV head) unit as a workgroup-level
// device routine (SparseSpec §4.1: Top-K over the aggregated block scores).
// Used by the stand-alone selection kernel and by the fused step kernel.
//
// Every exchange between threads goes through LDS, so the routines meet at
// LDS-only barriers (a selection's global reads and writes in flight are
// never waited for at a barrier).
//
// Exact radix select on 32-bit order-preserving keys of the fp32 scores:
// four 8-bit MSB-first histogram passes find the N-th largest key T; the
// blocks with key > T are taken, plus the lowest-index blocks with key == T
// until N are taken.  Histograms count with LDS integer atomics (order
// independent), ranks come from prefix sums in index order, so the
// selection is bit-exact and deterministic.  Output is ascending: each
// thread emits a contiguous range of candidates at offsets from two
// workgroup prefix sums (ties before it, selections before it).
#pragma once

#include "sss_common.h"

namespace sss {

// Monotone map of an fp32 score to uint32 (larger score -> larger key);
// -0.0 is folded onto +0.0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Candidates of a unit (blocks that start before the window) and the number
// of blocks it selects.
__device__ __forceinline__ void topk_bounds(int L, int bs, int window, int max_blocks, int budget,
                                            int max_sel, int& ncand, int& n) {
  if (L < 0) L = 0;
  const long long nblk = ((long long)L + bs - 1) / bs;
  const int ws = window_start(L, window);
  long long c = ((long long)ws + bs - 1) / bs;
  if (c > nblk) c = nblk;
  if (c > max_blocks) c = max_blocks;
  ncand = (int)c;
  n = budget < 0 ? 0 : budget;
  if (n > ncand) n = ncand;
  if (n > max_sel) n = max_sel;
}

// histogram bins of a radix digit (8 bits)
constexpr int kTopkBins = 256;
// LDS words topk_select needs.
constexpr int kTopkLdsWords = kTopkBins + 16 + 2;
// scores loaded per thread before they are used
constexpr int kTopkBatch = 8;

// Exclusive prefix sum of v over the workgroup in thread order, and the
// total.  `scratch` holds NT / 64 ints.
template <int NT>
__device__ __forceinline__ int wg_exclusive_sum(int v, int* scratch, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  lds_barrier();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = scratch[w];
    if (w < wave) before += c;
    total += c;
  }
  lds_barrier();
  return before + incl - v;
}

// hist[bin] += 1 for every lane with `act`.  Scores crowd into few bins
// (one histogram bin spans two binades in the first pass), and LDS atomics
// to one address serialise lane by lane, so the two most common bins among
// the wave's first active lanes are counted with one atomic each and only
// the remaining lanes add one by one.
__device__ __forceinline__ void hist_count(int* hist, bool act, uint32_t bin) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const unsigned long long am = __ballot(act);
    if (am == 0) return;
    const int leader = __builtin_ctzll(am);
    const uint32_t b0 = __builtin_amdgcn_readlane(bin, leader);
    const bool same = act && bin == b0;
    const unsigned long long sm = __ballot(same);
    if ((threadIdx.x & 63) == leader) atomicAdd(&hist[b0], (int)__popcll(sm));
    act = act && !same;
  }
  if (act) atomicAdd(&hist[bin], 1);
}

// Where the selection reads its keys: the fp32 scores themselves, or their
// keys parked in LDS.
struct ScoreSrc {
  const float* sc;
  __device__ __forceinline__ uint32_t operator()(int j) const { return score_key(sc[j]); }
};
struct KeySrc {
  const uint32_t* k;
  __device__ __forceinline__ uint32_t operator()(int j) const { return k[j]; }
};

// Radix select and ascending emission over keys key(0 .. ncand-1), with
// 0 < n < ncand.  `B` keys are read per thread before they are used.
template <int NT, int B, typename Src, bool OUT = true>
__device__ void topk_core(Src key, int ncand, int n, int32_t* __restrict__ out, int32_t* out_lds,
                          int* lds) {
  int* hist = lds;
  int* scan_scratch = lds + kTopkBins;
  int* s_digit = lds + kTopkBins + 16;
  int* s_rem = lds + kTopkBins + 17;
  const int tid = threadIdx.x;
  constexpr int PT = (kTopkBins + NT - 1) / NT;  // bins per thread in the digit search

  // ---- radix select of the n-th largest key: four 8-bit digits ----
  uint32_t prefix = 0, pmask = 0;
  int rem = n;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t dmask = 255u;
    for (int i = tid; i < kTopkBins; i += NT) hist[i] = 0;
    lds_barrier();
    // indices past the end re-read the last key and count nothing
    for (int j0 = tid; j0 < ncand; j0 += B * NT) {
      uint32_t k[B];
#pragma unroll
      for (int e = 0; e < B; ++e) k[e] = key(min(j0 + e * NT, ncand - 1));
#pragma unroll
      for (int e = 0; e < B; ++e)
        hist_count(hist, j0 + e * NT < ncand && (k[e] & pmask) == prefix, (k[e] >> shift) & dmask);
    }
    lds_barrier();
    // the digit holding the rem-th largest key: bins in descending order,
    // PT consecutive ones per thread
    int c[PT], local = 0;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int bin = kTopkBins - 1 - (tid * PT + i);
      c[i] = bin >= 0 ? hist[bin] : 0;
      local += c[i];
    }
    int tot;
    const int excl = wg_exclusive_sum<NT>(local, scan_scratch, tot);
    if (excl < rem && rem <= excl + local) {
      int cum = excl;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        if (cum + c[i] >= rem) {
          *s_digit = kTopkBins - 1 - (tid * PT + i);
          *s_rem = rem - cum;
          break;
        }
        cum += c[i];
      }
    }
    lds_barrier();
    prefix |= (uint32_t)*s_digit << shift;
    pmask |= dmask << shift;
    rem = *s_rem;
    lds_barrier();
  }
  const uint32_t T = prefix;
  const int need_eq = rem;

  // ---- ascending emission: thread t owns candidates [t*per, (t+1)*per);
  // an odd `per` keeps the lanes of a wave on distinct LDS banks ----
  const int per = ((ncand + NT - 1) / NT) | 1;
  const int j0 = min(tid * per, ncand), j1 = min(j0 + per, ncand);
  int n_gt = 0, n_eq = 0;
  for (int jb = j0; jb < j1; jb += B) {
    uint32_t k[B];
#pragma unroll
    for (int e = 0; e < B; ++e) k[e] = key(min(jb + e, j1 - 1));
#pragma unroll
    for (int e = 0; e < B; ++e)
      if (jb + e < j1) {
        n_gt += k[e] > T;
        n_eq += k[e] == T;
      }
  }
  int tot;
  const int eq_before = wg_exclusive_sum<NT>(n_eq, scan_scratch, tot);
  // ties are taken lowest index first: this thread's share of the need_eq
  const int eq_take = min(max(need_eq - eq_before, 0), n_eq);
  int pos = wg_exclusive_sum<NT>(n_gt + eq_take, scan_scratch, tot);
  int eq_seen = 0;
  for (int jb = j0; jb < j1; jb += B) {
    uint32_t k[B];
#pragma unroll
    for (int e = 0; e < B; ++e) k[e] = key(min(jb + e, j1 - 1));
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const int j = jb + e;
      if (j >= j1) break;
      bool take = k[e] > T;
      if (k[e] == T) take = eq_seen++ < eq_take;
      if (take) {
        if constexpr (OUT) out[pos] = j;
        if (out_lds) out_lds[pos] = j;
        ++pos;
      }
    }
  }
  lds_barrier();
}

// The n largest of sc[0, ncand) (ties to the lower index), ascending, into
// out[0, n); out[n, max_sel) = -1 (OUT = false: no global output, out is
// not touched).  When out_lds is given, out_lds[0, n) receives the same
// list.  `lds` holds kTopkLdsWords ints.  With `keys`
// (LDS room for keys_cap words) and ncand <= keys_cap, the keys are read
// from global memory once and parked there for the passes.  All NT threads
// of the workgroup call it; it ends with a barrier.
template <int NT, bool OUT = true>
__device__ void topk_select(const float* sc, int ncand, int n, int32_t* __restrict__ out,
                            int max_sel, int32_t* out_lds, int* lds, uint32_t* keys = nullptr,
                            int keys_cap = 0) {
  static_assert(NT % 64 == 0 && NT >= 64 && NT <= 1024, "workgroup of whole waves");
  const int tid = threadIdx.x;

  // every candidate kept, or none: the list is 0..n-1; otherwise positions
  // [0, n) are written by the emission
  for (int j = tid; OUT && j < max_sel; j += NT) {
    if (n == ncand)
      out[j] = j < n ? j : -1;
    else if (j >= n)
      out[j] = -1;
  }
  if (n == 0 || n == ncand) {
    if (out_lds)
      for (int j = tid; j < n; j += NT) out_lds[j] = j;
    lds_barrier();
    return;
  }
  if (keys && ncand <= keys_cap) {
    for (int j0 = tid; j0 < ncand; j0 += kTopkBatch * NT) {
      float x[kTopkBatch];
#pragma unroll
      for (int e = 0; e < kTopkBatch; ++e) x[e] = sc[min(j0 + e * NT, ncand - 1)];
#pragma unroll
      for (int e = 0; e < kTopkBatch; ++e)
        if (j0 + e * NT < ncand) keys[j0 + e * NT] = score_key(x[e]);
    }
    lds_barrier();
    topk_core<NT, 4, KeySrc, OUT>(KeySrc{keys}, ncand, n, out, out_lds, lds);
  } else {
    topk_core<NT, kTopkBatch, ScoreSrc, OUT>(ScoreSrc{sc}, ncand, n, out, out_lds, lds);
  }
}

// topk_select over keys already parked in LDS (keys[0, ncand), score_key of
// each score), e.g. by the routine that computed the scores.
template <int NT>
__device__ void topk_select_parked(const uint32_t* keys, int ncand, int n,
                                   int32_t* __restrict__ out, int max_sel, int32_t* out_lds,
                                   int* lds) {
  static_assert(NT % 64 == 0 && NT >= 64 && NT <= 1024, "workgroup of whole waves");
  const int tid = threadIdx.x;
  for (int j = tid; j < max_sel; j += NT) {
    if (n == ncand)
      out[j] = j < n ? j : -1;
    else if (j >= n)
      out[j] = -1;
  }
  if (n == 0 || n == ncand) {
    if (out_lds)
      for (int j = tid; j < n; j += NT) out_lds[j] = j;
    lds_barrier();
    return;
  }
  topk_core<NT, 4>(KeySrc{keys}, ncand, n, out, out_lds, lds);
}

// ---- one-wave selection ----
//
// The same selection as topk_select (the n largest keys, lowest index first
// among equal ones, emitted ascending) made by a single wave with no
// workgroup barrier: for units of at most 64 * KPL candidates the
// workgroup version's ~25 barriers and their dependent LDS round trips set
// its latency, which a persistent workgroup pays per unit.  Lane l owns
// candidates [l * KPL, (l + 1) * KPL) in registers.  Radix passes over
// 8-bit digits (MSB first) count the keys still matching the prefix in a
// 256-bin LDS histogram (LDS operations of one wave complete in issue
// order), a wave scan over the bins in descending order finds the digit of
// the rem-th largest key, and the search stops as soon as that digit's bin
// is taken whole.  Emission compares masked keys with the prefix: greater
// ones are taken, and the first `rem` equal ones (by index).

// Inclusive scan of v over the wave's lanes in lane order.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  return v;
}

// The n largest of key(0 .. ncand-1) (0 < n < ncand <= 64 * KPL; `key` as
// for topk_core), ascending into out[0, n) and, if given, out_lds[0, n).
// `hist` is 256 ints of LDS (16-byte aligned) owned by this wave.  Called
// by one whole wave.
template <int KPL, typename Src>
__device__ __forceinline__ void topk_wave_core(Src key, int ncand, int n, int32_t* __restrict__ out,
                               int32_t* out_lds, int* hist) {
  const int lane = threadIdx.x & 63;
  const int j0 = lane * KPL;
  uint32_t k[KPL];
#pragma unroll
  for (int e = 0; e < KPL; ++e) k[e] = key(min(j0 + e, ncand - 1));
  bool live[KPL];
#pragma unroll
  for (int e = 0; e < KPL; ++e) live[e] = j0 + e < ncand;

  uint32_t prefix = 0, pmask = 0;
  int rem = n;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    *reinterpret_cast<int4*>(hist + 4 * lane) = int4{0, 0, 0, 0};
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < KPL; ++e)
      if (live[e] && (k[e] & pmask) == prefix) atomicAdd(&hist[(k[e] >> shift) & 255u], 1);
    wave_lds_sync();
    // lane l holds bins 255 - 4l .. 252 - 4l (descending)
    const int4 h4 = *reinterpret_cast<const int4*>(hist + 252 - 4 * lane);
    const int c0 = h4.w, c1 = h4.z, c2 = h4.y, c3 = h4.x;
    const int local = c0 + c1 + c2 + c3;
    const int incl = wave_inclusive_sum(local);
    const int excl = incl - local;
    // the lane whose bins hold the rem-th largest
    const bool here = excl < rem && rem <= incl;
    const unsigned long long hm = __ballot(here);
    const int src = __builtin_ctzll(hm);
    int cum = excl, digit = 0, cnt = 0;
    if (cum + c0 >= rem) {
      digit = 255 - 4 * lane;
      cnt = c0;
    } else if ((cum += c0) + c1 >= rem) {
      digit = 254 - 4 * lane;
      cnt = c1;
    } else if ((cum += c1) + c2 >= rem) {
      digit = 253 - 4 * lane;
      cnt = c2;
    } else {
      cum += c2;
      digit = 252 - 4 * lane;
      cnt = c3;
    }
    const int d = __builtin_amdgcn_readlane(digit, src);
    const int r = rem - __builtin_amdgcn_readlane(cum, src);
    const int c = __builtin_amdgcn_readlane(cnt, src);
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
    rem = r;
    wave_lds_sync();  // every lane has read the bins before the next pass clears them
    if (c == r) break;  // every key of this bin is taken
  }
  // ---- ascending emission ----
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < KPL; ++e)
    if (live[e]) {
      const uint32_t m = k[e] & pmask;
      n_gt += m > prefix;
      n_eq += m == prefix;
    }
  const int eq_incl = wave_inclusive_sum(n_eq);
  const int eq_take = min(max(rem - (eq_incl - n_eq), 0), n_eq);
  const int take = n_gt + eq_take;
  int pos = wave_inclusive_sum(take) - take;
  int eq_seen = 0;
#pragma unroll
  for (int e = 0; e < KPL; ++e)
    if (live[e]) {
      const uint32_t m = k[e] & pmask;
      bool t = m > prefix;
      if (m == prefix) t = eq_seen++ < eq_take;
      if (t) {
        out[pos] = j0 + e;
        if (out_lds) out_lds[pos] = j0 + e;
        ++pos;
      }
    }
  wave_lds_sync();
}

// topk_select for one wave (ncand <= 64 * KPL candidates; keys from `key`):
// out[0, n) ascending, out[n, max_sel) = -1, out_lds[0, n) if given.
template <int KPL, typename Src>
__device__ __forceinline__ void topk_wave(Src key, int ncand, int n, int32_t* __restrict__ out, int max_sel,
                          int32_t* out_lds, int* hist) {
  const int lane = threadIdx.x & 63;
  for (int j = lane; j < max_sel; j += 64) {
    if (n == ncand)
      out[j] = j < n ? j : -1;
    else if (j >= n)
      out[j] = -1;
  }
  if (n == 0 || n == ncand) {
    if (out_lds)
      for (int j = lane; j < n; j += 64) out_lds[j] = j;
    wave_lds_sync();
    return;
  }
  topk_wave_core<KPL>(key, ncand, n, out, out_lds, hist);
}

}  // namespace sss
