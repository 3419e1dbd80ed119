// Top-N block selection of one (request, KV head) unit as a workgroup-level
// device routine (SparseSpec §4.1: Top-K over the aggregated block scores).
// Used by the stand-alone selection kernel and by the fused step kernel.
//
// Exact radix select on 32-bit order-preserving keys of the fp32 scores:
// four 8-bit MSB-first histogram passes find the N-th largest key T; the
// blocks with key > T are taken, plus the lowest-index blocks with key == T
// until N are taken.  Histograms count with LDS integer atomics (order
// independent), ranks come from ballot prefix sums in index order, so the
// selection is bit-exact and deterministic.  Output is ascending.
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

// LDS words topk_select needs.
constexpr int kTopkLdsWords = 256 + 16 + 2;

// Exclusive prefix count of `flag` over the workgroup in thread order, and
// the workgroup total.  `scratch` holds NT / 64 ints.
template <int NT>
__device__ __forceinline__ int wg_exclusive_count(bool flag, int* scratch, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) scratch[wave] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = scratch[w];
    if (w < wave) before += c;
    total += c;
  }
  __syncthreads();
  return before + below;
}

// The n largest of sc[0, ncand) (ties to the lower index), ascending, into
// out[0, n); out[n, max_sel) = -1.  When out_lds is given, out_lds[0, n)
// receives the same list.  `lds` holds kTopkLdsWords ints.  All NT threads
// of the workgroup call it; it ends with a barrier.
template <int NT>
__device__ void topk_select(const float* sc, int ncand, int n, int32_t* __restrict__ out,
                            int max_sel, int32_t* out_lds, int* lds) {
  static_assert(NT % 64 == 0 && NT >= 64 && NT <= 1024, "workgroup of whole waves");
  int* hist = lds;
  int* scan_scratch = lds + 256;
  int* s_digit = lds + 272;
  int* s_rem = lds + 273;
  const int tid = threadIdx.x;

  // every candidate kept, or none: the list is 0..n-1; otherwise positions
  // [0, n) are written by the emission below
  for (int j = tid; j < max_sel; j += NT) {
    if (n == ncand)
      out[j] = j < n ? j : -1;
    else if (j >= n)
      out[j] = -1;
  }
  if (n == 0 || n == ncand) {
    if (out_lds)
      for (int j = tid; j < n; j += NT) out_lds[j] = j;
    __syncthreads();
    return;
  }

  // ---- radix select of the n-th largest key ----
  uint32_t prefix = 0, pmask = 0;
  int rem = n;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < ncand; j += NT) {
      const uint32_t k = score_key(sc[j]);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      const int lane = tid;
      int c[4], local = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - (4 * lane + e)];  // descending digit order
        local += c[e];
      }
      int incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const int excl = incl - local;
      if (excl < rem && rem <= incl) {
        int cum = excl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (cum + c[e] >= rem) {
            *s_digit = 255 - (4 * lane + e);
            *s_rem = rem - cum;
            break;
          }
          cum += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)*s_digit << shift;
    pmask |= 255u << shift;
    rem = *s_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = rem;

  // ---- ascending emission ----
  int taken = 0, ties = 0;
  for (int base = 0; base < ncand; base += NT) {
    const int j = base + tid;
    const bool valid = j < ncand;
    const uint32_t k = valid ? score_key(sc[j]) : 0u;
    const bool gt = valid && k > T;
    const bool eq = valid && k == T;
    int tie_total;
    const int tie_rank = ties + wg_exclusive_count<NT>(eq, scan_scratch, tie_total);
    const bool take = gt || (eq && tie_rank < need_eq);
    int take_total;
    const int pos = taken + wg_exclusive_count<NT>(take, scan_scratch, take_total);
    if (take) {
      out[pos] = j;
      if (out_lds) out_lds[pos] = j;
    }
    ties += tie_total;
    taken += take_total;
  }
  __syncthreads();
}

}  // namespace sss
