// Top-N block selection (SparseSpec §4.1: Top-K over the aggregated block
// scores), one workgroup per (request, KV head).
//
// Exact radix select on 32-bit order-preserving keys of the fp32 scores:
// four 8-bit MSB-first histogram passes find the N-th largest key T; the
// blocks with key > T are taken, plus the lowest-index blocks with key == T
// until N are taken.  Histograms count with LDS integer atomics (order
// independent), ranks come from ballot prefix sums in index order, so the
// selection is bit-exact and deterministic.  Output is ascending.
#include "sss_common.h"

namespace sss {
namespace {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;

// Monotone map of an fp32 score to uint32 (larger score -> larger key);
// -0.0 is folded onto +0.0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix count of `flag` over the workgroup in thread order, and
// the workgroup total.  Uses `scratch` (kTopkWaves ints).
__device__ __forceinline__ int wg_exclusive_count(bool flag, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) scratch[wave] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int c = scratch[w];
    if (w < wave) before += c;
    total += c;
  }
  __syncthreads();
  return before + below;
}

__global__ void __launch_bounds__(kTopkThreads)
    topk_kernel(const float* __restrict__ scores, int hkv, int max_blocks,
                const int32_t* __restrict__ seq_lens, int bs, const int32_t* __restrict__ budget,
                int window, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
                int max_sel) {
  __shared__ int hist[256];
  __shared__ int scan_scratch[kTopkWaves];
  __shared__ uint32_t s_digit;
  __shared__ int s_rem;

  const int u = blockIdx.x;
  const int b = u / hkv;
  int L = seq_lens[b];
  if (L < 0) L = 0;
  const long long nblk = ((long long)L + bs - 1) / bs;
  const int ws = window_start(L, window);
  long long ncand_l = ((long long)ws + bs - 1) / bs;
  if (ncand_l > nblk) ncand_l = nblk;
  if (ncand_l > max_blocks) ncand_l = max_blocks;
  const int ncand = (int)ncand_l;
  int n = budget[b];
  if (n < 0) n = 0;
  if (n > ncand) n = ncand;
  if (n > max_sel) n = max_sel;

  const float* sc = scores + (long long)u * max_blocks;
  int32_t* out = sel + (long long)u * max_sel;
  if (threadIdx.x == 0) sel_count[u] = n;
  // every candidate kept, or none: the list is 0..n-1; otherwise positions
  // [0, n) are written by the emission below
  for (int j = threadIdx.x; j < max_sel; j += kTopkThreads) {
    if (n == ncand)
      out[j] = j < n ? j : -1;
    else if (j >= n)
      out[j] = -1;
  }
  if (n == 0 || n == ncand) return;

  // ---- radix select of the n-th largest key ----
  uint32_t prefix = 0, pmask = 0;
  int rem = n;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < ncand; j += kTopkThreads) {
      const uint32_t k = score_key(sc[j]);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
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
            s_digit = (uint32_t)(255 - (4 * lane + e));
            s_rem = rem - cum;
            break;
          }
          cum += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    rem = s_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = rem;

  // ---- ascending emission ----
  int taken = 0, ties = 0;
  for (int base = 0; base < ncand; base += kTopkThreads) {
    const int j = base + threadIdx.x;
    const bool valid = j < ncand;
    const uint32_t k = valid ? score_key(sc[j]) : 0u;
    const bool gt = valid && k > T;
    const bool eq = valid && k == T;
    int tie_total;
    const int tie_rank = ties + wg_exclusive_count(eq, scan_scratch, tie_total);
    const bool take = gt || (eq && tie_rank < need_eq);
    int take_total;
    const int pos = taken + wg_exclusive_count(take, scan_scratch, take_total);
    if (take) out[pos] = j;
    ties += tie_total;
    taken += take_total;
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int batch, int hkv, int max_blocks,
                       const int32_t* seq_lens, int block_size, const int32_t* budget, int window,
                       int32_t* sel, int32_t* sel_count, int max_sel, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)batch * hkv);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(grid), dim3(kTopkThreads), 0, s, scores, hkv, max_blocks,
                     seq_lens, block_size, budget, window, sel, sel_count, max_sel);
  return hipGetLastError();
}

}  // namespace sss
