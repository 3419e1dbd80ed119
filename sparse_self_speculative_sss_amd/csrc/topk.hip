// Top-N block selection kernel: one workgroup per (request, KV head), the
// selection itself is topk_select (topk_dev.h).
#include "topk_dev.h"

namespace sss {
namespace {

// keys parked in LDS up to this many candidates (64 KiB)
constexpr int kTopkMaxKeys = 16384;

template <int NT>
__global__ void __launch_bounds__(NT)
    topk_kernel(const float* __restrict__ scores, int hkv, int max_blocks,
                const int32_t* __restrict__ seq_lens, int bs, const int32_t* __restrict__ budget,
                int window, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
                int max_sel, int skip_len) {
  __shared__ int lds[kTopkLdsWords];
  // the unit's keys, when max_blocks of them fit (dynamic LDS)
  extern __shared__ uint32_t keys[];
  const int u = blockIdx.x;
  const int b = u / hkv;
  // units no longer than skip_len were selected by the fused step kernel
  if (skip_len >= 0 && seq_lens[b] <= skip_len) return;
  int ncand, n;
  topk_bounds(seq_lens[b], bs, window, max_blocks, budget[b], max_sel, ncand, n);
  if (threadIdx.x == 0) sel_count[u] = n;
  topk_select<NT>(scores + (long long)u * max_blocks, ncand, n, sel + (long long)u * max_sel,
                  max_sel, nullptr, lds, keys, max_blocks <= kTopkMaxKeys ? max_blocks : 0);
}

// One wave per unit for units of at most 64 * KPL candidates (topk_wave:
// no workgroup barrier), four units per workgroup.
template <int KPL>
__global__ void __launch_bounds__(256)
    topk_wave_kernel(const float* __restrict__ scores, int units, int hkv, int max_blocks,
                     const int32_t* __restrict__ seq_lens, int bs,
                     const int32_t* __restrict__ budget, int window, int32_t* __restrict__ sel,
                     int32_t* __restrict__ sel_count, int max_sel, int skip_len) {
  __shared__ __attribute__((aligned(16))) int hist[4][kTopkBins];
  const int w = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + w;
  if (u >= units) return;
  const int b = u / hkv;
  if (skip_len >= 0 && seq_lens[b] <= skip_len) return;
  int ncand, n;
  topk_bounds(seq_lens[b], bs, window, max_blocks, budget[b], max_sel, ncand, n);
  if ((threadIdx.x & 63) == 0) sel_count[u] = n;
  topk_wave<KPL>(ScoreSrc{scores + (long long)u * max_blocks}, ncand, n, sel + (long long)u * max_sel,
                 max_sel, nullptr, hist[w]);
}

}  // namespace

hipError_t launch_topk(const float* scores, int batch, int hkv, int max_blocks,
                       const int32_t* seq_lens, int block_size, const int32_t* budget, int window,
                       int32_t* sel, int32_t* sel_count, int max_sel, int skip_len,
                       hipStream_t s) {
  const unsigned grid = (unsigned)((long long)batch * hkv);
  if (grid == 0) return hipSuccess;
  const size_t smem = max_blocks <= kTopkMaxKeys ? (size_t)max_blocks * 4 : 0;
  // few units with many candidates: a wider workgroup per unit (the units
  // then run one wave of workgroups at once; 8 units of 2046 blocks: 11.1 us
  // against 12.8 us with 256 threads); many units of few candidates: 256
  // threads, so that more workgroups share a CU
  auto go = [&](auto kern, int nt) -> hipError_t {
    // dynamic LDS above 64 KiB (with the static part) must be opted into
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        kTopkMaxKeys * 4);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nt), smem, s, scores, hkv, max_blocks, seq_lens,
                       block_size, budget, window, sel, sel_count, max_sel, skip_len);
    return hipGetLastError();
  };
  // many units of at most 1024 candidates: one wave per unit, no barrier
  // (batch 128 x 8 heads, 508 candidates: see DESIGN)
  if (max_blocks <= 1024 && grid > 256) {
    const unsigned wgrid = (grid + 3) / 4;
    auto wkern = max_blocks <= 512 ? topk_wave_kernel<8> : topk_wave_kernel<16>;
    hipLaunchKernelGGL(wkern, dim3(wgrid), dim3(256), 0, s, scores, (int)grid, hkv, max_blocks,
                       seq_lens, block_size, budget, window, sel, sel_count, max_sel, skip_len);
    return hipGetLastError();
  }
  if (grid <= 256 && max_blocks >= 1024) return go(topk_kernel<1024>, 1024);
  // many units of thousands of candidates (single-token selection): 512
  // threads (1024 units of 8128 tokens: 43 us against 49 us with 256)
  if (max_blocks >= 4096) return go(topk_kernel<512>, 512);
  return go(topk_kernel<256>, 256);
}

}  // namespace sss
