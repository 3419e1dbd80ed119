// Split-KV merge and block-score finalisation.
//
// Partials over disjoint KV chunks combine exactly through their
// log-sum-exp: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
// Block scores (SparseSpec §4.1: dumped logits + LSE rematerialise the exact
// attention scores) are sum_r exp(ell_{r,j} - LSE_r) over the scored rows,
// where ell_{r,j} is the log probability mass row r put on block j in the
// frame of its running max (log2 domain here).
#include "sss_common.h"

namespace sss {
namespace {

constexpr int kFinThreads = 256;
constexpr int kMaxRows = 128;
constexpr int kMaxStage = 8192;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ void store_out(void* o, int dtype, long long idx, float v) {
  if (dtype == SSS_BF16)
    reinterpret_cast<bf16*>(o)[idx] = from_f32<bf16>(v);
  else
    reinterpret_cast<float*>(o)[idx] = v;
}

// Grid: (unit, part).  Every workgroup of a unit recomputes the unit's row
// LSEs (S values per row, staged in LDS with one coalesced pass) and then
// merges its share of the rows and scores its share of the blocks, so small
// batches still fill the GPU.  Both of those phases spread each output's
// reduction over several lanes with their loads issued together: the
// merge splits the partials of an output over `slices` threads (float4
// elements, loads kMergeUnroll deep) and sums the slices through LDS; a
// block's score splits its rows over `lpb` lanes (float4 loads) and sums
// them with lane shuffles.  (One thread per output looping over all
// partials, or over all rows of a block, left each thread waiting on a
// chain of dependent loads: 64 partials x 80 rows on the long-context
// shape took 20-27 us per launch.)
constexpr int kMergeUnroll = 8;
constexpr int kStageDepth = 8;
constexpr int kLseUnroll = 8;

__global__ void __launch_bounds__(kFinThreads) finalize_kernel(FinalizeParams p) {
  __shared__ float lse2[kMaxRows];
  __shared__ float stage[kMaxStage];          // partial LSEs [partial][row]
  __shared__ f32x4 red[kFinThreads];          // merge slices [slice][element]
  const int u = blockIdx.x;
  const int part = blockIdx.y, nparts = gridDim.y;
  const int tid = threadIdx.x;
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
  const int R = p.rows, D = p.head_dim, G = p.group;
  const int L = p.seq_lens[b];
  if (p.skip_len >= 0 && L <= p.skip_len) return;
  const int minL = p.draft ? 1 : p.n_q;
  const bool ok =
      L >= minL && L <= p.max_seq_len && (long long)L <= (long long)p.max_pages * p.page_size;

  auto out_row = [&](int r) -> long long {
    const int iq = r / G, g = r % G;
    return ((long long)b * p.n_q + iq) * (p.num_kv_heads * G) + h * G + g;
  };

  // this workgroup's rows and blocks
  const int rows_per = ceil_div(R, nparts);
  const int r_lo = min(part * rows_per, R), r_hi = min(r_lo + rows_per, R);
  const int blk_per = ceil_div(p.max_blocks, nparts);
  const int j_lo = min(part * blk_per, p.max_blocks), j_hi = min(j_lo + blk_per, p.max_blocks);

  if (!ok) {
    for (int idx = r_lo * D + tid; idx < r_hi * D; idx += kFinThreads)
      store_out(p.o, p.dtype, out_row(idx / D) * D + idx % D, qnan());
    for (int r = r_lo + tid; r < r_hi; r += kFinThreads) p.lse[out_row(r)] = qnan();
    if (p.ell)
      for (int j = j_lo + tid; j < j_hi; j += kFinThreads)
        p.block_scores[(long long)u * p.max_blocks + j] = qnan();
    return;
  }

  if (p.num_chunks > 1) {
    int S;
    if (p.list_len) {
      const int n = p.list_len[u];
      S = n > 0 ? ceil_div(n, p.chunk_items) : 1;
    } else if (!p.draft) {
      S = ceil_div(L, p.chunk_tokens);
    } else {
      const int ws = window_start(L, p.window);
      int nsel = p.sel_count[(long long)b * p.num_kv_heads + h];
      nsel = nsel < 0 ? 0 : (nsel > p.max_sel ? p.max_sel : nsel);
      const int n = p.simple_list ? draft_list_len_simple(nsel, p.block_size, L, ws)
                                  : draft_list_len_mfma(nsel, p.block_size, L, ws);
      S = n > 0 ? ceil_div(n, p.chunk_items) : 1;
    }
    if (S > p.num_chunks) S = p.num_chunks;
    if (S == 1 && p.single_done) return;  // the attention kernel finished this unit
    const float* lp = p.lse_part + (long long)u * p.num_chunks * R;
    // all partial LSEs of the unit -> LDS, kStageDepth independent coalesced
    // loads per thread in flight (a load-then-store loop waited for each)
    const bool staged = S * R <= kMaxStage;
    if (staged) {
      const int n = S * R;
      for (int i0 = 0; i0 < n; i0 += kStageDepth * kFinThreads) {
        float v[kStageDepth];
#pragma unroll
        for (int k = 0; k < kStageDepth; ++k) {
          const int i = i0 + k * kFinThreads + tid;
          v[k] = i < n ? lp[i] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kStageDepth; ++k) {
          const int i = i0 + k * kFinThreads + tid;
          if (i < n) stage[i] = v[k];
        }
      }
    }
    __syncthreads();
    // row LSEs: `lpr` lanes per row (a power of two), each over every
    // lpr-th partial, combined with lane shuffles
    int lpr = 1;
    while (lpr < 16 && 2 * lpr * R <= kFinThreads) lpr *= 2;
    const int q = tid % lpr;
    for (int r0s = 0; r0s < R; r0s += kFinThreads / lpr) {
      const int r = r0s + tid / lpr;
      const bool live = r < R;
      // kLseUnroll independent reads and accumulators per iteration (a
      // single running max waited for every LDS read in turn)
      auto part_lse = [&](int s0) -> float {
        return s0 < S ? (staged ? stage[s0 * R + r] : lp[(long long)s0 * R + r]) : neg_inf();
      };
      float mk[kLseUnroll];
      bool nan = false;
#pragma unroll
      for (int k = 0; k < kLseUnroll; ++k) mk[k] = neg_inf();
      if (live)
        for (int s0 = q; s0 < S; s0 += kLseUnroll * lpr) {
#pragma unroll
          for (int k = 0; k < kLseUnroll; ++k) {
            const float x = part_lse(s0 + k * lpr);
            nan |= (x != x);
            mk[k] = fmaxf(mk[k], x);
          }
        }
      float m = mk[0];
#pragma unroll
      for (int k = 1; k < kLseUnroll; ++k) m = fmaxf(m, mk[k]);
      for (int o = 1; o < lpr; o <<= 1) {
        m = fmaxf(m, __shfl_xor(m, o));
        nan |= __shfl_xor((int)nan, o) != 0;
      }
      float sk[kLseUnroll];
#pragma unroll
      for (int k = 0; k < kLseUnroll; ++k) sk[k] = 0.f;
      if (live && !nan && m != neg_inf())
        for (int s0 = q; s0 < S; s0 += kLseUnroll * lpr) {
#pragma unroll
          for (int k = 0; k < kLseUnroll; ++k) sk[k] += fexp2(part_lse(s0 + k * lpr) - m);
        }
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < kLseUnroll; ++k) sum += sk[k];
      for (int o = 1; o < lpr; o <<= 1) sum += __shfl_xor(sum, o);
      if (live && q == 0) {
        const float out = nan ? qnan() : (m == neg_inf() ? neg_inf() : m + flog2(sum));
        lse2[r] = out;
        if (r >= r_lo && r < r_hi) p.lse[out_row(r)] = out * kLn2;
      }
    }
    __syncthreads();
    // merge of this workgroup's rows: element e4 (a float4 of row
    // r_lo + e4 / (D/4)) gets slice `sl` of the partials from thread
    // sl * n4 + e4; the slices are then summed through LDS
    const int d4 = D / 4;
    const int n4 = (r_hi - r_lo) * d4;
    int slices = 1;
    while (slices * 2 * n4 <= kFinThreads && slices * 2 <= S) slices *= 2;
    const f32x4* op = reinterpret_cast<const f32x4*>(p.o_part) + (long long)u * p.num_chunks * R * d4;
    // a thread of the merge owns one (element, slice) pair; several
    // elements per thread when the rows do not fit one pass
    for (int base = 0; base < n4; base += kFinThreads / slices) {
      const int e4 = base + tid % (kFinThreads / slices);
      const int sl = tid / (kFinThreads / slices);
      const bool live = tid < slices * (kFinThreads / slices) && e4 < n4;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int r = live ? r_lo + e4 / d4 : r_lo;
      const float tot = lse2[r];
      if (live && tot != neg_inf() && tot == tot) {
        const f32x4* src = op + (long long)r * d4 + e4 % d4;
        for (int s0 = sl; s0 < S; s0 += kMergeUnroll * slices) {
          f32x4 v[kMergeUnroll];
          float w[kMergeUnroll];
#pragma unroll
          for (int k = 0; k < kMergeUnroll; ++k) {
            const int s1 = s0 + k * slices;
            const bool in = s1 < S;
            v[k] = in ? src[(long long)s1 * R * d4] : f32x4{0.f, 0.f, 0.f, 0.f};
            const float x = !in ? neg_inf()
                                : (staged ? stage[s1 * R + r] : lp[(long long)s1 * R + r]);
            w[k] = fexp2(x - tot);
          }
#pragma unroll
          for (int k = 0; k < kMergeUnroll; ++k) {
            acc[0] += w[k] * v[k][0];
            acc[1] += w[k] * v[k][1];
            acc[2] += w[k] * v[k][2];
            acc[3] += w[k] * v[k][3];
          }
        }
      }
      __syncthreads();
      red[tid] = acc;
      __syncthreads();
      if (live && sl == 0) {
        for (int k = 1; k < slices; ++k) {
          const f32x4 o2 = red[k * (kFinThreads / slices) + tid];
          acc[0] += o2[0];
          acc[1] += o2[1];
          acc[2] += o2[2];
          acc[3] += o2[3];
        }
        const long long at = out_row(r) * D + 4 * (e4 % d4);
        const bool nan = tot != tot;
#pragma unroll
        for (int c = 0; c < 4; ++c) store_out(p.o, p.dtype, at + c, nan ? qnan() : acc[c]);
      }
    }
  } else {
    for (int r = tid; r < R; r += kFinThreads) lse2[r] = p.lse[out_row(r)] * kLog2e;
    __syncthreads();
  }
  if (!p.ell) return;

  // block scores: `lpb` lanes per block (a power of two <= 16, sized so that
  // each lane loads at most two float4s of the block's rows, or a few rows)
  const int nblk = ceil_div(L, p.block_size);
  const int r0 = p.score_row_start * G;
  const float* ell = p.ell + (long long)u * p.max_blocks * R;
  const bool vec = (R % 4) == 0 && (r0 % 4) == 0;
  const int nr = R - r0;
  const int items = vec ? nr / 4 : nr;   // float4s or rows per block
  int lpb = 1;
  while (lpb < 16 && 2 * lpb < items) lpb *= 2;
  const int q = tid % lpb;
  for (int j0 = j_lo; j0 < j_hi; j0 += kFinThreads / lpb) {
    const int j = j0 + tid / lpb;
    float sc = 0.f;
    if (j < j_hi && j < nblk) {
      const float* e = ell + (long long)j * R + r0;
      if (vec) {
        for (int k = q; k < items; k += lpb) {
          const f32x4 x = reinterpret_cast<const f32x4*>(e)[k];
          const float* l2 = lse2 + r0 + 4 * k;
          sc += fexp2(x[0] - l2[0]) + fexp2(x[1] - l2[1]) + fexp2(x[2] - l2[2]) +
                fexp2(x[3] - l2[3]);
        }
      } else {
        for (int k = q; k < items; k += lpb) sc += fexp2(e[k] - lse2[r0 + k]);
      }
    }
    for (int o = 1; o < lpb; o <<= 1) sc += __shfl_xor(sc, o);
    if (q == 0 && j < j_hi) p.block_scores[(long long)u * p.max_blocks + j] = sc;
  }
}

// Public merge (natural-log LSEs in and out).  A workgroup merges
// kMergeRows rows: each of its waves reduces one row's partial LSEs (max,
// then sum of exponentials: one exp per partial and row), and the weights
// exp(lse_s - lse) of a tile of partials are staged in LDS, where every
// thread reads them for its (row, dim) elements of the weighted sum.
constexpr int kMergeThreads = 256;
constexpr int kMergeRows = kMergeThreads / 64;
constexpr int kMergeTile = 1024;                        // partials per weight tile
constexpr int kMergeAcc = kMergeRows * 1024 / kMergeThreads;  // head_dim <= 1024

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ void __launch_bounds__(kMergeThreads)
    merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int S,
                 int rows, int D, void* o, int dtype, float* lse) {
  __shared__ float tot_s[kMergeRows];
  __shared__ float w_s[kMergeRows][kMergeTile];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r0 = blockIdx.x * kMergeRows;
  const int nr = min(kMergeRows, rows - r0);
  // row LSE, once per row
  if (wv < nr) {
    const int r = r0 + wv;
    float m = neg_inf();
    bool nan = false;
    for (int s = lane; s < S; s += 64) {
      const float x = lse_parts[(long long)s * rows + r];
      nan |= (x != x);
      m = fmaxf(m, x);
    }
    m = wave_max(m);
    nan = __any(nan);
    float tot;
    if (nan) {
      tot = qnan();
    } else if (m == neg_inf()) {
      tot = neg_inf();
    } else {
      float sum = 0.f;
      for (int s = lane; s < S; s += 64) sum += expf(lse_parts[(long long)s * rows + r] - m);
      tot = m + logf(wave_sum(sum));
    }
    if (lane == 0) {
      tot_s[wv] = tot;
      if (lse) lse[r] = tot;
    }
  }
  __syncthreads();
  float acc[kMergeAcc];
#pragma unroll
  for (int k = 0; k < kMergeAcc; ++k) acc[k] = 0.f;
  const int n = nr * D;  // this workgroup's elements, contiguous in every partial
  for (int s0 = 0; s0 < S; s0 += kMergeTile) {
    const int ns = min(kMergeTile, S - s0);
    if (wv < nr) {
      const float tot = tot_s[wv];
      const bool live = tot == tot && tot != neg_inf();
      for (int i = lane; i < ns; i += 64)
        w_s[wv][i] = live ? expf(lse_parts[(long long)(s0 + i) * rows + r0 + wv] - tot) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMergeAcc; ++k) {
      const int idx = tid + k * kMergeThreads;
      if (idx < n) {
        const int rr = idx / D;
        const float* src = o_parts + (long long)s0 * rows * D + (long long)r0 * D + idx;
        float a = acc[k];
        for (int i = 0; i < ns; ++i) a += w_s[rr][i] * src[(long long)i * rows * D];
        acc[k] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kMergeAcc; ++k) {
    const int idx = tid + k * kMergeThreads;
    if (idx < n) {
      const float tot = tot_s[idx / D];
      store_out(o, dtype, (long long)r0 * D + idx, tot != tot ? qnan() : acc[k]);
    }
  }
}

}  // namespace

hipError_t launch_finalize(const FinalizeParams& p, hipStream_t s) {
  const long long units = (long long)p.batch * p.num_kv_heads;
  if (units == 0) return hipSuccess;
  // enough workgroups to cover the GPU: about 2048 in total, at most one
  // per 64 blocks (scores) or per row (merge) of a unit, and at most 128
  long long parts = (2048 + units - 1) / units;
  const long long cap = (p.max_blocks + 63) / 64 > p.rows ? (p.max_blocks + 63) / 64 : p.rows;
  if (parts > cap) parts = cap;
  if (parts > 128) parts = 128;
  if (parts < 1) parts = 1;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)units, (unsigned)parts), dim3(kFinThreads), 0,
                     s, p);
  return hipGetLastError();
}

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int num_parts, int rows,
                        int head_dim, void* o, int o_dtype, float* lse, hipStream_t s) {
  if (rows == 0 || head_dim == 0) return hipSuccess;
  if (head_dim > 1024) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((rows + kMergeRows - 1) / kMergeRows);
  hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(kMergeThreads), 0, s, o_parts, lse_parts,
                     num_parts, rows, head_dim, o, o_dtype, lse);
  return hipGetLastError();
}

}  // namespace sss
