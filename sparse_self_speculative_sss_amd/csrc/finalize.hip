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
constexpr int kMaxWeights = 2048;
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
// LSEs (S values per row, cheap) and then merges its share of the rows and
// scores its share of the blocks, so small batches still fill the GPU.
__global__ void __launch_bounds__(kFinThreads) finalize_kernel(FinalizeParams p) {
  __shared__ float lse2[kMaxRows];
  __shared__ float wts[kMaxWeights];  // merge weights [partial][row of this workgroup]
  __shared__ float stage[kMaxStage];  // partial LSEs [partial][row]
  const int u = blockIdx.x;
  const int part = blockIdx.y, nparts = gridDim.y;
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
    for (int idx = r_lo * D + threadIdx.x; idx < r_hi * D; idx += kFinThreads)
      store_out(p.o, p.dtype, out_row(idx / D) * D + idx % D, qnan());
    for (int r = r_lo + threadIdx.x; r < r_hi; r += kFinThreads) p.lse[out_row(r)] = qnan();
    if (p.ell)
      for (int j = j_lo + threadIdx.x; j < j_hi; j += kFinThreads)
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
    // all partial LSEs of the unit -> LDS with independent coalesced loads,
    // then one thread per row reduces them
    const bool staged = S * R <= kMaxStage;
    if (staged)
      for (int i = threadIdx.x; i < S * R; i += kFinThreads) stage[i] = lp[i];
    __syncthreads();
    for (int r = threadIdx.x; r < R; r += kFinThreads) {
      float m = neg_inf();
      bool nan = false;
      for (int s0 = 0; s0 < S; ++s0) {
        const float x = staged ? stage[s0 * R + r] : lp[(long long)s0 * R + r];
        nan |= (x != x);
        m = fmaxf(m, x);
      }
      float sum = 0.f;
      if (!nan && m != neg_inf())
        for (int s0 = 0; s0 < S; ++s0)
          sum += fexp2((staged ? stage[s0 * R + r] : lp[(long long)s0 * R + r]) - m);
      const float out = nan ? qnan() : (m == neg_inf() ? neg_inf() : m + flog2(sum));
      lse2[r] = out;
      if (r >= r_lo && r < r_hi) p.lse[out_row(r)] = out * kLn2;
    }
    __syncthreads();
    // merge weights of this workgroup's rows, then coalesced weighted sums
    const int nr = r_hi - r_lo;
    const bool wfit = S * nr <= kMaxWeights;
    if (wfit)
      for (int i = threadIdx.x; i < S * nr; i += kFinThreads) {
        const int s0 = i / nr, r = r_lo + i % nr;
        const float tot = lse2[r];
        const float x = staged ? stage[s0 * R + r] : lp[(long long)s0 * R + r];
        wts[i] = (tot == neg_inf() || tot != tot) ? 0.f : fexp2(x - tot);
      }
    __syncthreads();
    const float* op = p.o_part + (long long)u * p.num_chunks * R * D;
    for (int idx = r_lo * D + threadIdx.x; idx < r_hi * D; idx += kFinThreads) {
      const int r = idx / D, d = idx % D;
      const float tot = lse2[r];
      float acc = 0.f;
      if (tot != neg_inf()) {
#pragma unroll 8
        for (int s0 = 0; s0 < S; ++s0) {
          const float w = wfit ? wts[s0 * nr + (r - r_lo)] : fexp2(lp[(long long)s0 * R + r] - tot);
          acc += w * op[((long long)s0 * R + r) * D + d];
        }
      }
      if (tot != tot) acc = qnan();
      store_out(p.o, p.dtype, out_row(r) * D + d, acc);
    }
  } else {
    for (int r = threadIdx.x; r < R; r += kFinThreads) lse2[r] = p.lse[out_row(r)] * kLog2e;
    __syncthreads();
  }
  if (!p.ell) return;

  const int nblk = ceil_div(L, p.block_size);
  const int r0 = p.score_row_start * G;
  const float* ell = p.ell + (long long)u * p.max_blocks * R;
  for (int j = j_lo + threadIdx.x; j < j_hi; j += kFinThreads) {
    float sc = 0.f;
    if (j < nblk) {
      const float* e = ell + (long long)j * R;
#pragma unroll 8
      for (int r = r0; r < R; ++r) sc += fexp2(e[r] - lse2[r]);
    }
    p.block_scores[(long long)u * p.max_blocks + j] = sc;
  }
}

// Public merge: one thread per (row, dim); natural-log LSE in and out.
__global__ void merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lse_parts,
                             int S, int rows, int D, void* o, int dtype, float* lse) {
  const long long n = (long long)rows * D;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int r = (int)(idx / D), d = (int)(idx % D);
    float m = neg_inf();
    bool nan = false;
    for (int s = 0; s < S; ++s) {
      const float x = lse_parts[(long long)s * rows + r];
      nan |= (x != x);
      m = fmaxf(m, x);
    }
    float tot, acc = 0.f;
    if (nan) {
      tot = acc = qnan();
    } else if (m == neg_inf()) {
      tot = neg_inf();
    } else {
      float sum = 0.f;
      for (int s = 0; s < S; ++s) sum += expf(lse_parts[(long long)s * rows + r] - m);
      tot = m + logf(sum);
      for (int s = 0; s < S; ++s)
        acc += expf(lse_parts[(long long)s * rows + r] - tot) * o_parts[((long long)s * rows + r) * D + d];
    }
    store_out(o, dtype, idx, acc);
    if (lse && d == 0) lse[r] = tot;
  }
}

}  // namespace

hipError_t launch_finalize(const FinalizeParams& p, hipStream_t s) {
  const long long units = (long long)p.batch * p.num_kv_heads;
  if (units == 0) return hipSuccess;
  // enough workgroups to cover the GPU: about 2048 in total, at most one
  // per 64 blocks (scores) or per row (merge) of a unit
  long long parts = (2048 + units - 1) / units;
  const long long cap = (p.max_blocks + 63) / 64 > p.rows ? (p.max_blocks + 63) / 64 : p.rows;
  if (parts > cap) parts = cap;
  if (parts > 64) parts = 64;
  if (parts < 1) parts = 1;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)units, (unsigned)parts), dim3(kFinThreads), 0,
                     s, p);
  return hipGetLastError();
}

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int num_parts, int rows,
                        int head_dim, void* o, int o_dtype, float* lse, hipStream_t s) {
  const long long n = (long long)rows * head_dim;
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, o_parts, lse_parts,
                     num_parts, rows, head_dim, o, o_dtype, lse);
  return hipGetLastError();
}

}  // namespace sss
