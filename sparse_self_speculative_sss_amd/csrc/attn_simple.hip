// Vector-ALU paged attention: the path for fp32 caches and for page or block
// sizes that are not multiples of 16.  One workgroup computes one row of one
// chunk of one unit.  It makes two passes over the chunk's tokens: the first
// finds the chunk's log-sum-exp, the second accumulates O and the per-block
// probability masses in that fixed frame (so a block's mass is a plain sum).
// Same outputs as the matrix-core kernel: final O/LSE for one chunk,
// log2-domain partials otherwise, and per-(block, row) log2 masses for verify.
#include "sss_common.h"

namespace sss {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < kThreads / 64; ++w) r += red[w];
  return r;
}

template <typename T, bool DRAFT>
__global__ void __launch_bounds__(kThreads) attn_simple_kernel(AttnParams p) {
  __shared__ float qs[128];
  __shared__ float ps[kThreads];
  __shared__ int ts[kThreads];
  __shared__ long long rows_s[kThreads];   // K/V row offset of each entry's token
  __shared__ float ored[kThreads];         // per-group partial O, reduced at the end
  __shared__ float red[kThreads / 64];
  __shared__ float carry;
  __shared__ int bad_flag;

  const int R = p.rows, D = p.head_dim;
  const int r = blockIdx.x % R;
  const int uc = blockIdx.x / R;
  const int u = uc / p.num_chunks, c = uc % p.num_chunks;
  const int b = u / p.num_kv_heads, h = u % p.num_kv_heads;
  const int iq = r / p.group, hq = h * p.group + r % p.group;
  const long long orow = ((long long)b * p.n_q + iq) * p.num_q_heads + hq;
  const int L = p.seq_lens[b];
  const int minL = DRAFT ? 1 : p.n_q;
  const bool unit_ok =
      L >= minL && L <= p.max_seq_len && (long long)L <= (long long)p.max_pages * p.page_size;
  const bool final_out = p.num_chunks == 1;
  if (!unit_ok) {
    if (final_out) {
      for (int d = threadIdx.x; d < D; d += kThreads)
        reinterpret_cast<T*>(p.o)[orow * D + d] = from_f32<T>(qnan());
      if (threadIdx.x == 0) p.lse[orow] = qnan();
    }
    return;
  }

  // this chunk's list range [k_lo, k_hi)
  int k_lo, k_hi, nsel = 0, ws = L;
  if (!DRAFT) {
    k_lo = c * p.chunk_tokens;
    if (k_lo >= L) return;
    k_hi = min(k_lo + p.chunk_tokens, L);
  } else {
    ws = window_start(L, p.window);
    nsel = p.sel_count[(long long)b * p.num_kv_heads + h];
    nsel = nsel < 0 ? 0 : (nsel > p.max_sel ? p.max_sel : nsel);
    const int n = draft_list_len_simple(nsel, p.block_size, L, ws);
    k_lo = c * p.chunk_items;
    if (k_lo >= n && c > 0) return;
    k_hi = min(k_lo + p.chunk_items, n);
  }
  const int pos = DRAFT ? L - 1 : L - p.n_q + iq;
  const T* kc = reinterpret_cast<const T*>(p.k);
  const T* vc = reinterpret_cast<const T*>(p.v);
  const T* q = reinterpret_cast<const T*>(p.q) + orow * D;
  for (int d = threadIdx.x; d < D; d += kThreads) qs[d] = to_f32(q[d]);
  if (threadIdx.x == 0) bad_flag = 0;
  __syncthreads();

  // list entry -> token (or -1 when the entry attends to nothing)
  auto token_of = [&](int k) -> int {
    if (!DRAFT) return k <= pos ? k : -1;
    if (k < nsel * p.block_size) {
      const int j = p.sel[((long long)b * p.num_kv_heads + h) * p.max_sel + k / p.block_size];
      if (j < 0 || j >= ceil_div(ws, p.block_size)) return -1;
      const int t = j * p.block_size + k % p.block_size;
      return t < ws ? t : -1;
    }
    const int t = ws + (k - nsel * p.block_size);
    return t < L ? t : -1;
  };
  auto row_of = [&](int t) -> long long {  // element offset of token t's K/V row
    int pg = p.page_table[(long long)b * p.max_pages + t / p.page_size];
    if (pg < 0 || pg >= p.num_pages) {
      bad_flag = 1;
      pg = 0;
    }
    return (((long long)pg * p.num_kv_heads + h) * p.page_size + t % p.page_size) * D;
  };
  auto logit = [&](int t) -> float {
    const T* kr = kc + row_of(t);
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc += qs[d] * to_f32(kr[d]);
    return acc * p.scale_log2;
  };

  // pass 1: log2-sum-exp of the chunk
  float m = neg_inf(), l = 0.f;
  for (int base = k_lo; base < k_hi; base += kThreads) {
    const int k = base + threadIdx.x;
    const int t = k < k_hi ? token_of(k) : -1;
    const float s = t >= 0 ? logit(t) : neg_inf();
    const float mt = block_max(s, red);
    const float mn = fmaxf(m, mt);
    const float mu = mn == neg_inf() ? 0.f : mn;
    const float st = block_sum(fexp2(s - mu), red);
    l = l * fexp2(m - mu) + st;
    m = mn;
  }
  const float lse2 = l > 0.f ? m + flog2(l) : neg_inf();
  const float frame = l > 0.f ? lse2 : 0.f;

  // pass 2: O and block masses in the fixed frame.  Each thread resolves its
  // own entry's token (weight and cache row) once; then the workgroup splits
  // into kThreads / D groups, group g accumulating O over entries g, g + NG,
  // ... with thread d owning O[d] (several loads in flight per thread)
  const int NG = kThreads / D;  // D is 64 or 128
  const int og = threadIdx.x / D, od = threadIdx.x % D;
  float oacc = 0.f;
  if (threadIdx.x == 0) carry = 0.f;
  for (int base = k_lo; base < k_hi; base += kThreads) {
    const int k = base + threadIdx.x;
    const int t = k < k_hi ? token_of(k) : -1;
    __syncthreads();
    ps[threadIdx.x] = t >= 0 ? fexp2(logit(t) - frame) : 0.f;
    ts[threadIdx.x] = t;
    rows_s[threadIdx.x] = t >= 0 ? row_of(t) : 0;
    __syncthreads();
    const int n_here = min(kThreads, k_hi - base);
    {
      int i = og;
      for (; i + 3 * NG < n_here; i += 4 * NG) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = to_f32(vc[rows_s[i + e * NG] + od]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ts[i + e * NG] >= 0) oacc += ps[i + e * NG] * x[e];
      }
      for (; i < n_here; i += NG)
        if (ts[i] >= 0) oacc += ps[i] * to_f32(vc[rows_s[i] + od]);
    }
    if (!DRAFT) {
      // verify: the entries base..base+n_here-1 are consecutive tokens and
      // cover blocks j0..j1; a block that continues into the next tile hands
      // its partial sum over through `carry`
      const int bs = p.block_size;
      const int j0 = base / bs, j1 = (base + n_here - 1) / bs;
      const int nb = j1 - j0 + 1;
      const bool last_cont = min((long long)(j1 + 1) * bs, (long long)k_hi) > base + n_here;
      float* ell = p.ell + (long long)u * p.max_blocks * R;
      float cont_val = 0.f;
      for (int jj = threadIdx.x; jj < nb; jj += kThreads) {
        const int j = j0 + jj;
        const int a = max(j * bs, base), e = min((j + 1) * bs, base + n_here);
        float sum = 0.f;
        for (int i = a; i < e; ++i) sum += ps[i - base];
        if (jj == 0) sum += carry;
        if (jj == nb - 1 && last_cont)
          cont_val = sum;
        else
          ell[(long long)j * R + r] = frame + flog2(sum);
      }
      __syncthreads();
      if (last_cont) {
        if (threadIdx.x == (nb - 1) % kThreads) carry = cont_val;
      } else if (threadIdx.x == 0) {
        carry = 0.f;
      }
    }
  }
  // combine the groups' partial O (group 0's threads own the result)
  __syncthreads();
  ored[threadIdx.x] = oacc;
  __syncthreads();
  if (og == 0)
    for (int g = 1; g < NG; ++g) oacc += ored[g * D + od];
  const bool bad = bad_flag != 0;
  // oacc was accumulated with the normalised weights exp2(s - lse2)
  const float poison = bad ? qnan() : 1.f;
  if (final_out) {
    if (threadIdx.x < D) reinterpret_cast<T*>(p.o)[orow * D + threadIdx.x] = from_f32<T>(oacc * poison);
    if (threadIdx.x == 0) p.lse[orow] = bad ? qnan() : lse2 * kLn2;
  } else {
    const long long prow = ((long long)u * p.num_chunks + c) * R + r;
    if (threadIdx.x < D) p.o_part[prow * D + threadIdx.x] = oacc * poison;
    if (threadIdx.x == 0) p.lse_part[prow] = bad ? qnan() : lse2;
  }
}

}  // namespace

hipError_t launch_attn_simple(const AttnParams& p, int dtype, bool draft, hipStream_t s) {
  const long long grid = (long long)p.batch * p.num_kv_heads * p.num_chunks * p.rows;
  if (grid == 0) return hipSuccess;
  if (dtype == SSS_F32) {
    if (draft)
      hipLaunchKernelGGL((attn_simple_kernel<float, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((attn_simple_kernel<float, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  } else {
    if (draft)
      hipLaunchKernelGGL((attn_simple_kernel<bf16, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((attn_simple_kernel<bf16, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sss
