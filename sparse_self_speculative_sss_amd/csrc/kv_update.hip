// KV update around a verification step (SpecSA, 核心创新 / 刷新/复用NSA内核融合:
// the KV of accepted speculative tokens is reused by later queries, the KV
// of rejected ones is refreshed).
//
// kv_write_kernel scatters the K and V rows of new token positions into the
// paged cache, one thread per 16-byte piece of a (request, new token, KV
// head) row.  kv_commit_kernel shortens each request to the speculative
// positions it keeps; dropped positions are not touched (a position at or
// past a request's length is never read).
#include "sss_common.h"

namespace sss {
namespace {

constexpr int kWriteThreads = 256;

// One thread per 16-byte piece of a (request, new token, KV head) row.
__global__ void __launch_bounds__(kWriteThreads) kv_write_kernel(KvWriteParams p) {
  const long long row_bytes = (long long)p.head_dim * p.elem_bytes;
  const int chunks = (int)(row_bytes / 16);
  const long long rows = (long long)p.batch * p.n_new * p.num_kv_heads;
  const long long idx = (long long)blockIdx.x * kWriteThreads + threadIdx.x;
  if (idx >= rows * chunks) return;
  const long long row = idx / chunks;
  const int c = (int)(idx % chunks);
  const int h = (int)(row % p.num_kv_heads);
  const int i = (int)((row / p.num_kv_heads) % p.n_new);
  const int b = (int)(row / ((long long)p.num_kv_heads * p.n_new));
  const long long t = (long long)p.pos0[b] + i;
  if (t < 0 || t / p.page_size >= p.max_pages) return;
  const int pg = p.page_table[(long long)b * p.max_pages + t / p.page_size];
  if (pg < 0 || pg >= p.num_pages) return;
  const long long dst = (((long long)pg * p.num_kv_heads + h) * p.page_size + t % p.page_size) *
                            row_bytes + 16 * c;
  const long long src = row * row_bytes + 16 * c;
  const uint4 kv = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.k_new) + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.v_new) + src);
  *reinterpret_cast<uint4*>(static_cast<char*>(p.k) + dst) = kv;
  *reinterpret_cast<uint4*>(static_cast<char*>(p.v) + dst) = vv;
}

__global__ void kv_commit_kernel(const int32_t* seq_lens, const int32_t* keep, int batch, int n_q,
                                 int32_t* out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  int kp = keep[b];
  kp = kp < 0 ? 0 : (kp > n_q ? n_q : kp);
  const int L = seq_lens[b] - n_q + kp;
  out[b] = L > 0 ? L : 0;
}

}  // namespace

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t s) {
  const long long pieces =
      (long long)p.batch * p.n_new * p.num_kv_heads * (p.head_dim * p.elem_bytes / 16);
  if (pieces == 0) return hipSuccess;
  const long long blocks = (pieces + kWriteThreads - 1) / kWriteThreads;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(kWriteThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_kv_commit(const int32_t* seq_lens, const int32_t* keep, int batch, int n_q,
                            int32_t* out, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_commit_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, s,
                     seq_lens, keep, batch, n_q, out);
  return hipGetLastError();
}

}  // namespace sss
