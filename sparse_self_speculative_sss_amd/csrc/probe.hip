// Bandwidth probes (sss_probe.h): kernels that only read, with the 16-byte
// non-temporal global loads of the attention kernels, and fold what they
// read into one XOR per workgroup so that the loads stay live.
#include "../../include/sss_probe.h"
#include "sss_common.h"

namespace sss {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeGrid = SSS_PROBE_SINK_WORDS;
constexpr int kStreamDepth = 8;  // loads in flight per lane
constexpr int kPagedDepth = 8;   // (page, head) runs in flight per workgroup

__device__ __forceinline__ u32x4 nt_load(const u32x4* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ uint32_t fold(const u32x4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

// XOR of every thread's value -> sink[blockIdx.x] (a vector store).
__device__ void sink_xor(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t part[kProbeThreads / 64];
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

// Streaming read of n16 16-byte words: each workgroup iteration reads a
// contiguous block of 256 * kStreamDepth words (lane l: words l, l + 256,
// ...), blocks dealt round-robin over the grid.  (Loads one grid stride
// apart instead, 16 MiB between a lane's loads in flight, streamed at
// 6.43 TB/s against 7.0 TB/s for contiguous blocks on MI355X.)
__global__ void __launch_bounds__(kProbeThreads)
    stream_read_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* sink) {
  constexpr size_t kBlock = (size_t)kProbeThreads * kStreamDepth;
  const size_t n_full = n16 / kBlock;
  uint32_t acc = 0;
  for (size_t blk = blockIdx.x; blk < n_full; blk += gridDim.x) {
    const u32x4* p = src + blk * kBlock + threadIdx.x;
    u32x4 v[kStreamDepth];
#pragma unroll
    for (int k = 0; k < kStreamDepth; ++k) v[k] = nt_load(p + k * kProbeThreads);
#pragma unroll
    for (int k = 0; k < kStreamDepth; ++k) acc ^= fold(v[k]);
  }
  // the last partial block: workgroup 0
  if (blockIdx.x == 0)
    for (size_t i = n_full * kBlock + threadIdx.x; i < n16; i += kProbeThreads)
      acc ^= fold(nt_load(src + i));
  sink_xor(acc, sink);
}

struct PagedProbe {
  const char* k;
  const char* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t num_pages, page_size, num_kv_heads, max_pages, max_seq_len, batch;
  int32_t run16;        // 16-byte words per (page, head) run
  int32_t parts;        // page-slot ranges per unit (work items = units x parts)
  long long run_bytes;  // bytes per (page, head) run
  uint32_t* sink;
};

// Work item i = (unit u = i / parts, part c = i % parts), unit u = (request
// b, KV head h): the part's page slots of the request, kPagedDepth (page,
// head) runs of K and of V in flight per iteration, every lane reading its
// words of each -- the way a verify workgroup walks its unit.  A slot past
// the request's length (or with an invalid page id) reads the runs of page 0
// and discards them: loads stay unconditional, and those few lines are
// served from L2 after the first.
__global__ void __launch_bounds__(kProbeThreads) paged_read_kernel(PagedProbe p) {
  const long long n_items = (long long)p.batch * p.num_kv_heads * p.parts;
  const int per = (p.max_pages + p.parts - 1) / p.parts;
  uint32_t acc = 0;
  for (long long it = blockIdx.x; it < n_items; it += gridDim.x) {
    const long long u = it / p.parts;
    const int c = (int)(it % p.parts);
    const int b = (int)(u / p.num_kv_heads), h = (int)(u % p.num_kv_heads);
    int L = p.seq_lens[b];
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    const int npg = (L + p.page_size - 1) / p.page_size;
    const int s_lo = c * per, s_hi = min(s_lo + per, npg);
    const int32_t* row = p.page_table + (long long)b * p.max_pages;
    for (int s0 = s_lo; s0 < s_hi; s0 += kPagedDepth) {
      long long off[kPagedDepth];
      bool live[kPagedDepth];
#pragma unroll
      for (int k = 0; k < kPagedDepth; ++k) {
        const int slot = s0 + k;
        const int pg = slot < s_hi ? row[slot] : -1;
        live[k] = pg >= 0 && pg < p.num_pages;
        off[k] = live[k] ? ((long long)pg * p.num_kv_heads + h) * p.run_bytes : 0;
      }
      for (int w = threadIdx.x; w < p.run16; w += kProbeThreads) {
        u32x4 kv[2 * kPagedDepth];
#pragma unroll
        for (int k = 0; k < kPagedDepth; ++k) {
          kv[2 * k] = nt_load(reinterpret_cast<const u32x4*>(p.k + off[k] + 16LL * w));
          kv[2 * k + 1] = nt_load(reinterpret_cast<const u32x4*>(p.v + off[k] + 16LL * w));
        }
#pragma unroll
        for (int k = 0; k < kPagedDepth; ++k)
          if (live[k]) acc ^= fold(kv[2 * k]) ^ fold(kv[2 * k + 1]);
      }
    }
  }
  sink_xor(acc, p.sink);
}

}  // namespace
}  // namespace sss

extern "C" {

sss_status sss_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  using namespace sss;
  if (!src || !sink || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0 || bytes % 16 != 0)
    return SSS_ERR_INVALID_ARGUMENT;
  if (bytes == 0) return SSS_OK;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kProbeGrid), dim3(kProbeThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? SSS_OK : SSS_ERR_HIP;
}

sss_status sss_probe_paged_read(const sss_paged_kv* kv, int32_t batch, uint32_t* sink,
                                void* stream) {
  using namespace sss;
  if (!kv || batch < 0 || !sink || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return SSS_ERR_INVALID_ARGUMENT;
  if (kv->dtype != SSS_F32 && kv->dtype != SSS_BF16) return SSS_ERR_UNSUPPORTED;
  if (kv->page_size < 1 || kv->num_kv_heads < 1 || kv->num_pages < 1 || kv->head_dim < 1 ||
      kv->max_pages_per_req < 1 || kv->max_seq_len < 0)
    return SSS_ERR_INVALID_ARGUMENT;
  const long long run_bytes =
      (long long)kv->page_size * kv->head_dim * (kv->dtype == SSS_BF16 ? 2 : 4);
  if (run_bytes % 16 != 0 || run_bytes / 16 > (1LL << 30)) return SSS_ERR_UNSUPPORTED;
  if (batch == 0) return SSS_OK;
  if (!kv->k || !kv->v || !kv->page_table || !kv->seq_lens ||
      reinterpret_cast<uintptr_t>(kv->k) % 16 != 0 || reinterpret_cast<uintptr_t>(kv->v) % 16 != 0)
    return SSS_ERR_INVALID_ARGUMENT;
  PagedProbe p;
  p.k = static_cast<const char*>(kv->k);
  p.v = static_cast<const char*>(kv->v);
  p.page_table = kv->page_table;
  p.seq_lens = kv->seq_lens;
  p.num_pages = kv->num_pages;
  p.page_size = kv->page_size;
  p.num_kv_heads = kv->num_kv_heads;
  p.max_pages = kv->max_pages_per_req;
  p.max_seq_len = kv->max_seq_len;
  p.batch = batch;
  p.run16 = (int32_t)(run_bytes / 16);
  p.run_bytes = run_bytes;
  p.sink = sink;
  // at least 1024 work items (four workgroups per compute unit), each unit
  // in as few parts as give that
  const long long units = (long long)batch * kv->num_kv_heads;
  long long parts = (1024 + units - 1) / units;
  if (parts > kv->max_pages_per_req) parts = kv->max_pages_per_req;
  p.parts = (int32_t)parts;
  const long long items = units * parts;
  const unsigned grid = (unsigned)(items < kProbeGrid ? items : kProbeGrid);
  hipLaunchKernelGGL(paged_read_kernel, dim3(grid), dim3(kProbeThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? SSS_OK : SSS_ERR_HIP;
}

}  // extern "C"
