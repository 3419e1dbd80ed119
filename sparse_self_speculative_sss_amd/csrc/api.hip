// C ABI of libsss: host-side validation, work planning and dispatch.  No
// state survives a call except the per-thread error message.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "sss_common.h"

namespace sss {
int mfma_token_groups(int rows, bool draft, long long units);  // attn_mfma.hip
}

namespace {

using namespace sss;

thread_local char g_err[512] = "";

sss_status fail(sss_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sss_status ok() {
  g_err[0] = '\0';
  return SSS_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

long long lcm_ll(long long a, long long b) {
  long long x = a, y = b;
  while (y) {
    const long long t = x % y;
    x = y;
    y = t;
  }
  return a / x * b;
}

// The library targets MI355X: 256 compute units, and the matrix-core kernels
// keep up to 8 waves resident per compute unit.  Planning uses these fixed
// figures so that the workspace query and the call always agree.
constexpr long long kTargetWaves = 256 * 8;
constexpr int kMinChunkTokens = 256;
// units from which a chained step of whole units runs persistently: two
// per compute unit
constexpr long long kPersistMinUnits = 256 * 2;

// Compute units of the current device (the persistent step's grid); the
// planning figures above stay fixed.
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

sss_status check_kv(const sss_paged_kv* kv, int batch) {
  if (!kv) return fail(SSS_ERR_INVALID_ARGUMENT, "kv is NULL");
  if (kv->dtype != SSS_F32 && kv->dtype != SSS_BF16)
    return fail(SSS_ERR_UNSUPPORTED, "kv->dtype %d is neither SSS_F32 nor SSS_BF16", kv->dtype);
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(SSS_ERR_UNSUPPORTED, "kv->head_dim %d (supported: 64, 128)", kv->head_dim);
  if (kv->page_size < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "kv->page_size %d < 1", kv->page_size);
  if (kv->num_kv_heads < 1)
    return fail(SSS_ERR_INVALID_ARGUMENT, "kv->num_kv_heads %d < 1", kv->num_kv_heads);
  if (kv->num_pages < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "kv->num_pages %d < 1", kv->num_pages);
  if (kv->max_pages_per_req < 1)
    return fail(SSS_ERR_INVALID_ARGUMENT, "kv->max_pages_per_req %d < 1", kv->max_pages_per_req);
  if (kv->max_seq_len < 1)
    return fail(SSS_ERR_INVALID_ARGUMENT, "kv->max_seq_len %d < 1", kv->max_seq_len);
  // kernels address the pool by 32-bit token rows (page, head, slot)
  if ((long long)kv->num_pages * kv->num_kv_heads * kv->page_size >= (1LL << 31))
    return fail(SSS_ERR_UNSUPPORTED, "the pool holds %lld token rows per tensor (limit 2^31 - 1)",
                (long long)kv->num_pages * kv->num_kv_heads * kv->page_size);
  if ((long long)kv->max_pages_per_req * kv->page_size < kv->max_seq_len)
    return fail(SSS_ERR_INVALID_ARGUMENT,
                "kv->max_pages_per_req * page_size = %lld < max_seq_len %d",
                (long long)kv->max_pages_per_req * kv->page_size, kv->max_seq_len);
  if (batch > 0) {
    if (!kv->k || !kv->v) return fail(SSS_ERR_INVALID_ARGUMENT, "kv->k or kv->v is NULL");
    if (!kv->page_table || !kv->seq_lens)
      return fail(SSS_ERR_INVALID_ARGUMENT, "kv->page_table or kv->seq_lens is NULL");
    if (!aligned(kv->k, 16) || !aligned(kv->v, 16))
      return fail(SSS_ERR_INVALID_ARGUMENT, "kv->k and kv->v must be 16-byte aligned");
    if (!aligned(kv->page_table, 4) || !aligned(kv->seq_lens, 4))
      return fail(SSS_ERR_INVALID_ARGUMENT, "page_table and seq_lens must be 4-byte aligned");
  }
  return ok();
}

// Matrix-core path: BF16 caches.  Verify reads 16-token page runs (pages of
// a multiple of 16 tokens) and scores blocks of 16 tokens, of a multiple of
// 32 (a block then ends where a 32-token tile ends), or single tokens.
// Draft reads blocks of a multiple of 16 tokens as page runs (same page
// rule), or single selected tokens gathered one row at a time (one row
// tile: G <= 32).
bool use_mfma_verify(const sss_paged_kv* kv, int block_size) {
  return kv->dtype == SSS_BF16 && kv->page_size % kSeg == 0 &&
         (block_size == kSeg || block_size % (2 * kSeg) == 0 || block_size == 1);
}
bool use_mfma_draft(const sss_paged_kv* kv, int block_size, int group) {
  if (kv->dtype != SSS_BF16) return false;
  if (block_size == 1) return group <= 32;
  return kv->page_size % kSeg == 0 && block_size % kSeg == 0;
}

struct Plan {
  bool mfma;
  int rows, num_chunks, chunk;  // chunk: tokens (verify) or list entries (draft)
  bool ell_in_lds = false;
  long long ell_lds_floats = 0;
  size_t ell_off, opart_off, lpart_off, bytes;
  size_t list_off = 0;  // sparse verify: segment list length per unit
};

void layout(Plan& pl, long long units, int head_dim, long long ell_elems) {
  size_t off = 0;
  pl.ell_off = off;
  off += align_up((size_t)ell_elems * 4, 256);
  pl.opart_off = off;
  pl.lpart_off = off;
  if (pl.num_chunks > 1) {
    off += align_up((size_t)units * pl.num_chunks * pl.rows * head_dim * 4, 256);
    pl.lpart_off = off;
    off += align_up((size_t)units * pl.num_chunks * pl.rows * 4, 256);
  }
  pl.bytes = off;
}

sss_status plan_verify(const sss_paged_kv* kv, int batch, int n_q, int hq, int block_size,
                       int max_blocks, int num_splits, Plan& pl) {
  sss_status st = check_kv(kv, batch);
  if (st != SSS_OK) return st;
  if (batch < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (n_q < 1 || n_q > 32) return fail(SSS_ERR_INVALID_ARGUMENT, "n_q %d outside [1, 32]", n_q);
  if (hq < 1 || hq % kv->num_kv_heads != 0)
    return fail(SSS_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                hq, kv->num_kv_heads);
  const int G = hq / kv->num_kv_heads;
  if ((long long)n_q * G > 128)
    return fail(SSS_ERR_UNSUPPORTED, "n_q * G = %lld rows per KV head exceeds 128", (long long)n_q * G);
  if (block_size < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "block_size %d < 1", block_size);
  if (kv->max_seq_len < n_q)
    return fail(SSS_ERR_INVALID_ARGUMENT, "kv->max_seq_len %d < n_q %d", kv->max_seq_len, n_q);
  if (max_blocks < ceil_div(kv->max_seq_len, block_size))
    return fail(SSS_ERR_INVALID_ARGUMENT, "max_blocks %d < ceil(max_seq_len / block_size) = %d",
                max_blocks, ceil_div(kv->max_seq_len, block_size));
  if (num_splits < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "num_splits %d < 0", num_splits);

  pl.mfma = use_mfma_verify(kv, block_size);
  pl.rows = n_q * G;
  const long long units = (long long)batch * kv->num_kv_heads;
  const int nwt = pl.mfma ? mfma_token_groups(pl.rows, false, units) : 1;
  const int nwr = ceil_div(pl.rows, 32);
  const long long align =
      pl.mfma ? lcm_ll((long long)nwt * 32, (long long)nwt * block_size) : (long long)block_size;
  const long long Lmax = kv->max_seq_len;
  long long S = num_splits;
  if (S == 0) {
    if (pl.mfma) {
      const long long wgs_target = kTargetWaves / ((long long)nwr * nwt);
      S = units > 0 ? (wgs_target + units - 1) / units : 1;
      const long long cap = (Lmax + kMinChunkTokens - 1) / kMinChunkTokens;
      if (S > cap) S = cap;
    } else {
      S = 1;
    }
  }
  if (S < 1) S = 1;
  long long chunk = (Lmax + S - 1) / S;
  chunk = (chunk + align - 1) / align * align;
  if (num_splits == 0 && pl.mfma && block_size != 1 && nwr == 3 && units > 0) {
    // three row tiles run as four-wave workgroups (three compute waves and
    // a load wave, verify_rows.hip) when a chunk's block masses fit in LDS:
    // split so that the grid is two of them per compute unit (8 units of
    // 80 rows x 128K tokens: 64 chunks; the plan above gave 86, so 688
    // workgroups ran in 1.34 rounds of 512)
    const long long wgs = kTargetWaves / kVerifyRowsWaves;
    long long Sr = (wgs + units - 1) / units;
    const long long cap = (Lmax + kMinChunkTokens - 1) / kMinChunkTokens;
    if (Sr > cap) Sr = cap;
    long long cr = (Lmax + Sr - 1) / Sr;
    cr = (cr + align - 1) / align * align;
    if (cr <= (1LL << 30) && verify_rows_fits_shape(kv->head_dim, pl.rows, block_size, kv->page_size,
                                            (int)cr))
      chunk = cr;
  }
  if (chunk > (1LL << 30)) return fail(SSS_ERR_UNSUPPORTED, "chunk too large");
  pl.chunk = (int)chunk;
  pl.num_chunks = (int)((Lmax + chunk - 1) / chunk);
  // block log masses in LDS: an unsplit unit's when they fit; a split
  // chunk's (one row tile) when two-token-group workgroups holding Q in
  // registers still fit twice per compute unit -- the chunk then copies them
  // to the workspace in one burst at its end instead of storing each block's
  // as it completes between the KV loads (16 requests x 4K tokens in 4
  // chunks: verify + merge 0.078 -> 0.074 ms).  Otherwise they go to the
  // workspace block by block.
  pl.ell_lds_floats = (long long)ceil_div(pl.chunk, block_size) * pl.rows;
  pl.ell_in_lds =
      pl.mfma && block_size != 1 &&
      (pl.num_chunks == 1
           ? mfma_smem_bytes(kv->head_dim, nwr, nwt, pl.ell_lds_floats) <= kMaxLds
           : (nwr == 1 &&
              mfma_smem_bytes(kv->head_dim, 1, 2, pl.ell_lds_floats, true) <= kMaxLds / 2));
  const bool ell_global = !pl.ell_in_lds || pl.num_chunks > 1;
  layout(pl, units, kv->head_dim, ell_global ? units * (long long)max_blocks * pl.rows : 0);
  return ok();
}

sss_status plan_draft(const sss_paged_kv* kv, int batch, int hq, int block_size, int max_sel,
                      int window, int num_splits, Plan& pl) {
  sss_status st = check_kv(kv, batch);
  if (st != SSS_OK) return st;
  if (batch < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (hq < 1 || hq % kv->num_kv_heads != 0)
    return fail(SSS_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                hq, kv->num_kv_heads);
  const int G = hq / kv->num_kv_heads;
  if (G > 128) return fail(SSS_ERR_UNSUPPORTED, "group size %d exceeds 128", G);
  if (block_size < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "block_size %d < 1", block_size);
  if (max_sel < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "max_sel %d < 1", max_sel);
  if (window < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "window %d < 0", window);
  if (num_splits < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "num_splits %d < 0", num_splits);

  pl.mfma = use_mfma_draft(kv, block_size, G);
  pl.rows = G;
  const long long units = (long long)batch * kv->num_kv_heads;
  const int nwt = pl.mfma ? mfma_token_groups(G, true, units) : 1;
  const int nwr = ceil_div(G, 32);
  const long long Lmax = kv->max_seq_len;
  const long long wtok = window > 0 ? (window < Lmax ? window : Lmax) : 0;
  long long list_max, align;
  if (pl.mfma && block_size == 1) {
    // single tokens: the list holds tokens, tiles take 32 of them
    list_max = (long long)max_sel + wtok;
    align = 32LL * nwt;
  } else if (pl.mfma) {
    list_max = (long long)max_sel * (block_size / kSeg) + (wtok > 0 ? (wtok + kSeg - 1) / kSeg + 1 : 0);
    align = 2LL * nwt;
  } else {
    list_max = (long long)max_sel * block_size + wtok;
    align = 1;
  }
  if (list_max < 1) list_max = 1;
  long long S = num_splits;
  if (S == 0) {
    // split only lists long enough to keep every token group of each chunk
    // busy: a short list in several chunks costs more in per-workgroup
    // latency and the merge launch than the extra workgroups bring (16
    // requests x 8 heads with 18-segment lists: 16 us unsplit, 23 us in 4
    // chunks; 8 units with 73-segment lists: 20 us in 10 chunks, 25 us
    // unsplit)
    const long long long_list = (pl.mfma && block_size % kSeg == 0) ? 64 : 64LL * kSeg;
    if (pl.mfma && list_max >= long_list) {
      const long long wgs_target = kTargetWaves / ((long long)nwr * nwt);
      S = units > 0 ? (wgs_target + units - 1) / units : 1;
    } else {
      S = 1;
    }
  }
  if (S < 1) S = 1;
  long long chunk = (list_max + S - 1) / S;
  chunk = (chunk + align - 1) / align * align;
  if (pl.mfma && block_size == 1) {
    // the chunk's token list (4 bytes per entry) sits in LDS after the tiles
    const long long room =
        ((long long)kMaxLds - (long long)mfma_smem_bytes(kv->head_dim, nwr, nwt, 0)) / 4;
    const long long cap = room / align * align;
    if (cap < align) return fail(SSS_ERR_UNSUPPORTED, "no LDS room for a token list");
    if (chunk > cap) chunk = cap;
  }
  if (chunk > (1LL << 30)) return fail(SSS_ERR_UNSUPPORTED, "chunk too large");
  pl.chunk = (int)chunk;
  pl.num_chunks = (int)((list_max + chunk - 1) / chunk);
  layout(pl, units, kv->head_dim, 0);
  return ok();
}

// Sparse verify (a layout per query position): always the matrix-core path.
// The list of a unit is the union of its positions' layouts (at most
// min(max_blocks, n_q * max_sel) blocks) in 16-token segments, then the
// window; its chunks are split like a draft list's.
sss_status plan_sparse(const sss_paged_kv* kv, int batch, int n_q, int hq, int block_size,
                       int max_sel, int window, int num_splits, Plan& pl) {
  sss_status st = check_kv(kv, batch);
  if (st != SSS_OK) return st;
  if (batch < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (n_q < 1 || n_q > 32) return fail(SSS_ERR_INVALID_ARGUMENT, "n_q %d outside [1, 32]", n_q);
  if (hq < 1 || hq % kv->num_kv_heads != 0)
    return fail(SSS_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                hq, kv->num_kv_heads);
  const int G = hq / kv->num_kv_heads;
  if ((long long)n_q * G > 128)
    return fail(SSS_ERR_UNSUPPORTED, "n_q * G = %lld rows per KV head exceeds 128", (long long)n_q * G);
  if (block_size < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "block_size %d < 1", block_size);
  if (max_sel < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "max_sel %d < 1", max_sel);
  if (window < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "window %d < 0", window);
  if (num_splits < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "num_splits %d < 0", num_splits);
  if (kv->max_seq_len < n_q)
    return fail(SSS_ERR_INVALID_ARGUMENT, "kv->max_seq_len %d < n_q %d", kv->max_seq_len, n_q);
  if (kv->dtype != SSS_BF16 || kv->page_size % kSeg != 0 || block_size % kSeg != 0)
    return fail(SSS_ERR_UNSUPPORTED,
                "sparse verify needs a BF16 cache with page_size and block_size multiples of 16");
  pl.mfma = true;
  pl.rows = n_q * G;
  const int nwr = ceil_div(pl.rows, 32);
  const int nwt = mfma_token_groups(pl.rows, false, 0);
  const int max_blocks = ceil_div(kv->max_seq_len, block_size);
  if (mfma_smem_bytes(kv->head_dim, nwr, nwt, 0) + sparse_union_lds_bytes(max_blocks, n_q, max_sel) >
          kMaxLds ||
      !sparse_union_fits(kv->head_dim, nwr, max_blocks))
    return fail(SSS_ERR_UNSUPPORTED, "%d blocks per request leave no LDS room for the layout union",
                max_blocks);
  const long long units = (long long)batch * kv->num_kv_heads;
  const long long Lmax = kv->max_seq_len;
  const long long wtok = window > 0 ? (window < Lmax ? window : Lmax) : 0;
  const long long umax = std::min<long long>(max_blocks, (long long)n_q * max_sel);
  long long list_max = umax * (block_size / kSeg) + (wtok > 0 ? (wtok + kSeg - 1) / kSeg + 1 : 0);
  if (list_max < 1) list_max = 1;
  const long long align = 2LL * nwt;
  long long S = num_splits;
  if (S == 0) {
    const long long wgs_target = kTargetWaves / ((long long)nwr * nwt);
    S = units > 0 ? (wgs_target + units - 1) / units : 1;
  }
  if (S < 1) S = 1;
  long long chunk = (list_max + S - 1) / S;
  chunk = (chunk + align - 1) / align * align;
  if (chunk > (1LL << 30)) return fail(SSS_ERR_UNSUPPORTED, "chunk too large");
  pl.chunk = (int)chunk;
  pl.num_chunks = (int)((list_max + chunk - 1) / chunk);
  layout(pl, units, kv->head_dim, 0);
  pl.list_off = pl.bytes;
  if (pl.num_chunks > 1) pl.bytes += align_up((size_t)units * 4, 256);
  return ok();
}

AttnParams base_params(const sss_paged_kv* kv, const void* q, int batch, int n_q, int hq,
                       float sm_scale, const Plan& pl) {
  AttnParams p = {};
  p.k = kv->k;
  p.v = kv->v;
  p.page_table = kv->page_table;
  p.seq_lens = kv->seq_lens;
  p.num_pages = kv->num_pages;
  p.page_size = kv->page_size;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  p.max_pages = kv->max_pages_per_req;
  p.max_seq_len = kv->max_seq_len;
  p.q = q;
  p.batch = batch;
  p.n_q = n_q;
  p.num_q_heads = hq;
  p.group = hq / kv->num_kv_heads;
  p.rows = pl.rows;
  p.scale_log2 = sm_scale * kLog2e;
  p.num_chunks = pl.num_chunks;
  p.skip_len = -1;
  return p;
}

bool same_cache(const sss_paged_kv& a, const sss_paged_kv& b) {
  return a.k == b.k && a.v == b.v && a.dtype == b.dtype && a.num_pages == b.num_pages &&
         a.page_size == b.page_size && a.num_kv_heads == b.num_kv_heads &&
         a.head_dim == b.head_dim && a.max_pages_per_req == b.max_pages_per_req &&
         a.page_table == b.page_table && a.seq_lens == b.seq_lens && a.max_seq_len == b.max_seq_len;
}

// Everything sss_fused_step derives from its arguments on the host.
struct FusedSetup {
  bool has_v = false, has_d = false, split_v = false, split_d = false;
  int rows_v = 0, group_d = 0, head_dim = 0;
  long long nv = 0, nd = 0;
  FusedPlan pl = {};
  Plan chain_draft = {};  // chained draft of split units (one-launch-per-stage kernels)
  size_t ell_off = 0, opv_off = 0, lpv_off = 0, opd_off = 0,
         lpd_off = 0, chain_off = 0, bytes = 0;
  // chained step of whole units run as two launches: the unsplit verify
  // kernel (block masses in LDS), then selection + draft per unit
  bool two_launch = false;
  // with many units the two-launch form's second launch is split in two:
  // the Top-N kernel, then the draft kernel (one wave per unit) over
  // chain_draft
  bool select_then_draft_launches = false;
  // ... or one launch of one wave per unit that selects and drafts (units
  // of at most 1024 candidates, one-chunk draft lists)
  bool select_draft_wave = false;
  Plan vplan = {};
  // chained step of whole units run as one persistent launch (persist.hip)
  bool persist = false;
  // chained step of split units of three row tiles: the load-wave verify
  // and its merge (plan fs.vplan), then one workgroup per draft chunk that
  // selects and drafts (plan rs_draft), then the draft merge; workspace
  // regions of the two plans
  bool rows_split = false;
  Plan rs_draft = {};
  size_t rs_v_off = 0, rs_d_off = 0;
};

sss_status setup_fused(const sss_verify_step* v, const sss_draft_step* d, int chained,
                       FusedSetup& fs) {
  fs = FusedSetup();
  fs.has_v = v && v->batch > 0;
  fs.has_d = d && d->batch > 0;
  if (v) {
    Plan pv;
    sss_status st = plan_verify(&v->kv, v->batch, v->n_q, v->num_q_heads, v->block_size,
                                v->max_blocks, 0, pv);
    if (st != SSS_OK) return st;
    if (!std::isfinite(v->sm_scale)) return fail(SSS_ERR_INVALID_ARGUMENT, "verify sm_scale is not finite");
    if (v->score_row_start < 0 || v->score_row_start >= v->n_q)
      return fail(SSS_ERR_INVALID_ARGUMENT, "verify score_row_start %d outside [0, n_q)",
                  v->score_row_start);
    if (v->sel) {
      if (v->window < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "verify window %d < 0", v->window);
      if (v->max_sel < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "verify max_sel %d < 1", v->max_sel);
    }
    if (fs.has_v) {
      if (!pv.mfma)
        return fail(SSS_ERR_UNSUPPORTED,
                    "fused step needs a BF16 cache with page_size a multiple of 16 and "
                    "block_size 16 or a multiple of 32");
      if (!v->q || !v->o || !v->lse || !v->block_scores)
        return fail(SSS_ERR_INVALID_ARGUMENT, "verify q, o, lse and block_scores must be non-NULL");
      if (!aligned(v->q, 16) || !aligned(v->o, 16))
        return fail(SSS_ERR_INVALID_ARGUMENT, "verify q and o must be 16-byte aligned");
      if (!aligned(v->lse, 4) || !aligned(v->block_scores, 4))
        return fail(SSS_ERR_INVALID_ARGUMENT, "verify lse and block_scores must be 4-byte aligned");
      if (v->sel && (!v->budget || !v->sel_count || !aligned(v->sel, 4) ||
                     !aligned(v->sel_count, 4) || !aligned(v->budget, 4)))
        return fail(SSS_ERR_INVALID_ARGUMENT,
                    "verify budget, sel and sel_count must be non-NULL and 4-byte aligned");
      if (v->block_size % kSeg != 0)
        return fail(SSS_ERR_UNSUPPORTED, "fused step needs block_size a multiple of 16");
      fs.rows_v = pv.rows;
      fs.nv = (long long)v->batch * v->kv.num_kv_heads;
      fs.head_dim = v->kv.head_dim;
    }
  }
  int list_max_d = 0;
  if (d) {
    Plan pd;
    sss_status st = plan_draft(&d->kv, d->batch, d->num_q_heads, d->block_size, d->max_sel,
                               d->window, 0, pd);
    if (st != SSS_OK) return st;
    if (!std::isfinite(d->sm_scale)) return fail(SSS_ERR_INVALID_ARGUMENT, "draft sm_scale is not finite");
    if (fs.has_d) {
      if (!pd.mfma)
        return fail(SSS_ERR_UNSUPPORTED,
                    "fused step needs a BF16 cache with page_size and block_size multiples of 16");
      if (pd.rows > 32)
        return fail(SSS_ERR_UNSUPPORTED, "fused step drafts groups of at most 32 heads (G = %d)",
                    pd.rows);
      if (d->block_size % kSeg != 0)
        return fail(SSS_ERR_UNSUPPORTED, "fused step needs block_size a multiple of 16");
      if (!d->q || !d->o || !d->lse || !d->sel || !d->sel_count)
        return fail(SSS_ERR_INVALID_ARGUMENT, "draft q, o, lse, sel and sel_count must be non-NULL");
      if (!aligned(d->q, 16) || !aligned(d->o, 16))
        return fail(SSS_ERR_INVALID_ARGUMENT, "draft q and o must be 16-byte aligned");
      if (!aligned(d->lse, 4) || !aligned(d->sel, 4) || !aligned(d->sel_count, 4))
        return fail(SSS_ERR_INVALID_ARGUMENT, "draft lse, sel and sel_count must be 4-byte aligned");
      if (fs.has_v && d->kv.head_dim != v->kv.head_dim)
        return fail(SSS_ERR_UNSUPPORTED, "verify and draft head_dim differ (%d, %d)",
                    v->kv.head_dim, d->kv.head_dim);
      fs.group_d = pd.rows;
      fs.head_dim = d->kv.head_dim;
      const long long wtok = d->window > 0 ? std::min<long long>(d->window, d->kv.max_seq_len) : 0;
      const long long lm = (long long)d->max_sel * (d->block_size / kSeg) +
                           (wtok > 0 ? (wtok + kSeg - 1) / kSeg + 1 : 0);
      if (lm > (1 << 28)) return fail(SSS_ERR_UNSUPPORTED, "draft list too long");
      list_max_d = (int)lm;
    }
  }
  if (chained) {
    if (!fs.has_v || !fs.has_d)
      return fail(SSS_ERR_INVALID_ARGUMENT, "a chained step needs both halves with batch > 0");
    if (!v->sel) return fail(SSS_ERR_INVALID_ARGUMENT, "a chained step needs verify->sel");
    if (d->batch != v->batch || !same_cache(d->kv, v->kv))
      return fail(SSS_ERR_INVALID_ARGUMENT,
                  "a chained step drafts the verify requests: batch and kv must be equal");
    if (d->sel != v->sel || d->sel_count != v->sel_count || d->max_sel != v->max_sel ||
        d->block_size != v->block_size)
      return fail(SSS_ERR_INVALID_ARGUMENT,
                  "a chained step reads the selection it writes: draft sel, sel_count, max_sel "
                  "and block_size must equal the verify half's");
  } else if (fs.has_v && fs.has_d && v->sel &&
             (v->sel == d->sel || v->sel_count == d->sel_count)) {
    return fail(SSS_ERR_INVALID_ARGUMENT,
                "the verify half's selection output aliases the draft half's input");
  }
  if (!fs.has_v && !fs.has_d) return ok();

  FusedPlanIn in = {};
  in.head_dim = fs.head_dim;
  in.rows_v = fs.has_v ? fs.rows_v : 0;
  in.nv = fs.nv;
  in.max_len_v = fs.has_v ? v->kv.max_seq_len : 0;
  in.block_size_v = fs.has_v ? v->block_size : kSeg;
  in.nd = (fs.has_d && !chained) ? (long long)d->batch * d->kv.num_kv_heads : 0;
  in.list_max_d = list_max_d;
  in.chained = chained ? 1 : 0;
  in.max_sel = chained ? v->max_sel : 0;
  fused_plan(in, fs.pl);
  fs.nd = in.nd;
  if (fs.has_v && fs.pl.chunk_v <= 0)
    return fail(SSS_ERR_UNSUPPORTED, "fused step: block masses of one chunk do not fit in LDS");
  if (fs.pl.lds_bytes > kMaxLds)
    return fail(SSS_ERR_UNSUPPORTED, "fused step needs %zu bytes of LDS (max_sel too large?)",
                fs.pl.lds_bytes);
  if (fs.pl.max_items > (1LL << 30))
    return fail(SSS_ERR_UNSUPPORTED, "fused step: too many work items");
  fs.split_v = fs.has_v && fs.pl.maxch_v > 1;
  fs.split_d = fs.nd > 0 && fs.pl.maxch_d > 1;
  if (chained && !fs.split_v && fs.nd == 0) {
    // Whole units of a chained step: the unsplit verify kernel keeps two
    // workgroups' worth of streaming per CU busy while no unit's selection
    // and draft hold a CU, and the selection + draft kernel then runs every
    // unit at once.  Used when that verify plan keeps its block masses in
    // LDS and needs no workspace.
    Plan vp;
    if (plan_verify(&v->kv, v->batch, v->n_q, v->num_q_heads, v->block_size, v->max_blocks, 1,
                    vp) == SSS_OK &&
        vp.mfma && vp.num_chunks == 1 && vp.ell_in_lds && vp.bytes == 0) {
      int32_t a, b;
      if (select_draft_lds(fs.head_dim, v->max_sel, v->max_blocks, a, b) <= kMaxLds) {
        fs.two_launch = true;
        fs.vplan = vp;
        // units enough for one-wave drafts: the Top-N kernel and the draft
        // kernel beat one select-and-draft workgroup per unit (batch 128 x 8
        // heads, 8K tokens on MI355X: 12.5 + 46.5 us against 75 us)
        if (mfma_token_groups(fs.group_d, true, fs.nv) == 1) {
          sss_status st = plan_draft(&d->kv, d->batch, d->num_q_heads, d->block_size, d->max_sel,
                                     d->window, 0, fs.chain_draft);
          if (st != SSS_OK) return st;
          fs.select_then_draft_launches = true;
          int32_t off;
          fs.select_draft_wave = v->max_blocks <= 1024 && fs.chain_draft.num_chunks == 1 &&
                                 select_draft_wave_lds(fs.head_dim, v->max_sel, off) <= kMaxLds / 2;
        }
      }
    }
  }
  if (fs.two_launch) {
    // At least two units per compute unit whose unsplit verify runs as
    // two-token-group workgroups (Q in registers, the unit's block masses in
    // LDS, two workgroups per CU), draft lists of at most 64 segments per
    // token group: one persistent launch verifies, scores, selects and
    // drafts every unit (persist.hip), the drafts overlapping the verify
    // stream instead of following it.  Not when one wave per unit selects
    // and drafts after the verify launch: that form is faster (batch 128 x
    // 8 heads, 8K tokens on MI355X, interleaved: 0.723 ms per step against
    // 0.735 persistent and 0.728 for the separate entry points).  The
    // workspace stays that of the two-launch form, so the size query never
    // depends on this choice.
    const int D = fs.head_dim;
    const long long ellf = fs.vplan.ell_lds_floats;
    const bool two_per_cu = fs.rows_v <= 32 && v->block_size != 1 &&
                            mfma_smem_bytes(D, 1, 4, ellf) > kMaxLds / 2 &&
                            mfma_smem_bytes(D, 1, 2, ellf, true) <= kMaxLds / 2;
    int32_t offs[5];
    const size_t lds = persist_lds(D, fs.rows_v, fs.group_d, v->max_blocks, v->max_sel, offs);
    fs.persist = !fs.select_draft_wave && two_per_cu && lds > 0 && lds <= kMaxLds / 2 &&
                 fs.group_d <= 32 &&
                 list_max_d <= 2 * 64 && fs.nv >= kPersistMinUnits;
  }
  if (chained && fs.split_v) {
    // split units draft after their selection, with the one-launch kernels
    sss_status st = plan_draft(&d->kv, d->batch, d->num_q_heads, d->block_size, d->max_sel,
                               d->window, 0, fs.chain_draft);
    if (st != SSS_OK) return st;
  }

  // Chained split units of three row tiles (65-96 rows) whose verify runs
  // as load-wave workgroups (verify_rows.hip), with a draft of one row tile
  // and four token groups per chunk (fewer than 1024 units): the verify and
  // merge of sss_verify_attn, then one launch in which each draft chunk's
  // workgroup selects its unit's Top-N and drafts its chunk, then the merge
  // of sss_draft_attn -- the per-stage calls without the Top-N launch (8
  // units of 80 rows x 128K tokens: the work list's three-row-wave verify is
  // slower than the load-wave kernel).  Its workspace is counted whenever
  // the shapes qualify.
  size_t rs_bytes = 0;
  if (chained && fs.has_v && fs.has_d && fs.nd == 0 && !fs.two_launch) {
    Plan vp, dp;
    if (plan_verify(&v->kv, v->batch, v->n_q, v->num_q_heads, v->block_size, v->max_blocks, 0,
                    vp) == SSS_OK &&
        plan_draft(&d->kv, d->batch, d->num_q_heads, d->block_size, d->max_sel, d->window, 0,
                   dp) == SSS_OK &&
        vp.mfma && dp.mfma && vp.num_chunks > 1 && ceil_div(vp.rows, 32) == 3 &&
        v->block_size != 1 && dp.rows <= 32 &&
        mfma_token_groups(dp.rows, true, fs.nv) == 4 &&
        verify_rows_fits_shape(v->kv.head_dim, vp.rows, v->block_size, v->kv.page_size,
                               vp.chunk)) {
      int32_t off_sel, cap;
      if (select_draft_split_lds(fs.head_dim, v->max_sel, v->max_blocks, off_sel, cap) <=
          kMaxLds) {
        size_t o = 0;
        fs.rs_v_off = o;
        o += align_up(vp.bytes, 256);
        fs.rs_d_off = o;
        o += align_up(dp.bytes, 256);
        rs_bytes = o;
        fs.rows_split = true;
        fs.vplan = vp;
        fs.rs_draft = dp;
      }
    }
  }

  const int D = fs.head_dim;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t at = off;
    off += align_up(n, 256);
    return at;
  };
  fs.ell_off = take(fs.split_v ? (size_t)fs.nv * v->max_blocks * fs.rows_v * 4 : 0);
  fs.opv_off = take(fs.split_v ? (size_t)fs.nv * fs.pl.maxch_v * fs.rows_v * D * 4 : 0);
  fs.lpv_off = take(fs.split_v ? (size_t)fs.nv * fs.pl.maxch_v * fs.rows_v * 4 : 0);
  fs.opd_off = take(fs.split_d ? (size_t)fs.nd * fs.pl.maxch_d * fs.group_d * D * 4 : 0);
  fs.lpd_off = take(fs.split_d ? (size_t)fs.nd * fs.pl.maxch_d * fs.group_d * 4 : 0);
  fs.chain_off = take(fs.chain_draft.bytes);
  fs.bytes = std::max(off, rs_bytes);
  return ok();
}

FinalizeParams finalize_of(const AttnParams& p, int dtype, bool draft, int num_chunks, int chunk,
                           int skip_len) {
  FinalizeParams f = {};
  f.batch = p.batch;
  f.num_kv_heads = p.num_kv_heads;
  f.n_q = p.n_q;
  f.group = p.group;
  f.rows = p.rows;
  f.head_dim = p.head_dim;
  f.num_chunks = num_chunks;
  f.chunk_tokens = draft ? 0 : chunk;
  f.chunk_items = draft ? chunk : 0;
  f.dtype = dtype;
  f.seq_lens = p.seq_lens;
  f.max_seq_len = p.max_seq_len;
  f.max_pages = p.max_pages;
  f.page_size = p.page_size;
  f.o_part = p.o_part;
  f.lse_part = p.lse_part;
  f.o = p.o;
  f.lse = p.lse;
  f.ell = draft ? nullptr : p.ell;
  f.block_scores = draft ? nullptr : p.block_scores;
  f.block_size = p.block_size;
  f.max_blocks = p.max_blocks;
  f.score_row_start = p.score_row_start;
  f.sel_count = p.sel_count;
  f.max_sel = p.max_sel;
  f.window = p.window;
  f.draft = draft ? 1 : 0;
  f.simple_list = 0;
  f.single_done = 1;
  f.skip_len = skip_len;
  return f;
}

}  // namespace

extern "C" {

const char* sss_status_string(sss_status status) {
  switch (status) {
    case SSS_OK: return "SSS_OK";
    case SSS_ERR_INVALID_ARGUMENT: return "SSS_ERR_INVALID_ARGUMENT";
    case SSS_ERR_UNSUPPORTED: return "SSS_ERR_UNSUPPORTED";
    case SSS_ERR_WORKSPACE_TOO_SMALL: return "SSS_ERR_WORKSPACE_TOO_SMALL";
    case SSS_ERR_HIP: return "SSS_ERR_HIP";
  }
  return "unknown sss_status";
}

const char* sss_last_error(void) { return g_err; }

int32_t sss_version(void) { return 100; }

size_t sss_verify_workspace_size(const sss_paged_kv* kv, int32_t batch, int32_t n_q,
                                 int32_t num_q_heads, int32_t block_size, int32_t max_blocks,
                                 int32_t num_splits) {
  Plan pl;
  if (plan_verify(kv, batch, n_q, num_q_heads, block_size, max_blocks, num_splits, pl) != SSS_OK)
    return 0;
  return pl.bytes;
}

size_t sss_draft_workspace_size(const sss_paged_kv* kv, int32_t batch, int32_t num_q_heads,
                                int32_t block_size, int32_t max_sel, int32_t window,
                                int32_t num_splits) {
  Plan pl;
  if (plan_draft(kv, batch, num_q_heads, block_size, max_sel, window, num_splits, pl) != SSS_OK)
    return 0;
  return pl.bytes;
}

}  // extern "C"

namespace {

// Host checks of sss_verify_attn's arguments other than the workspace;
// fills the plan.  SSS_OK with batch == 0 means there is nothing to do.
sss_status verify_checks(const sss_paged_kv* kv, const void* q, int32_t batch, int32_t n_q,
                         int32_t num_q_heads, float sm_scale, int32_t block_size,
                         int32_t score_row_start, int32_t num_splits, void* o, float* lse,
                         float* block_scores, int32_t max_blocks, Plan& pl) {
  sss_status st = plan_verify(kv, batch, n_q, num_q_heads, block_size, max_blocks, num_splits, pl);
  if (st != SSS_OK) return st;
  if (!std::isfinite(sm_scale)) return fail(SSS_ERR_INVALID_ARGUMENT, "sm_scale is not finite");
  if (score_row_start < 0 || score_row_start >= n_q)
    return fail(SSS_ERR_INVALID_ARGUMENT, "score_row_start %d outside [0, n_q)", score_row_start);
  if (batch == 0) return ok();
  if (!q || !o || !lse || !block_scores)
    return fail(SSS_ERR_INVALID_ARGUMENT, "q, o, lse and block_scores must be non-NULL");
  if (!aligned(q, 16) || !aligned(o, 16))
    return fail(SSS_ERR_INVALID_ARGUMENT, "q and o must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(block_scores, 4))
    return fail(SSS_ERR_INVALID_ARGUMENT, "lse and block_scores must be 4-byte aligned");
  return ok();
}

// The launches of a verify call whose arguments passed verify_checks, with
// a workspace of at least pl.bytes bytes.
sss_status verify_launch(const sss_paged_kv* kv, const void* q, int32_t batch, int32_t n_q,
                         int32_t num_q_heads, float sm_scale, int32_t block_size,
                         int32_t score_row_start, void* o, float* lse, float* block_scores,
                         int32_t max_blocks, void* workspace, const Plan& pl, void* stream) {
  char* ws = static_cast<char*>(workspace);
  AttnParams p = base_params(kv, q, batch, n_q, num_q_heads, sm_scale, pl);
  p.chunk_tokens = pl.chunk;
  p.chunk_items = 0;
  p.o_part = reinterpret_cast<float*>(ws + pl.opart_off);
  p.lse_part = reinterpret_cast<float*>(ws + pl.lpart_off);
  p.o = o;
  p.lse = lse;
  p.block_size = block_size;
  p.max_blocks = max_blocks;
  p.score_row_start = score_row_start;
  p.ell = reinterpret_cast<float*>(ws + pl.ell_off);
  p.block_scores = block_scores;
  p.ell_in_lds = pl.ell_in_lds ? 1 : 0;
  p.ell_lds_floats = (int32_t)pl.ell_lds_floats;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = pl.mfma ? launch_verify_mfma(p, s) : launch_attn_simple(p, kv->dtype, false, s);
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "verify launch: %s", hipGetErrorString(e));
  // an unsplit matrix-core launch finalises the block scores itself
  if (pl.mfma && pl.num_chunks == 1) return ok();

  FinalizeParams f = {};
  f.batch = batch;
  f.num_kv_heads = kv->num_kv_heads;
  f.n_q = n_q;
  f.group = p.group;
  f.rows = pl.rows;
  f.head_dim = kv->head_dim;
  f.num_chunks = pl.num_chunks;
  f.chunk_tokens = pl.chunk;
  f.dtype = kv->dtype;
  f.seq_lens = kv->seq_lens;
  f.max_seq_len = kv->max_seq_len;
  f.max_pages = kv->max_pages_per_req;
  f.page_size = kv->page_size;
  f.o_part = p.o_part;
  f.lse_part = p.lse_part;
  f.o = o;
  f.lse = lse;
  f.ell = p.ell;
  f.block_scores = block_scores;
  f.block_size = block_size;
  f.max_blocks = max_blocks;
  f.score_row_start = score_row_start;
  f.single_done = pl.mfma ? 1 : 0;
  f.skip_len = -1;
  e = launch_finalize(f, s);
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "verify finalize launch: %s", hipGetErrorString(e));
  return ok();
}


// ---- allocation-free verify: the workspace is a static device array ----

// Scratch of sss_verify_attn_noalloc.  In host code `scratch` names a
// host-side shadow, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device (each GPU holds its own
// copy), kept per device below.
static __device__ __align__(256) char scratch[SSS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept until the process ends.
sss_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSS_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SSS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return SSS_OK;
}

}  // namespace

extern "C" {

sss_status sss_verify_attn(const sss_paged_kv* kv, const void* q, int32_t batch, int32_t n_q,
                           int32_t num_q_heads, float sm_scale, int32_t block_size,
                           int32_t score_row_start, int32_t num_splits, void* o, float* lse,
                           float* block_scores, int32_t max_blocks, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Plan pl;
  sss_status st = verify_checks(kv, q, batch, n_q, num_q_heads, sm_scale, block_size,
                                score_row_start, num_splits, o, lse, block_scores, max_blocks, pl);
  if (st != SSS_OK || batch == 0) return st;
  if (workspace_bytes < pl.bytes)
    return fail(SSS_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes %zu < required %zu", workspace_bytes,
                pl.bytes);
  if (pl.bytes > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(SSS_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  return verify_launch(kv, q, batch, n_q, num_q_heads, sm_scale, block_size, score_row_start, o,
                       lse, block_scores, max_blocks, workspace, pl, stream);
}

sss_status sss_verify_attn_noalloc(const sss_paged_kv* kv, const void* q, int32_t batch,
                                   int32_t n_q, int32_t num_q_heads, float sm_scale,
                                   int32_t block_size, int32_t score_row_start, int32_t num_splits,
                                   void* o, float* lse, float* block_scores, int32_t max_blocks,
                                   void* stream) {
  Plan pl;
  sss_status st = verify_checks(kv, q, batch, n_q, num_q_heads, sm_scale, block_size,
                                score_row_start, num_splits, o, lse, block_scores, max_blocks, pl);
  if (st != SSS_OK || batch == 0) return st;
  if (pl.bytes > (size_t)SSS_NOALLOC_SCRATCH_BYTES)
    return fail(SSS_ERR_WORKSPACE_TOO_SMALL,
                "these arguments need %zu bytes of scratch; sss_verify_attn_noalloc has %zu "
                "(call sss_verify_attn with a workspace, or pass fewer splits or requests)",
                pl.bytes, (size_t)SSS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (pl.bytes > 0) {
    st = scratch_of_current_device(&ws);
    if (st != SSS_OK) return st;
  }
  return verify_launch(kv, q, batch, n_q, num_q_heads, sm_scale, block_size, score_row_start, o,
                       lse, block_scores, max_blocks, ws, pl, stream);
}

sss_status sss_block_topk(const float* block_scores, int32_t batch, int32_t num_kv_heads,
                          int32_t max_blocks, const int32_t* seq_lens, int32_t block_size,
                          const int32_t* budget, int32_t window, int32_t* sel,
                          int32_t* sel_count, int32_t max_sel, void* stream) {
  if (batch < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (num_kv_heads < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "num_kv_heads %d < 1", num_kv_heads);
  if (max_blocks < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "max_blocks %d < 1", max_blocks);
  if (block_size < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "block_size %d < 1", block_size);
  if (window < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "window %d < 0", window);
  if (max_sel < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "max_sel %d < 1", max_sel);
  if (batch == 0) return ok();
  if (!block_scores || !seq_lens || !budget || !sel || !sel_count)
    return fail(SSS_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(block_scores, 4) || !aligned(seq_lens, 4) || !aligned(budget, 4) ||
      !aligned(sel, 4) || !aligned(sel_count, 4))
    return fail(SSS_ERR_INVALID_ARGUMENT, "arrays must be 4-byte aligned");
  hipError_t e = launch_topk(block_scores, batch, num_kv_heads, max_blocks, seq_lens, block_size,
                             budget, window, sel, sel_count, max_sel, -1,
                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "topk launch: %s", hipGetErrorString(e));
  return ok();
}

sss_status sss_draft_attn(const sss_paged_kv* kv, const void* q, int32_t batch,
                          int32_t num_q_heads, float sm_scale, int32_t block_size,
                          const int32_t* sel, const int32_t* sel_count, int32_t max_sel,
                          int32_t window, int32_t num_splits, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  sss_status st = plan_draft(kv, batch, num_q_heads, block_size, max_sel, window, num_splits, pl);
  if (st != SSS_OK) return st;
  if (!std::isfinite(sm_scale)) return fail(SSS_ERR_INVALID_ARGUMENT, "sm_scale is not finite");
  if (batch == 0) return ok();
  if (!q || !o || !lse || !sel || !sel_count)
    return fail(SSS_ERR_INVALID_ARGUMENT, "q, o, lse, sel and sel_count must be non-NULL");
  if (!aligned(q, 16) || !aligned(o, 16))
    return fail(SSS_ERR_INVALID_ARGUMENT, "q and o must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(sel, 4) || !aligned(sel_count, 4))
    return fail(SSS_ERR_INVALID_ARGUMENT, "lse, sel and sel_count must be 4-byte aligned");
  if (workspace_bytes < pl.bytes)
    return fail(SSS_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes %zu < required %zu", workspace_bytes,
                pl.bytes);
  if (pl.bytes > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(SSS_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  AttnParams p = base_params(kv, q, batch, 1, num_q_heads, sm_scale, pl);
  p.chunk_tokens = 0;
  p.chunk_items = pl.chunk;
  p.o_part = reinterpret_cast<float*>(ws + pl.opart_off);
  p.lse_part = reinterpret_cast<float*>(ws + pl.lpart_off);
  p.o = o;
  p.lse = lse;
  p.block_size = block_size;
  p.sel = sel;
  p.sel_count = sel_count;
  p.max_sel = max_sel;
  p.window = window;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = pl.mfma ? launch_draft_mfma(p, s) : launch_attn_simple(p, kv->dtype, true, s);
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "draft launch: %s", hipGetErrorString(e));
  if (pl.num_chunks > 1) {
    FinalizeParams f = {};
    f.batch = batch;
    f.num_kv_heads = kv->num_kv_heads;
    f.n_q = 1;
    f.group = p.group;
    f.rows = pl.rows;
    f.head_dim = kv->head_dim;
    f.num_chunks = pl.num_chunks;
    f.chunk_items = pl.chunk;
    f.dtype = kv->dtype;
    f.seq_lens = kv->seq_lens;
    f.max_seq_len = kv->max_seq_len;
    f.max_pages = kv->max_pages_per_req;
    f.page_size = kv->page_size;
    f.o_part = p.o_part;
    f.lse_part = p.lse_part;
    f.o = o;
    f.lse = lse;
    f.ell = nullptr;
    f.block_size = block_size;
    f.sel_count = sel_count;
    f.max_sel = max_sel;
    f.window = window;
    f.draft = 1;
    // lists counted in 16-token segments, or token by token
    f.simple_list = (pl.mfma && block_size % kSeg == 0) ? 0 : 1;
    f.single_done = pl.mfma ? 1 : 0;
    f.skip_len = -1;
    e = launch_finalize(f, s);
    if (e != hipSuccess) return fail(SSS_ERR_HIP, "draft finalize launch: %s", hipGetErrorString(e));
  }
  return ok();
}

size_t sss_sparse_verify_workspace_size(const sss_paged_kv* kv, int32_t batch, int32_t n_q,
                                        int32_t num_q_heads, int32_t block_size, int32_t max_sel,
                                        int32_t window, int32_t num_splits) {
  Plan pl;
  if (plan_sparse(kv, batch, n_q, num_q_heads, block_size, max_sel, window, num_splits, pl) !=
      SSS_OK)
    return 0;
  return pl.bytes;
}

sss_status sss_sparse_verify_attn(const sss_paged_kv* kv, const void* q, int32_t batch,
                                  int32_t n_q, int32_t num_q_heads, float sm_scale,
                                  int32_t block_size, const int32_t* row_sel,
                                  const int32_t* row_sel_count, int32_t max_sel, int32_t window,
                                  int32_t num_splits, void* o, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Plan pl;
  sss_status st =
      plan_sparse(kv, batch, n_q, num_q_heads, block_size, max_sel, window, num_splits, pl);
  if (st != SSS_OK) return st;
  if (!std::isfinite(sm_scale)) return fail(SSS_ERR_INVALID_ARGUMENT, "sm_scale is not finite");
  if (batch == 0) return ok();
  if (!q || !o || !lse || !row_sel || !row_sel_count)
    return fail(SSS_ERR_INVALID_ARGUMENT, "q, o, lse, row_sel and row_sel_count must be non-NULL");
  if (!aligned(q, 16) || !aligned(o, 16))
    return fail(SSS_ERR_INVALID_ARGUMENT, "q and o must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(row_sel, 4) || !aligned(row_sel_count, 4))
    return fail(SSS_ERR_INVALID_ARGUMENT, "lse, row_sel and row_sel_count must be 4-byte aligned");
  if (workspace_bytes < pl.bytes)
    return fail(SSS_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes %zu < required %zu", workspace_bytes,
                pl.bytes);
  if (pl.bytes > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(SSS_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  AttnParams p = base_params(kv, q, batch, n_q, num_q_heads, sm_scale, pl);
  p.chunk_tokens = 0;
  p.chunk_items = pl.chunk;
  p.o_part = reinterpret_cast<float*>(ws + pl.opart_off);
  p.lse_part = reinterpret_cast<float*>(ws + pl.lpart_off);
  p.o = o;
  p.lse = lse;
  p.block_size = block_size;
  p.max_blocks = ceil_div(kv->max_seq_len, block_size);
  p.sel = row_sel;
  p.sel_count = row_sel_count;
  p.max_sel = max_sel;
  p.window = window;
  p.list_len = pl.num_chunks > 1 ? reinterpret_cast<int32_t*>(ws + pl.list_off) : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_sparse_verify_mfma(p, s);
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "sparse verify launch: %s", hipGetErrorString(e));
  if (pl.num_chunks == 1) return ok();
  FinalizeParams f = {};
  f.batch = batch;
  f.num_kv_heads = kv->num_kv_heads;
  f.n_q = n_q;
  f.group = p.group;
  f.rows = pl.rows;
  f.head_dim = kv->head_dim;
  f.num_chunks = pl.num_chunks;
  f.chunk_items = pl.chunk;
  f.dtype = kv->dtype;
  f.seq_lens = kv->seq_lens;
  f.max_seq_len = kv->max_seq_len;
  f.max_pages = kv->max_pages_per_req;
  f.page_size = kv->page_size;
  f.o_part = p.o_part;
  f.lse_part = p.lse_part;
  f.o = o;
  f.lse = lse;
  f.ell = nullptr;
  f.block_size = block_size;
  f.max_blocks = p.max_blocks;
  f.single_done = 1;
  f.skip_len = -1;
  f.list_len = p.list_len;
  e = launch_finalize(f, s);
  if (e != hipSuccess)
    return fail(SSS_ERR_HIP, "sparse verify finalize launch: %s", hipGetErrorString(e));
  return ok();
}

sss_status sss_kv_write(const sss_paged_kv* kv, const void* k_new, const void* v_new,
                        int32_t batch, int32_t n_new, const int32_t* pos0, void* stream) {
  sss_status st = check_kv(kv, batch);
  if (st != SSS_OK) return st;
  if (batch < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (n_new < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "n_new %d < 0", n_new);
  if (batch == 0 || n_new == 0) return ok();
  if (!k_new || !v_new || !pos0)
    return fail(SSS_ERR_INVALID_ARGUMENT, "k_new, v_new and pos0 must be non-NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos0, 4))
    return fail(SSS_ERR_INVALID_ARGUMENT, "k_new and v_new must be 16-byte aligned, pos0 4-byte");
  KvWriteParams p = {};
  p.k = const_cast<void*>(kv->k);
  p.v = const_cast<void*>(kv->v);
  p.k_new = k_new;
  p.v_new = v_new;
  p.page_table = kv->page_table;
  p.pos0 = pos0;
  p.num_pages = kv->num_pages;
  p.page_size = kv->page_size;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  p.max_pages = kv->max_pages_per_req;
  p.elem_bytes = kv->dtype == SSS_BF16 ? 2 : 4;
  p.batch = batch;
  p.n_new = n_new;
  hipError_t e = launch_kv_write(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "kv write launch: %s", hipGetErrorString(e));
  return ok();
}

sss_status sss_kv_commit(const int32_t* seq_lens, const int32_t* keep, int32_t batch, int32_t n_q,
                         int32_t* new_seq_lens, void* stream) {
  if (batch < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (n_q < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "n_q %d < 1", n_q);
  if (batch == 0) return ok();
  if (!seq_lens || !keep || !new_seq_lens)
    return fail(SSS_ERR_INVALID_ARGUMENT, "seq_lens, keep and new_seq_lens must be non-NULL");
  if (!aligned(seq_lens, 4) || !aligned(keep, 4) || !aligned(new_seq_lens, 4))
    return fail(SSS_ERR_INVALID_ARGUMENT, "arrays must be 4-byte aligned");
  hipError_t e = launch_kv_commit(seq_lens, keep, batch, n_q, new_seq_lens,
                                  reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "kv commit launch: %s", hipGetErrorString(e));
  return ok();
}

sss_status sss_merge(const float* o_parts, const float* lse_parts, int32_t num_parts, int32_t rows,
                     int32_t head_dim, void* o, int32_t o_dtype, float* lse, void* stream) {
  if (num_parts < 1) return fail(SSS_ERR_INVALID_ARGUMENT, "num_parts %d < 1", num_parts);
  if (rows < 0) return fail(SSS_ERR_INVALID_ARGUMENT, "rows %d < 0", rows);
  if (head_dim < 1 || head_dim > 1024)
    return fail(SSS_ERR_INVALID_ARGUMENT, "head_dim %d outside [1, 1024]", head_dim);
  if (o_dtype != SSS_F32 && o_dtype != SSS_BF16)
    return fail(SSS_ERR_UNSUPPORTED, "o_dtype %d is neither SSS_F32 nor SSS_BF16", o_dtype);
  if (rows == 0) return ok();
  if (!o_parts || !lse_parts || !o) return fail(SSS_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(o, o_dtype == SSS_F32 ? 4 : 2) ||
      (lse && !aligned(lse, 4)))
    return fail(SSS_ERR_INVALID_ARGUMENT, "misaligned array");
  hipError_t e = launch_merge(o_parts, lse_parts, num_parts, rows, head_dim, o, o_dtype, lse,
                              reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  return ok();
}

size_t sss_fused_workspace_size(const sss_verify_step* verify, const sss_draft_step* draft,
                                int32_t chained) {
  FusedSetup fs;
  if (setup_fused(verify, draft, chained, fs) != SSS_OK) return 0;
  return fs.bytes;
}

int32_t sss_fused_step_form(const sss_verify_step* verify, const sss_draft_step* draft,
                            int32_t chained) {
  FusedSetup fs;
  if (setup_fused(verify, draft, chained, fs) != SSS_OK) return -1;
  if (!fs.has_v && !fs.has_d) return SSS_FUSED_NOTHING;
  if (fs.persist) return SSS_FUSED_PERSISTENT;
  if (fs.rows_split) return SSS_FUSED_ROWS_SPLIT;
  if (fs.two_launch) return SSS_FUSED_TWO_LAUNCH;
  return SSS_FUSED_WORK_LIST;
}

// The fused step; `mark`, when given, is recorded on the stream once the
// launch that produces the verify outputs is enqueued (two-launch form:
// after the verify kernel; persistent form: after its one launch; work
// list: after the work-list launch, before the launches of split units).
static sss_status fused_step_impl(const sss_verify_step* verify, const sss_draft_step* draft,
                                  int32_t chained, void* workspace, size_t workspace_bytes,
                                  void* stream, hipEvent_t mark) {
  FusedSetup fs;
  sss_status st = setup_fused(verify, draft, chained, fs);
  if (st != SSS_OK) return st;
  auto record_mark = [&]() -> hipError_t {
    return mark ? hipEventRecord(mark, reinterpret_cast<hipStream_t>(stream)) : hipSuccess;
  };
  if (!fs.has_v && !fs.has_d) {
    const hipError_t e = record_mark();
    if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step mark: %s", hipGetErrorString(e));
    return ok();
  }
  if (workspace_bytes < fs.bytes)
    return fail(SSS_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes %zu < required %zu", workspace_bytes,
                fs.bytes);
  if (fs.bytes > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(SSS_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  AttnParams pv = {};
  pv.skip_len = -1;
  if (fs.has_v) {
    const sss_verify_step* v = verify;
    Plan pl = {};
    pl.rows = fs.rows_v;
    pl.num_chunks = fs.pl.maxch_v;
    pv = base_params(&v->kv, v->q, v->batch, v->n_q, v->num_q_heads, v->sm_scale, pl);
    pv.chunk_tokens = fs.pl.chunk_v;
    pv.o_part = reinterpret_cast<float*>(ws + fs.opv_off);
    pv.lse_part = reinterpret_cast<float*>(ws + fs.lpv_off);
    pv.o = v->o;
    pv.lse = v->lse;
    pv.block_size = v->block_size;
    pv.max_blocks = v->max_blocks;
    pv.score_row_start = v->score_row_start;
    pv.ell = reinterpret_cast<float*>(ws + fs.ell_off);
    pv.block_scores = v->block_scores;
  }
  AttnParams pd = {};
  pd.skip_len = -1;
  if (fs.has_d) {
    const sss_draft_step* d = draft;
    Plan pl = {};
    pl.rows = fs.group_d;
    pl.num_chunks = std::max(fs.pl.maxch_d, 1);
    pd = base_params(&d->kv, d->q, d->batch, 1, d->num_q_heads, d->sm_scale, pl);
    pd.chunk_items = fs.pl.chunk_d;
    pd.o_part = reinterpret_cast<float*>(ws + fs.opd_off);
    pd.lse_part = reinterpret_cast<float*>(ws + fs.lpd_off);
    pd.o = d->o;
    pd.lse = d->lse;
    pd.block_size = d->block_size;
    pd.sel = d->sel;
    pd.sel_count = d->sel_count;
    pd.max_sel = d->max_sel;
    pd.window = d->window;
  }
  FusedParams f = {};
  f.nv_units = (int32_t)fs.nv;
  f.nd_units = (int32_t)fs.nd;
  f.chunk_v = fs.pl.chunk_v;
  f.maxch_v = fs.pl.maxch_v;
  f.chunk_d = fs.pl.chunk_d;
  f.maxch_d = fs.pl.maxch_d;
  const bool topk = fs.has_v && verify->sel;
  f.topk = topk ? 1 : 0;
  if (topk) {
    f.topk_window = verify->window;
    f.max_sel = verify->max_sel;
    f.budget = verify->budget;
    f.sel = verify->sel;
    f.sel_count = verify->sel_count;
  }
  f.chained = chained ? 1 : 0;
  f.off_ell = fs.pl.off_ell;
  f.off_sel = fs.pl.off_sel;
  if (fs.persist) {
    const sss_verify_step* v = verify;
    AttnParams p = base_params(&v->kv, v->q, v->batch, v->n_q, v->num_q_heads, v->sm_scale, fs.vplan);
    p.o = v->o;
    p.lse = v->lse;
    p.block_size = v->block_size;
    p.max_blocks = v->max_blocks;
    p.score_row_start = v->score_row_start;
    p.block_scores = v->block_scores;
    // two workgroups per compute unit, a multiple of 8 (the XCD-aware unit
    // order assumes slot i runs on XCD i % 8)
    const int grid = std::max(8, 2 * device_cus() / 8 * 8);
    hipError_t e = launch_persist_step(p, pd, v->max_sel, v->window, v->budget, v->sel,
                                       v->sel_count, grid, s);
    if (e == hipSuccess) e = record_mark();
    if (e != hipSuccess)
      return fail(SSS_ERR_HIP, "fused step persistent launch: %s", hipGetErrorString(e));
    return ok();
  }
  if (fs.rows_split) {
    const sss_verify_step* v = verify;
    const Plan& vp = fs.vplan;
    const Plan& dp = fs.rs_draft;
    // the verify and merge of sss_verify_attn
    char* wv = ws + fs.rs_v_off;
    AttnParams p = base_params(&v->kv, v->q, v->batch, v->n_q, v->num_q_heads, v->sm_scale, vp);
    p.chunk_tokens = vp.chunk;
    p.o_part = reinterpret_cast<float*>(wv + vp.opart_off);
    p.lse_part = reinterpret_cast<float*>(wv + vp.lpart_off);
    p.o = v->o;
    p.lse = v->lse;
    p.block_size = v->block_size;
    p.max_blocks = v->max_blocks;
    p.score_row_start = v->score_row_start;
    p.ell = reinterpret_cast<float*>(wv + vp.ell_off);
    p.block_scores = v->block_scores;
    p.ell_in_lds = vp.ell_in_lds ? 1 : 0;
    p.ell_lds_floats = (int32_t)vp.ell_lds_floats;
    hipError_t e = launch_verify_mfma(p, s);
    if (e == hipSuccess)
      e = launch_finalize(finalize_of(p, SSS_BF16, false, vp.num_chunks, vp.chunk, -1), s);
    if (e == hipSuccess) e = record_mark();
    if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step verify launch: %s", hipGetErrorString(e));
    // selection and draft per draft chunk, then the merge of sss_draft_attn
    AttnParams q = pd;
    q.num_chunks = dp.num_chunks;
    q.chunk_tokens = 0;
    q.chunk_items = dp.chunk;
    q.o_part = reinterpret_cast<float*>(ws + fs.rs_d_off + dp.opart_off);
    q.lse_part = reinterpret_cast<float*>(ws + fs.rs_d_off + dp.lpart_off);
    q.skip_len = -1;
    select_draft_split_lds(fs.head_dim, f.max_sel, v->max_blocks, f.off_sel, f.fin_keys_cap);
    e = launch_select_draft_split(f, p, q, fs.head_dim, s);
    if (e == hipSuccess && dp.num_chunks > 1)
      e = launch_finalize(finalize_of(q, SSS_BF16, true, dp.num_chunks, dp.chunk, -1), s);
    if (e != hipSuccess)
      return fail(SSS_ERR_HIP, "fused step select + draft launch: %s", hipGetErrorString(e));
    return ok();
  }
  if (fs.two_launch) {
    const sss_verify_step* v = verify;
    const Plan& vp = fs.vplan;
    AttnParams p = base_params(&v->kv, v->q, v->batch, v->n_q, v->num_q_heads, v->sm_scale, vp);
    p.chunk_tokens = vp.chunk;
    p.o = v->o;
    p.lse = v->lse;
    p.block_size = v->block_size;
    p.max_blocks = v->max_blocks;
    p.score_row_start = v->score_row_start;
    p.block_scores = v->block_scores;
    p.ell_in_lds = 1;
    p.ell_lds_floats = (int32_t)vp.ell_lds_floats;
    hipError_t e = launch_verify_mfma(p, s);
    if (e == hipSuccess) e = record_mark();
    if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step verify launch: %s", hipGetErrorString(e));
    if (fs.select_draft_wave) {
      select_draft_wave_lds(fs.head_dim, f.max_sel, f.off_sel);
      AttnParams q = pd;
      q.num_chunks = 1;
      q.chunk_tokens = 0;
      q.chunk_items = fs.chain_draft.chunk;
      q.skip_len = -1;
      e = launch_select_draft_wave(f, pv, q, fs.head_dim, s);
      if (e != hipSuccess)
        return fail(SSS_ERR_HIP, "fused step select + draft launch: %s", hipGetErrorString(e));
      return ok();
    }
    if (fs.select_then_draft_launches) {
      e = launch_topk(v->block_scores, v->batch, v->kv.num_kv_heads, v->max_blocks, v->kv.seq_lens,
                      v->block_size, v->budget, v->window, v->sel, v->sel_count, v->max_sel, -1, s);
      if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step topk launch: %s", hipGetErrorString(e));
      const Plan& cp = fs.chain_draft;
      AttnParams q = pd;
      q.num_chunks = cp.num_chunks;
      q.chunk_tokens = 0;
      q.chunk_items = cp.chunk;
      q.o_part = reinterpret_cast<float*>(ws + fs.chain_off + cp.opart_off);
      q.lse_part = reinterpret_cast<float*>(ws + fs.chain_off + cp.lpart_off);
      q.skip_len = -1;
      e = launch_draft_mfma(q, s);
      if (e == hipSuccess && cp.num_chunks > 1)
        e = launch_finalize(finalize_of(q, SSS_BF16, true, cp.num_chunks, cp.chunk, -1), s);
      if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step draft launch: %s", hipGetErrorString(e));
      return ok();
    }
    select_draft_lds(fs.head_dim, f.max_sel, v->max_blocks, f.off_sel, f.off_ell);
    e = launch_select_draft(f, pv, pd, fs.head_dim, s);
    if (e != hipSuccess)
      return fail(SSS_ERR_HIP, "fused step select + draft launch: %s", hipGetErrorString(e));
    return ok();
  }
  hipError_t e = launch_fused(f, pv, pd, fs.pl, fs.head_dim, s);
  if (e == hipSuccess) e = record_mark();
  if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step launch: %s", hipGetErrorString(e));

  // units split over several chunks: merge and score, select, then draft
  if (fs.split_v) {
    // a unit's partials small enough for one workgroup: merge, score and
    // select in one launch; otherwise spread the merge, then select
    const size_t unit_partials = (size_t)fs.pl.maxch_v * fs.rows_v * fs.head_dim * 4;
    bool drafted = false;
    if (unit_partials <= ((size_t)1 << 20)) {
      // a chained draft whose lists need no split runs in the finishing
      // workgroup, right after the unit's selection
      const bool fin_draft = chained && fs.chain_draft.num_chunks == 1 && fs.group_d <= 32;
      const size_t lds = finish_lds(f, fs.head_dim, verify->max_blocks, fin_draft);
      e = launch_fused_finish(f, pv, pd, fs.head_dim, lds, s);
      if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step finish launch: %s", hipGetErrorString(e));
      drafted = fin_draft;
    } else {
      e = launch_finalize(finalize_of(pv, SSS_BF16, false, fs.pl.maxch_v, fs.pl.chunk_v,
                                      fs.pl.chunk_v), s);
      if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step merge launch: %s", hipGetErrorString(e));
      if (topk) {
        e = launch_topk(verify->block_scores, verify->batch, verify->kv.num_kv_heads,
                        verify->max_blocks, verify->kv.seq_lens, verify->block_size,
                        verify->budget, verify->window, verify->sel, verify->sel_count,
                        verify->max_sel, fs.pl.chunk_v, s);
        if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step topk launch: %s", hipGetErrorString(e));
      }
    }
    if (chained && !drafted) {
      const Plan& cp = fs.chain_draft;
      AttnParams q = pd;
      q.num_chunks = cp.num_chunks;
      q.chunk_tokens = 0;
      q.chunk_items = cp.chunk;
      q.o_part = reinterpret_cast<float*>(ws + fs.chain_off + cp.opart_off);
      q.lse_part = reinterpret_cast<float*>(ws + fs.chain_off + cp.lpart_off);
      q.skip_len = fs.pl.chunk_v;
      e = launch_draft_mfma(q, s);
      if (e == hipSuccess && cp.num_chunks > 1)
        e = launch_finalize(finalize_of(q, SSS_BF16, true, cp.num_chunks, cp.chunk, fs.pl.chunk_v),
                            s);
      if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step draft launch: %s", hipGetErrorString(e));
    }
  }
  if (fs.split_d) {
    e = launch_finalize(finalize_of(pd, SSS_BF16, true, fs.pl.maxch_d, fs.pl.chunk_d, -1), s);
    if (e != hipSuccess) return fail(SSS_ERR_HIP, "fused step merge launch: %s", hipGetErrorString(e));
  }
  return ok();
}

sss_status sss_fused_step(const sss_verify_step* verify, const sss_draft_step* draft,
                          int32_t chained, void* workspace, size_t workspace_bytes, void* stream) {
  return fused_step_impl(verify, draft, chained, workspace, workspace_bytes, stream, nullptr);
}

sss_status sss_fused_step_marked(const sss_verify_step* verify, const sss_draft_step* draft,
                                 int32_t chained, void* workspace, size_t workspace_bytes,
                                 void* stream, void* verify_done) {
  return fused_step_impl(verify, draft, chained, workspace, workspace_bytes, stream,
                         reinterpret_cast<hipEvent_t>(verify_done));
}

}  // extern "C"
