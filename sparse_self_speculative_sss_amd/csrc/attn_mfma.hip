// One-item-per-workgroup launches of the matrix-core attention routine
// (attn_item.h): workgroup blockIdx.x runs item i = xcd_item(blockIdx.x, p),
// chunk i % num_chunks of unit i / num_chunks.
#include "attn_item.h"

namespace sss {
namespace {

template <int D, int NWR, int NWT, bool DRAFT, bool ELL_LDS, bool TOKENS, bool SPARSE = false,
          bool QREG = false>
__global__ void __launch_bounds__(64 * NWR * NWT, QREG ? 1 : 2) attn_mfma_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const unsigned item = xcd_item(blockIdx.x, p);
  if (p.skip_len >= 0 && p.seq_lens[(item / p.num_chunks) / p.num_kv_heads] <= p.skip_len)
    return;
  Item it;
  it.u = item / p.num_chunks;
  it.c = item % p.num_chunks;
  it.chunk = (DRAFT || SPARSE) ? p.chunk_items : p.chunk_tokens;
  it.single = p.num_chunks == 1;
  it.part_row0 = (long long)it.u * p.num_chunks * p.rows;
  // block log masses of the chunk in LDS, after the routine's own area
  it.ell_off = (int)item_lds_bytes(D, NWR, NWT, QREG);
  it.sel_off = -1;
  it.nsel_s = 0;
  // after the tiles: a single-token draft's token list, the logit staging
  // slots of a single-token verify with several row tiles, or the union of
  // a sparse verify unit's layouts
  it.list_off = (int)item_lds_bytes(D, NWR, NWT, QREG);
  attn_item<D, NWR, NWT, DRAFT, ELL_LDS, TOKENS, SPARSE, QREG>(p, it, smem);
}

}  // namespace

// LDS bytes of one workgroup: the routine's own area (K/V tiles or the
// token-group merge scratch, Q tiles, row LSEs) and optional block log masses.
size_t mfma_smem_bytes(int D, int nwr, int nwt, long long ell_floats, bool qreg) {
  return item_lds_bytes(D, nwr, nwt, qreg) + (size_t)ell_floats * 4;
}

namespace {

template <int D, int NWR, int NWT, bool DRAFT, bool ELL_LDS, bool TOKENS, bool SPARSE = false,
          bool QREG = false>
hipError_t launch_one(const AttnParams& p, size_t smem, unsigned grid, hipStream_t s) {
  auto kern = attn_mfma_kernel<D, NWR, NWT, DRAFT, ELL_LDS, TOKENS, SPARSE, QREG>;
  // dynamic LDS above 64 KiB must be opted into; allow the whole LDS once
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kMaxLds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NWR * NWT), smem, s, p);
  return hipGetLastError();
}

template <int D, int NWR, int NWT, bool DRAFT>
hipError_t launch_cfg(const AttnParams& p, hipStream_t s) {
  typedef Geo<D> G;
  static_assert((size_t)NWT * G::GROUP_BYTES >=
                    (NWT > 1 ? ((size_t)(NWT - 1) * NWR * 32 * D + 2 * NWT * NWR * 32) * 4 : 0),
                "merge scratch must fit below the Q tiles");
  const unsigned grid = (unsigned)((long long)p.batch * p.num_kv_heads * p.num_chunks);
  if (grid == 0) return hipSuccess;
  if constexpr (DRAFT) {
    if (p.block_size == 1) {
      // single-token selection: gathered tiles, token list in LDS
      if constexpr (NWR == 1) {
        const size_t smem = mfma_smem_bytes(D, NWR, NWT, 0) + (size_t)p.chunk_items * 4;
        if (smem > kMaxLds) return hipErrorInvalidValue;
        return launch_one<D, NWR, NWT, true, false, true>(p, smem, grid, s);
      } else {
        return hipErrorInvalidValue;
      }
    }
    const size_t smem = mfma_smem_bytes(D, NWR, NWT, 0);
    return launch_one<D, NWR, NWT, true, false, false>(p, smem, grid, s);
  } else {
    // block log masses in LDS (verify units that fit in one chunk, when they
    // fit) or stored to the workspace as blocks complete
    const size_t smem = mfma_smem_bytes(D, NWR, NWT, p.ell_in_lds ? p.ell_lds_floats : 0);
    if (smem > kMaxLds) return hipErrorInvalidValue;
    // single-token blocks: every token's logit is stored (never in LDS),
    // staged per wave in the tile's K rows (one row tile) or in a 4 KiB
    // slot after the tiles
    if (p.block_size == 1) {
      const size_t smem_t = mfma_smem_bytes(D, NWR, NWT, 0) + (NWR > 1 ? (size_t)NWR * NWT * 4096 : 0);
      if (smem_t > kMaxLds) return hipErrorInvalidValue;
      return launch_one<D, NWR, NWT, false, false, true>(p, smem_t, grid, s);
    }
    if (p.ell_in_lds) return launch_one<D, NWR, NWT, false, true, false>(p, smem, grid, s);
    return launch_one<D, NWR, NWT, false, false, false>(p, smem, grid, s);
  }
}

// Token groups of a one-row-tile draft workgroup: four, or one when the
// units alone fill the GPU with four waves per compute unit -- every
// one-wave workgroup is then resident from the start, with no workgroup
// round and no token-group merge (batch 128 x 8 heads, 30-segment lists on
// MI355X: 61 us with four token groups, 52 us with one; deeper register
// prefetch in the one-wave form does not help).
constexpr int kDraftNwt = 4;
constexpr long long kDraftOneWaveUnits = 1024;
int draft_token_groups(long long units) { return units >= kDraftOneWaveUnits ? 1 : kDraftNwt; }

// A verify of one row tile whose four-token-group workgroup, with the
// block log masses of its unit (or chunk) in LDS, does not fit twice in a
// compute unit runs as two-token-group workgroups (Q in registers) that do:
// while one workgroup is in its prologue (page-table, then first-tile round
// trips) or epilogue (token-group merge, block scores), the other keeps
// loading.
template <int D>
bool verify_two_per_cu(const AttnParams& p) {
  if (!p.ell_in_lds || p.block_size == 1 || ceil_div(p.rows, 32) != 1) return false;
  return mfma_smem_bytes(D, 1, 4, p.ell_lds_floats) > kMaxLds / 2 &&
         mfma_smem_bytes(D, 1, 2, p.ell_lds_floats, true) <= kMaxLds / 2;
}

template <int D>
hipError_t launch_verify_two_per_cu(const AttnParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)p.batch * p.num_kv_heads * p.num_chunks);
  if (grid == 0) return hipSuccess;
  return launch_one<D, 1, 2, false, true, false, false, true>(
      p, mfma_smem_bytes(D, 1, 2, p.ell_lds_floats, true), grid, s);
}

template <bool DRAFT>
hipError_t dispatch(const AttnParams& p, hipStream_t s) {
  const int nwr = ceil_div(p.rows, 32);
  if (!DRAFT) {
    if (p.block_size != 1 && verify_rows_fits(p)) return launch_verify_rows(p, s);
    if (p.head_dim == 128 && verify_two_per_cu<128>(p)) return launch_verify_two_per_cu<128>(p, s);
    if (p.head_dim == 64 && verify_two_per_cu<64>(p)) return launch_verify_two_per_cu<64>(p, s);
  } else if (nwr == 1 && draft_token_groups((long long)p.batch * p.num_kv_heads) == 1) {
    if (p.head_dim == 128) return launch_cfg<128, 1, 1, true>(p, s);
    if (p.head_dim == 64) return launch_cfg<64, 1, 1, true>(p, s);
  }
  if (p.head_dim == 128) {
    switch (nwr) {
      case 1: return launch_cfg<128, 1, DRAFT ? kDraftNwt : 4, DRAFT>(p, s);
      case 2: return launch_cfg<128, 2, 2, DRAFT>(p, s);
      case 3: return launch_cfg<128, 3, 1, DRAFT>(p, s);
      case 4: return launch_cfg<128, 4, 1, DRAFT>(p, s);
    }
  } else if (p.head_dim == 64) {
    switch (nwr) {
      case 1: return launch_cfg<64, 1, DRAFT ? kDraftNwt : 4, DRAFT>(p, s);
      case 2: return launch_cfg<64, 2, 2, DRAFT>(p, s);
      case 3: return launch_cfg<64, 3, 1, DRAFT>(p, s);
      case 4: return launch_cfg<64, 4, 1, DRAFT>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Token groups per workgroup for a given row count and unit count (must
// match dispatch).
int mfma_token_groups(int rows, bool draft, long long units) {
  const int nwr = ceil_div(rows, 32);
  return (draft && nwr == 1) ? draft_token_groups(units) : token_groups_for(nwr);
}

hipError_t launch_verify_mfma(const AttnParams& p, hipStream_t s) { return dispatch<false>(p, s); }

// Sparse verify: the compacted union of a unit's layouts (block ids and
// position masks) follows the routine's area in LDS; the per-block masks
// it is built from, and a scan scratch, borrow the tile area first.
size_t sparse_union_lds_bytes(int max_blocks, int n_q, int max_sel) {
  return (size_t)union_max(max_blocks, n_q, max_sel) * 8;
}
bool sparse_union_fits(int head_dim, int nwr, int max_blocks) {
  const int nwt = token_groups_for(nwr);
  const size_t tiles = (size_t)tile_buffers(nwr, nwt) *
                       ((size_t)32 * (head_dim * 2 + 16) + (size_t)head_dim * 64);
  return (size_t)max_blocks * 4 + 16 * 4 <= tiles;
}

namespace {
template <int D, int NWR, int NWT>
hipError_t launch_sparse_cfg(const AttnParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)p.batch * p.num_kv_heads * p.num_chunks);
  if (grid == 0) return hipSuccess;
  const size_t smem =
      mfma_smem_bytes(D, NWR, NWT, 0) + sparse_union_lds_bytes(p.max_blocks, p.n_q, p.max_sel);
  if (smem > kMaxLds || !sparse_union_fits(D, NWR, p.max_blocks)) return hipErrorInvalidValue;
  return launch_one<D, NWR, NWT, false, false, false, true>(p, smem, grid, s);
}
}  // namespace

hipError_t launch_sparse_verify_mfma(const AttnParams& p, hipStream_t s) {
  const int nwr = ceil_div(p.rows, 32);
  if (p.head_dim == 128) {
    switch (nwr) {
      case 1: return launch_sparse_cfg<128, 1, 4>(p, s);
      case 2: return launch_sparse_cfg<128, 2, 2>(p, s);
      case 3: return launch_sparse_cfg<128, 3, 1>(p, s);
      case 4: return launch_sparse_cfg<128, 4, 1>(p, s);
    }
  } else if (p.head_dim == 64) {
    switch (nwr) {
      case 1: return launch_sparse_cfg<64, 1, 4>(p, s);
      case 2: return launch_sparse_cfg<64, 2, 2>(p, s);
      case 3: return launch_sparse_cfg<64, 3, 1>(p, s);
      case 4: return launch_sparse_cfg<64, 4, 1>(p, s);
    }
  }
  return hipErrorInvalidValue;
}
hipError_t launch_draft_mfma(const AttnParams& p, hipStream_t s) { return dispatch<true>(p, s); }

}  // namespace sss
