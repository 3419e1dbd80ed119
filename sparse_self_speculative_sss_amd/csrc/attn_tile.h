// Per-tile arithmetic of the matrix-core attention routines, as small
// wave-level helpers over one 32-row tile: S^T = K Q^T, the masked online
// softmax (log2 domain, lazy rescaling) and O^T += V^T P^T, with the LDS
// tile layouts of attn_item.h.  Used by the persistent step kernel.
#pragma once

#include "attn_item.h"

namespace sss {

template <int D>
struct Acc {
  f32x16 o[Geo<D>::MT];
  float m, l;
};

template <int D>
__device__ __forceinline__ void acc_init(Acc<D>& a) {
#pragma unroll
  for (int mt = 0; mt < Geo<D>::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) a.o[mt][i] = 0.f;
  a.m = neg_inf();
  a.l = 0.f;
}

// The Q^T operand of one row tile, read from global memory: lane (rl, hl)
// holds 16-byte chunk 2 ks + hl of its row (the layout the first MFMA of a
// tile reads).  `row` points at the row's head_dim elements; rows without
// one are zero.  A negative scale is folded in as an exact sign flip.
template <int D>
__device__ __forceinline__ void load_qreg(bf16x8 (&q)[Geo<D>::KS], const bf16* row, bool neg) {
  const int hl = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < Geo<D>::KS; ++ks) {
    uint4 v = {0u, 0u, 0u, 0u};
    if (row) v = *reinterpret_cast<const uint4*>(row + 16 * ks + 8 * hl);
    if (neg) {
      v.x ^= 0x80008000u;
      v.y ^= 0x80008000u;
      v.z ^= 0x80008000u;
      v.w ^= 0x80008000u;
    }
    q[ks] = *reinterpret_cast<const bf16x8*>(&v);
  }
}

// Masked logits of a tile (S^T in `sacc`) for a row at position pos_r:
// interior tiles need no mask.  Returns the row's (lane-local) max.
__device__ __forceinline__ float mask_logits(const f32x16& sacc, float (&s)[16], const Seg& ca,
                                             const Seg& cb, bool interior, int pos_r, int hl) {
  float mx = neg_inf();
  if (interior) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = sacc[i];
      mx = fmaxf(mx, s[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = (i >> 2) * 8 + 4 * hl + (i & 3);
      const Seg& sg = (m < kSeg) ? ca : cb;
      const int tok = sg.t0 + (m % kSeg);
      const bool ok = tok >= sg.lo && tok < sg.hi && tok <= pos_r;
      s[i] = ok ? sacc[i] : neg_inf();
      mx = fmaxf(mx, s[i]);
    }
  }
  return mx;
}

// Online softmax of a tile's masked logits into `a` (lazy rescaling as in
// attn_item: the reference max moves only past kRescaleSlack), then
// O^T += V^T P^T from the tile's V^T in LDS.  `extra` is rescaled with the
// running sums (a block's partial mass).  Returns the frame m_use of pr[].
template <int D>
__device__ __forceinline__ float softmax_pv(Acc<D>& a, const float (&s)[16], float mx, float scl,
                                            const char* vt, float (&pr)[16], float& psum,
                                            float& extra, int rl, int hl) {
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * scl;
  const float m_new = fmaxf(a.m, mx);
  const bool move = (a.m == neg_inf()) || (m_new > a.m + kRescaleSlack);
  if (__builtin_amdgcn_ballot_w64(move)) {
    const float m_tgt = move ? m_new : a.m;
    const float alpha = (m_tgt == neg_inf()) ? 1.f : fast_exp2(a.m - m_tgt);
    a.l *= alpha;
    extra *= alpha;
#pragma unroll
    for (int mt = 0; mt < Geo<D>::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) a.o[mt][i] *= alpha;
    a.m = m_tgt;
  }
  const float m_use = (a.m == neg_inf()) ? 0.f : a.m;
  psum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pr[i] = fast_exp2(fmaf(s[i], scl, -m_use));
    psum += pr[i];
  }
  a.l += psum;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = static_cast<bf16>(pr[8 * kk + j]);
    const int qd = 2 * kk + hl;
#pragma unroll
    for (int mt = 0; mt < Geo<D>::MT; ++mt) {
      const int d = 32 * mt + rl;
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(vt + vrow(d) * 64 + 16 * (qd ^ vq_swz(d)));
      a.o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, a.o[mt], 0, 0, 0);
    }
  }
  return m_use;
}

// S^T = K Q^T of the tile in LDS at gt.
template <int D>
__device__ __forceinline__ f32x16 qk_tile(const char* gt, const bf16x8 (&q)[Geo<D>::KS], int rl,
                                          int hl) {
  f32x16 sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < Geo<D>::KS; ++ks) {
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(gt + rl * Geo<D>::K_STRIDE + 32 * ks + 16 * hl);
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, q[ks], sacc, 0, 0, 0);
  }
  return sacc;
}

// S^T = K Q^T with the Q rows read from LDS (row stride K_STRIDE, as the
// K rows); rows >= nrows are zero.
template <int D>
__device__ __forceinline__ f32x16 qk_tile_lds(const char* gt, const char* qt, int nrows, int rl,
                                              int hl) {
  f32x16 sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < Geo<D>::KS; ++ks) {
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(gt + rl * Geo<D>::K_STRIDE + 32 * ks + 16 * hl);
    const bf16x8 z = {};
    const bf16x8 qb =
        rl < nrows ? *reinterpret_cast<const bf16x8*>(qt + rl * Geo<D>::K_STRIDE + 32 * ks + 16 * hl) : z;
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb, sacc, 0, 0, 0);
  }
  return sacc;
}

// Normalised O (bf16) and LSE (natural log) of row `orow`; bad poisons.
template <int D>
__device__ __forceinline__ float write_row(const Acc<D>& a, bf16* o, float* lse, long long orow,
                                           bool bad, int hl) {
  const bool empty = !(a.l > 0.f);
  const float inv = empty ? 0.f : 1.f / a.l;
  const float lse2 = bad ? qnan() : (empty ? neg_inf() : a.m + fast_log2(a.l));
  const float poison = bad ? qnan() : 1.f;
#pragma unroll
  for (int mt = 0; mt < Geo<D>::MT; ++mt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = from_f32<bf16>(a.o[mt][4 * q4 + e] * inv * poison);
      *reinterpret_cast<bf16x4*>(o + orow * D + 32 * mt + 8 * q4 + 4 * hl) = v4;
    }
  if (hl == 0) lse[orow] = lse2 * kLn2;
  return lse2;
}

}  // namespace sss
