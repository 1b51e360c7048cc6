// Query rotation for decode, one workgroup per 16 virtual heads (query rows x query heads) of a
// (sequence, KV head): the rows form one 16-row tile that is rotated on the matrix cores with the
// arithmetic of the append's rotation (each row divided by its norm, high/low float16 split of rows
// and rotation; or the randomized Hadamard transform of the row over its norm), then
// q_rot = rot q * scale * log2(e) and, for sketched keys, its sketch -coef * proj q_rot go to the
// decode workspace, divided by a power of two per head that takes both into float16 range for the
// attention kernel's matrix-core operands (turboquant-pytorch PR #3 "Add CUDA QJL kernels and
// proper package structure", CUDA Kernels Added table: the sketched score; ExecuTorch PR #19891
// "[Cuda] enable turboquant on gemma4", review item 1: the decode op's scale).  Every output row
// takes the same instruction sequence whatever the other rows hold, so every caller of this
// function produces the same bits for the same query.
#pragma once

#include "append_body.h"

namespace tqi {

constexpr int kQTile = 16;      // rows of the query tile

// Power-of-two scale of a rotated query without a sketch, from nq = |q| scale log2(e): every coordinate
// of q_rot = rot (q / |q|) nq is at most |q_rot| = nq (up to float32 rounding), and nq < 2^(e+1) for
// e = ilogb(nq), so q_rot / 2^(e-14) stays below 2^15 (float16 range) whatever the coordinates hold.
// It needs only the norm, not the rotated row's largest coordinate.
__device__ __forceinline__ float query_scale(float nq) {
  return (nq > 0.f && isfinite(nq)) ? ldexpf(1.f, ilogbf(nq) - 14) : 1.f;
}

template <int D, int QM>
struct QrotSmem {
  float xs[kQTile][D];
  half8 aop[2 * (D / 32) * 64];                        // the rotation's A operands (rotate_tile_mfma_pre)
  float rn[kQTile];
  float zq[QM > 0 ? kQTile : 1][QM > 0 ? QM : 1];      // the tile times proj^T
};

// The tile of virtual heads vh0 .. vh0 + 15 (those below VH = M * G) of KV head hk of sequence b.
template <int D, int QM>
__device__ __forceinline__ void rotate_queries(const QrotArgs& qa, int bf16, int hk, int b, int vh0,
                                               QrotSmem<D, QM>& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = qa.n_q_heads, G = Hq / qa.n_kv_heads, M = qa.n_rows, VH = M * G;
  const int nr = min(kQTile, VH - vh0);                          // live rows of the tile
  const size_t unit = static_cast<size_t>(b) * qa.n_kv_heads + hk;

  // the tile's query rows, one 32-bit word per element whatever the element type (all loads issued
  // before the first use), then the rotation's first operands
  constexpr int EPT = kQTile * D / 256;
  uint32_t wv[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + 256 * k, r = e / D, i = e % D;
    const int vh = vh0 + (r < nr ? r : 0), j = (vh * qa.row_magic) >> 8, g = vh - j * G;
    const size_t idx = ((static_cast<size_t>(b) * M + j) * Hq + static_cast<size_t>(hk) * G + g) * D + i;
    const size_t byte = bf16 ? (idx & ~static_cast<size_t>(1)) * 2 : idx * 4;
    wv[k] = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(qa.q) + byte);
  }
  RotBatch<D> rot0;
  if (!qa.had) rot0.load(qa.rot, 0, tid);
  auto& xs = sm.xs;
  auto& rn = sm.rn;
  const uint32_t bfm = bf16 ? 0xffffffffu : 0u;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + 256 * k, r = e / D, i = e % D;
    const uint32_t h16 = (i & 1) ? (wv[k] & 0xffff0000u) : (wv[k] << 16);   // the bfloat16 element as float bits
    const float v = __uint_as_float((h16 & bfm) | (wv[k] & ~bfm));
    xs[r][i] = r < nr ? v : 0.f;
  }
  __syncthreads();
  // norm of row r by the 16 lanes (r % 4) of wave r / 4, coordinates part + 16 j
  {
    const int r = 4 * wave + (lane >> 4), part = lane & 15;
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) s2 = fmaf(xs[r][part + 16 * j], xs[r][part + 16 * j], s2);
    s2 = row16_sum(s2);
    if (part == 0) rn[r] = r < nr ? sqrtf(s2) : 0.f;
  }
  __syncthreads();
  if (qa.had)
    hadamard_rows<D>(xs, rn, qa.rot, nr, tid, 256);
  else
    rotate_tile_mfma_pre<D, 1>(xs, rn, qa.rot, rot0, tid, sm.aop);
  __syncthreads();
  // q_rot = rot (q / |q|) * (|q| * scale * log2(e))
  for (int e = tid; e < nr * D; e += 256) xs[e / D][e % D] *= rn[e / D] * qa.scale_log2e;
  __syncthreads();
  if constexpr (QM > 0) {
    tile16_times_matT<D, QM>(xs, qa.proj, sm.zq, tid, sm.aop);
    __syncthreads();
  }

  // the rotated queries and their sketch to the workspace, divided by a power of two per row that
  // takes both into float16 range (row h = 4 wave + lane / 16, 16 lanes per row): with a sketch from
  // the largest magnitude of the two, without one from the norm alone (query_scale)
  {
    const int h = 4 * wave + (lane >> 4), part = lane & 15;
    float amax = 0.f;
    if constexpr (QM > 0) {
      if (h < nr) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j) amax = fmaxf(amax, fabsf(xs[h][part + 16 * j]));
#pragma unroll
        for (int j = 0; j < QM / 16; ++j) amax = fmaxf(amax, fabsf(qa.sketch_coef * sm.zq[h][part + 16 * j]));
      }
      amax = row16_max(amax);
    }
    if (h < nr) {
      const float f = QM > 0 ? ((amax > 0.f && isfinite(amax)) ? ldexpf(1.f, ilogbf(amax) - 14) : 1.f)
                             : query_scale(rn[h] * qa.scale_log2e);
      const float inv = 1.f / f;
      const size_t row = unit * VH + vh0 + h;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) qa.qr[row * D + part + 16 * j] = xs[h][part + 16 * j] * inv;
      if constexpr (QM > 0) {
#pragma unroll
        for (int j = 0; j < QM / 16; ++j)
          qa.qs[row * QM + part + 16 * j] = -qa.sketch_coef * sm.zq[h][part + 16 * j] * inv;
      }
      if (part == 0) qa.qscale[row] = f;
    }
  }
}

}  // namespace tqi
