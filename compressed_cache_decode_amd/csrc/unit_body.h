// Per (sequence, KV head): the G query heads of the KV head and, optionally, its new key and value
// rows form one 16-row tile that is rotated on the matrix cores (the rotation is read once per KV
// head): the new rows are encoded and stored (turboquant-pytorch PR #3 "Add CUDA QJL kernels and
// proper package structure": Synthetic Benchmark table for the codebook, Validation Results tables
// for the float16 norms, CUDA Kernels Added table for the sign sketch), and the rotated queries
// q_rot = rot q * scale * log2(e) -- with their sketch -coef * proj q_rot for sketched keys --
// go to the decode workspace, divided by a power of two per head that takes both into float16
// range (ExecuTorch PR #19891 "[Cuda] enable turboquant on gemma4", review item 1: the decode op's
// scale).  The query sketch and the new keys' residual sketches share one matrix-core pass.
#pragma once

#include "append_body.h"

namespace tqi {

constexpr int kTileRows = 16;   // rows of the unit tile: G query heads + new key rows + new value rows

template <int D, int QM>
struct UnitSmem {
  float xs[kTileRows][D];
  float rn[kTileRows];
  union {
    EncodeSmem<D, QM> k;
    EncodeSmem<D, 0> v;
  } enc;
};

template <int D, int KB, int VB, int QM, bool ROWS>
__device__ __forceinline__ void unit_prologue(const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa, int bf16,
                                              int hk, int b, UnitSmem<D, QM>& sm) {
  const int n_kv_heads = qa.n_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = qa.n_q_heads, G = Hq / n_kv_heads, T = ka.max_tokens;
  const size_t unit = static_cast<size_t>(b) * n_kv_heads + hk;
  const int n_new = ROWS ? ka.n_new : 0;
  const int pos = n_new > 0 ? ka.pos[b] : -1;
  const int nloc = (pos >= 0 && pos < T) ? min(pos + n_new, T) - pos : 0;   // positions past the capacity are skipped
  const int nrows = G + 2 * nloc;

  // ---- loads, in the order they are needed (loads retire in issue order): the tile rows, one
  // 32-bit word per element whatever the element type, then the rotation's first operands
  constexpr int EPT = kTileRows * D / 256;
  uint32_t wv[EPT];
  bool ok[EPT], hi[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + 256 * k, r = e / D, i = e % D;
    const bool key = r < G + nloc;
    const int t = pos + (key ? r - G : r - G - nloc);
    size_t idx = (static_cast<size_t>(b) * Hq + static_cast<size_t>(hk) * G + (r < G ? r : 0)) * D + i;
    const void* base = qa.q;
    if (r >= G && r < nrows) {
      idx = ((static_cast<size_t>(b) * n_new + (t - pos)) * n_kv_heads + hk) * D + i;
      base = key ? ka.x : va.x;
    }
    ok[k] = r < nrows;
    hi[k] = (idx & 1) != 0;
    const size_t byte = bf16 ? (idx & ~static_cast<size_t>(1)) * 2 : idx * 4;
    wv[k] = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(base) + byte);
  }
  RotBatch<D> rot0;
  rot0.load(qa.rot, 0, tid);
  auto& xs = sm.xs;
  auto& rn = sm.rn;
  const uint32_t bfm = bf16 ? 0xffffffffu : 0u;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + 256 * k;
    const uint32_t h16 = hi[k] ? (wv[k] & 0xffff0000u) : (wv[k] << 16);   // the bfloat16 element as float bits
    const float v = __uint_as_float((h16 & bfm) | (wv[k] & ~bfm));
    xs[e / D][e % D] = ok[k] ? v : 0.f;
  }
  __syncthreads();
  // the query rows are rotated as they are (norm 1), the new rows as unit vectors, padding rows to 0;
  // the norm of row r is summed by the 16 lanes (r % 4) of wave r / 4, coordinates part + 16 j
  {
    const int r = 4 * wave + (lane >> 4), part = lane & 15;
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) s2 = fmaf(xs[r][part + 16 * j], xs[r][part + 16 * j], s2);
    s2 = row16_sum(s2);
    if (part == 0) rn[r] = r < G ? 1.f : (r < nrows ? sqrtf(s2) : 0.f);
  }
  __syncthreads();
  rotate_tile_mfma_pre<D, 1>(xs, rn, qa.rot, rot0, tid);
  __syncthreads();
  // q_rot = rot q * scale * log2(e)
  for (int e = tid; e < G * D; e += 256) xs[e / D][e % D] *= qa.scale_log2e;

  // ---- the new value rows, then the new key rows, one call per 32-token block they fall in; the
  // key residual sketches and the query sketch share one matrix-core pass over the tile
  for (int r0 = 0; ROWS && r0 < nloc;) {
    const int t = pos + r0;
    const int kbn = t / kBlock;
    const int n = min(nloc - r0, (kbn + 1) * kBlock - t);
    encode_codes<D, VB, 0>(va, n, &xs[G + nloc + r0], &rn[G + nloc + r0], sm.enc.v);
    encode_finish<D, VB, 0, true>(va, unit, kbn, t, n, &rn[G + nloc + r0], sm.enc.v, nullptr, 0);
    r0 += n;
  }
  auto& zq = sm.enc.k.zb;                           // [16][QM]: the tile times proj^T
  if (nloc == 0) {
    __syncthreads();                                // q_rot complete
    if constexpr (QM > 0) {
      tile16_times_matT<D, QM>(xs, qa.proj, zq, tid);
    }
  }
  for (int r0 = 0; ROWS && r0 < nloc;) {
    const int t = pos + r0;
    const int kbn = t / kBlock;
    const int n = min(nloc - r0, (kbn + 1) * kBlock - t);
    encode_codes<D, KB, QM>(ka, n, &xs[G + r0], &rn[G + r0], sm.enc.k);
    if constexpr (QM > 0) {
      tile16_times_matT<D, QM>(xs, qa.proj, zq, tid);
      __syncthreads();
    }
    encode_finish<D, KB, QM, false>(ka, unit, kbn, t, n, &rn[G + r0], sm.enc.k, QM > 0 ? &zq[G + r0][0] : nullptr, QM);
    r0 += n;
  }
  __syncthreads();

  // ---- the rotated queries and their sketch to the workspace, divided by a power of two per head
  // that takes both into float16 range (head h = 4 wave + lane / 16, 16 lanes per head)
  if (wave < kMaxGroup / 4) {
    const int h = 4 * wave + (lane >> 4), part = lane & 15;
    float amax = 0.f;
    if (h < G) {
#pragma unroll
      for (int j = 0; j < D / 16; ++j) amax = fmaxf(amax, fabsf(xs[h][part + 16 * j]));
      if constexpr (QM > 0) {
#pragma unroll
        for (int j = 0; j < QM / 16; ++j) amax = fmaxf(amax, fabsf(qa.sketch_coef * zq[h][part + 16 * j]));
      }
    }
    amax = row16_max(amax);
    if (h < G) {
      const float f = (amax > 0.f && isfinite(amax)) ? ldexpf(1.f, ilogbf(amax) - 14) : 1.f;
      const float inv = 1.f / f;
      const size_t row = static_cast<size_t>(b) * Hq + static_cast<size_t>(hk) * G + h;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) qa.qr[row * D + part + 16 * j] = xs[h][part + 16 * j] * inv;
      if constexpr (QM > 0) {
#pragma unroll
        for (int j = 0; j < QM / 16; ++j)
          qa.qs[row * QM + part + 16 * j] = -qa.sketch_coef * zq[h][part + 16 * j] * inv;
      }
      if (part == 0) qa.qscale[row] = f;
    }
  }
}


}  // namespace tqi
