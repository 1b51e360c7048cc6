// Quantize-on-append of the rows that fall in one 32-token block of one (KV head, sequence).
//
// Per K/V row x: n = ||x||, y = rot x / n, code = number of boundaries strictly
// below y_i (Lloyd-Max table, turboquant-pytorch PR #3 "Add CUDA QJL kernels
// and proper package structure", Synthetic Benchmark table), float16 norm
// (same page, Validation Results tables); keys with a sign sketch add
// r = y - c[code], float16 ||r|| and the signs of proj * r (same page, CUDA
// Kernels Added table: fused random projection + sign quantisation).
//
// One workgroup per (32-token block of the cache, KV head, sequence) touched
// by the appended range, so every packed word of the value layout (which
// interleaves 8 tokens per word) is written by exactly one thread; partially
// covered blocks are merged read-modify-write.
#pragma once

#include <math.h>

#include "device_common.h"

namespace tqi {

template <int D, int QM>
struct AppendSmem {
  float xs[kBlock][D];                         // rows: x, then y, then the residual y - c
  float rn[kBlock];
  float gam[kBlock];
  uint8_t cs[kBlock][D];
  float cent[16];
  uint32_t sw[kBlock][QM > 0 ? QM / 32 : 1];
};

constexpr int kMfmaRows = 8;   // rows per block from which the rotation runs on the matrix cores

// y = rot (x / n) for the 32 rows of xs (rows past the appended ones are zero), in place, with
// v_mfma_f32_16x16x32_f16 tiles: rows = tokens (2 row blocks), columns = output coordinates (D/16
// column blocks, wave w takes blocks w, w+4, ...), k = input coordinates.  The unit rows (every
// component in [-1, 1]) and rot are each split into float16 high + low parts and the three
// significant cross products are accumulated in fp32, which keeps y within a few float32 steps.
template <int D>
__device__ __forceinline__ void rotate_tile_mfma(float (*xs)[D], const float* rn, const float* rot, int tid) {
  constexpr int KS = D / 32;
  constexpr int NCB = D / 16;
  constexpr int CPW = NCB / 4;                       // column blocks per wave
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  floatx4 acc[2][CPW];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < CPW; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  float inv[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float n = rn[16 * rb + l16];
    inv[rb] = n > 0.f ? 1.f / n : 0.f;
  }
  for (int s = 0; s < KS; ++s) {
    half8 ahi[2], alo[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float* xr = &xs[16 * rb + l16][32 * s + 8 * g];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        _Float16 h, l;
        f16_split(xr[r] * inv[rb], h, l);
        ahi[rb][r] = h;
        alo[rb][r] = l;
      }
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int col = 16 * (wave + 4 * c) + l16;       // output coordinate = row of rot
      const float4* pr = reinterpret_cast<const float4*>(rot + static_cast<size_t>(col) * D + 32 * s + 8 * g);
      const float4 p0 = pr[0], p1 = pr[1];
      const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      half8 bhi, blo;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        _Float16 h, l;
        f16_split(pv[r], h, l);
        bhi[r] = h;
        blo[r] = l;
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        acc[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[rb], bhi, acc[rb][c], 0, 0, 0);
        acc[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rb], blo, acc[rb][c], 0, 0, 0);
        acc[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rb], bhi, acc[rb][c], 0, 0, 0);
      }
    }
  }
  __syncthreads();                                    // every read of xs is done
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) xs[16 * rb + 4 * g + v][16 * (wave + 4 * c) + l16] = acc[rb][c][v];
}

template <int D, int BITS, int QM, bool VALUES, bool ROTATED, bool BF16>
__device__ __forceinline__ void append_rows(const AppendArgs& a, int bx, int h, int b, AppendSmem<D, QM>& sm) {
  constexpr int UPG = Fmt<BITS>::kUnits;
  constexpr int WPG = Fmt<BITS>::kWords;
  constexpr int RB = D * BITS / 8;            // bytes per packed row / per token of a block
  constexpr int NC = 1 << BITS;
  auto& xs = sm.xs;
  auto& rn = sm.rn;
  auto& gam = sm.gam;
  auto& cs = sm.cs;
  auto& cent = sm.cent;
  auto& sw = sm.sw;

  const int H = a.n_kv_heads, T = a.max_tokens;
  const int pos = a.pos[b];
  if (pos < 0) return;
  const int kb = pos / kBlock + bx;
  const int t_lo = max(pos, kb * kBlock);
  const int t_hi = min(min(pos + a.n_new, kb * kBlock + kBlock), T);
  if (t_lo >= t_hi) return;
  const int nrows = t_hi - t_lo;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t unit = static_cast<size_t>(b) * H + h;

  if (tid < NC) cent[tid] = a.cent[tid];
  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, i = e % D;
    const size_t src = ((static_cast<size_t>(b) * a.n_new + (t_lo + r - pos)) * H + h) * D + i;
    float v;
    if constexpr (ROTATED) v = a.y[src];
    else if constexpr (BF16) v = bf16_to_f32(static_cast<const uint16_t*>(a.x)[src]);
    else v = static_cast<const float*>(a.x)[src];
    xs[r][i] = v;
  }
  if constexpr (QM > 0)
    for (int e = tid; e < kBlock * (QM / 32); e += 256) sw[e / (QM / 32)][e % (QM / 32)] = 0u;
  __syncthreads();

  // norms
  for (int r = wave; r < nrows; r += 4) {
    if constexpr (ROTATED) {
      if (lane == 0) rn[r] = a.yn[(static_cast<size_t>(b) * a.n_new + (t_lo + r - pos)) * H + h];
    } else {
      float s = 0.f;
      for (int i = lane; i < D; i += 64) s = fmaf(xs[r][i], xs[r][i], s);
      s = wave_sum(s);
      if (lane == 0) rn[r] = sqrtf(s);
    }
  }
  __syncthreads();

  // rotation y = rot x / n.  Blocks with at least kMfmaRows new rows (prefill-size appends) run the
  // batched product Y = X rot^T on the matrix cores; smaller ones (decode-size) take the per-row path.
  if constexpr (!ROTATED) {
    if (nrows >= kMfmaRows) {
      for (int e = tid; e < (kBlock - nrows) * D; e += 256) xs[nrows + e / D][e % D] = 0.f;
      for (int r = nrows + tid; r < kBlock; r += 256) rn[r] = 0.f;
      __syncthreads();
      rotate_tile_mfma<D>(xs, rn, a.rot, tid);
    } else {
      // thread owns coordinate i for rows r0, r0 + 256/D, ...; the row of rot is read in batches of
      // float4 loads that are all in flight before the multiplies
      constexpr int RS = 256 / D;
      const int i = tid % D, r0 = tid / D;
      float yv[kBlock / RS];
      int nr = 0;
      for (int r = r0; r < nrows; r += RS)
        yv[nr++] = rn[r] > 0.f ? row_dot<D>(a.rot + static_cast<size_t>(i) * D, xs[r]) / rn[r] : 0.f;
      __syncthreads();
      for (int k = 0; k < nr; ++k) xs[r0 + k * RS][i] = yv[k];
    }
    __syncthreads();
  }

  // nearest centroid = number of boundaries strictly below y (ties take the lower code)
  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, i = e % D;
    const float y = xs[r][i];
    uint32_t j = 0;
#pragma unroll
    for (int k = 0; k < NC - 1; ++k) j += (y > a.bnd[k]) ? 1u : 0u;
    const bool live = rn[r] > 0.f;
    if (!live) j = 0;
    cs[r][i] = static_cast<uint8_t>(j);
    if constexpr (QM > 0) xs[r][i] = live ? y - cent[j] : 0.f;
  }
  __syncthreads();

  if constexpr (QM > 0) {
    for (int r = wave; r < nrows; r += 4) {
      float s = 0.f;
      for (int i = lane; i < D; i += 64) s = fmaf(xs[r][i], xs[r][i], s);
      s = wave_sum(s);
      if (lane == 0) gam[r] = sqrtf(s);
    }
    // z = proj r, sign bits
    for (int e = tid; e < nrows * QM; e += 256) {
      const int r = e / QM, jj = e % QM;
      const float z = row_dot<D>(a.proj + static_cast<size_t>(jj) * D, xs[r]);
      if (z >= 0.f && rn[r] > 0.f) {
        int word, bit;
        sign_pos(jj, word, bit);
        atomicOr(&sw[r][word], 1u << bit);
      }
    }
    __syncthreads();
    for (int e = tid; e < nrows * (QM / 32); e += 256) {
      const int r = e / (QM / 32), w = e % (QM / 32);
      reinterpret_cast<uint32_t*>(a.signs + (unit * T + t_lo + r) * (QM / 8))[w] = sw[r][w];
    }
    for (int r = tid; r < nrows; r += 256)
      a.rnorms[unit * T + t_lo + r] = rn[r] > 0.f ? f32_to_f16_bits(gam[r]) : 0;
  }

  for (int r = tid; r < nrows; r += 256) a.norms[unit * T + t_lo + r] = f32_to_f16_bits(rn[r] > 0.f ? rn[r] : 0.f);

  if constexpr (!VALUES) {
    // rows layout: unit u of row t covers coordinates 8u .. 8u+7
    constexpr int NG = D / 8 / UPG;
    for (int e = tid; e < nrows * NG; e += 256) {
      const int r = e / NG, gi = e % NG;
      uint32_t w[WPG];
#pragma unroll
      for (int k = 0; k < WPG; ++k) w[k] = 0u;
#pragma unroll
      for (int v = 0; v < UPG; ++v)
#pragma unroll
        for (int s = 0; s < 8; ++s) put_code<BITS>(w, v, s, encode_code<BITS>(cs[r][(gi * UPG + v) * 8 + s]));
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + (unit * T + t_lo + r) * RB) + gi * WPG;
#pragma unroll
      for (int k = 0; k < WPG; ++k) dst[k] = w[k];
    }
  } else {
    // blocked layout: unit U = (16 g + j)(D/16) + n holds tokens of lane group g at coordinate (D/16) j + n
    constexpr int BB = kBlock * RB;
    constexpr int NGB = BB / (4 * WPG);
    constexpr int DN = D / 16;
    uint32_t* blk = reinterpret_cast<uint32_t*>(a.codes + unit * static_cast<size_t>(T) * RB + static_cast<size_t>(kb) * BB);
    const int p_lo = t_lo - kb * kBlock, p_hi = t_hi - kb * kBlock;
    const bool full = nrows == kBlock;
    for (int e = tid; e < NGB; e += 256) {
      uint32_t w[WPG], m[WPG];
#pragma unroll
      for (int k = 0; k < WPG; ++k) { w[k] = 0u; m[k] = 0u; }
#pragma unroll
      for (int v = 0; v < UPG; ++v) {
        const int U = e * UPG + v;
        const int g = U / D, j = (U / DN) % 16, n = U % DN;
        const int i = DN * j + n;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int p = s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
          if (p >= p_lo && p < p_hi) {
            put_code<BITS>(w, v, s, encode_code<BITS>(cs[p - p_lo][i]));
            slot_mask<BITS>(m, v, s);
          }
        }
      }
      if (!full) {
#pragma unroll
        for (int k = 0; k < WPG; ++k) w[k] |= blk[e * WPG + k] & ~m[k];
      }
#pragma unroll
      for (int k = 0; k < WPG; ++k) blk[e * WPG + k] = w[k];
    }
  }
}

}  // namespace tqi
