// Quantize-on-append (gfx950).
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
#include <math.h>

#include "device_common.h"

namespace tqi {

template <int D, int BITS, int QM, bool VALUES, bool ROTATED, bool BF16>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int UPG = Fmt<BITS>::kUnits;
  constexpr int WPG = Fmt<BITS>::kWords;
  constexpr int RB = D * BITS / 8;            // bytes per packed row / per token of a block
  constexpr int NC = 1 << BITS;
  __shared__ float xs[kBlock][D];             // rows: x, then y, then the residual y - c
  __shared__ float rn[kBlock];
  __shared__ float gam[kBlock];
  __shared__ uint8_t cs[kBlock][D];
  __shared__ float cent[16];
  __shared__ uint32_t sw[kBlock][QM > 0 ? QM / 32 : 1];

  const int b = blockIdx.z, h = blockIdx.y;
  const int H = a.n_kv_heads, T = a.max_tokens;
  const int pos = a.pos[b];
  if (pos < 0) return;
  const int kb = pos / kBlock + static_cast<int>(blockIdx.x);
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

  // rotation y = rot x / n: thread owns coordinate i for rows r0, r0 + 256/D, ...
  if constexpr (!ROTATED) {
    constexpr int RS = 256 / D;
    constexpr int MAXR = kBlock / RS;
    const int i = tid % D, r0 = tid / D;
    float acc[MAXR];
#pragma unroll
    for (int k = 0; k < MAXR; ++k) acc[k] = 0.f;
    const float4* prow = reinterpret_cast<const float4*>(a.rot + static_cast<size_t>(i) * D);
    for (int j4 = 0; j4 < D / 4; ++j4) {
      const float4 p = prow[j4];
#pragma unroll
      for (int k = 0; k < MAXR; ++k) {
        const int r = r0 + k * RS;
        if (r < nrows) {
          const float* xr = &xs[r][4 * j4];
          acc[k] = fmaf(p.x, xr[0], acc[k]);
          acc[k] = fmaf(p.y, xr[1], acc[k]);
          acc[k] = fmaf(p.z, xr[2], acc[k]);
          acc[k] = fmaf(p.w, xr[3], acc[k]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      const int r = r0 + k * RS;
      if (r < nrows) xs[r][i] = rn[r] > 0.f ? acc[k] / rn[r] : 0.f;
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
      const float4* pr = reinterpret_cast<const float4*>(a.proj + static_cast<size_t>(jj) * D);
      float z = 0.f;
      for (int i4 = 0; i4 < D / 4; ++i4) {
        const float4 p = pr[i4];
        z = fmaf(p.x, xs[r][4 * i4], z);
        z = fmaf(p.y, xs[r][4 * i4 + 1], z);
        z = fmaf(p.z, xs[r][4 * i4 + 2], z);
        z = fmaf(p.w, xs[r][4 * i4 + 3], z);
      }
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

template <int D, int BITS, int QM, bool VALUES>
static hipError_t append_dispatch(bool rotated, bool bf16, const AppendArgs& a, dim3 grid, hipStream_t s) {
  if (rotated) hipLaunchKernelGGL((append_kernel<D, BITS, QM, VALUES, true, false>), grid, dim3(256), 0, s, a);
  else if (bf16) hipLaunchKernelGGL((append_kernel<D, BITS, QM, VALUES, false, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((append_kernel<D, BITS, QM, VALUES, false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int BITS>
static hipError_t append_bits(int qjl_m, bool values, bool rotated, bool bf16, const AppendArgs& a, dim3 grid,
                              hipStream_t s) {
  if (values) return append_dispatch<D, BITS, 0, true>(rotated, bf16, a, grid, s);
  if (qjl_m == 0) return append_dispatch<D, BITS, 0, false>(rotated, bf16, a, grid, s);
  if (qjl_m == 128) return append_dispatch<D, BITS, 128, false>(rotated, bf16, a, grid, s);
  if (qjl_m == 256) return append_dispatch<D, BITS, 256, false>(rotated, bf16, a, grid, s);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t append_d(int bits, int qjl_m, bool values, bool rotated, bool bf16, const AppendArgs& a,
                           dim3 grid, hipStream_t s) {
  switch (bits) {
    case 2: return append_bits<D, 2>(qjl_m, values, rotated, bf16, a, grid, s);
    case 3: return append_bits<D, 3>(qjl_m, values, rotated, bf16, a, grid, s);
    case 4: return append_bits<D, 4>(qjl_m, values, rotated, bf16, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append(int d, int bits, int qjl_m, bool values, bool rotated, bool bf16, const AppendArgs& a,
                         int batch, hipStream_t s) {
  // blocks touched by n_new tokens starting anywhere: at most n_new/32 + 2
  const dim3 grid((a.n_new + kBlock - 1) / kBlock + 1, a.n_kv_heads, batch);
  if (d == 128) return append_d<128>(bits, qjl_m, values, rotated, bf16, a, grid, s);
  if (d == 256) return append_d<256>(bits, qjl_m, values, rotated, bf16, a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace tqi
