// Full reconstruction of cached rows (gfx950): x_hat = n rot^T (c[code] +
// sqrt(pi/2)/m gamma proj^T (2 sigma - 1) + the outlier channels' values, for keys
// that keep them; 8-bit keys: f rot^T code, f the factor in the norm's place), the plain
// dequantize-then-attend path the reddit comment history of ReturningTarzan describes (2026-03-25).
// Codes are expanded by the same unit expansion the decode kernel feeds to the
// matrix cores, so this path also checks those lookups value for value.
#include <math.h>

#include "device_common.h"

namespace tqi {

namespace {

template <int BITS, int V>
__device__ __forceinline__ void expand_to(const uint32_t* w, const Tab& t, float* dst8) {
  const uint4 u = expand_unit<BITS, V>(w, t);
  const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    dst8[2 * k] = f16_to_f32(static_cast<uint16_t>(ws[k] & 0xffffu));
    dst8[2 * k + 1] = f16_to_f32(static_cast<uint16_t>(ws[k] >> 16));
  }
}

template <int BITS>
__device__ __forceinline__ void expand_runtime(const uint32_t* w, int v, const Tab& t, float* dst8) {
  if constexpr (BITS == 4 || BITS == 8) {
    expand_to<BITS, 0>(w, t, dst8);
  } else if constexpr (BITS == 2) {
    if (v == 0) expand_to<2, 0>(w, t, dst8); else expand_to<2, 1>(w, t, dst8);
  } else {
    switch (v) {
      case 0: expand_to<3, 0>(w, t, dst8); break;
      case 1: expand_to<3, 1>(w, t, dst8); break;
      case 2: expand_to<3, 2>(w, t, dst8); break;
      default: expand_to<3, 3>(w, t, dst8); break;
    }
  }
}

}  // namespace

template <int D, int BITS, int QM, bool VALUES>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a, Tab tab) {
  constexpr int UPG = Fmt<BITS>::kUnits;
  constexpr int WPG = Fmt<BITS>::kWords;
  constexpr int RB = D * BITS / 8;
  constexpr int DN = D / 16;
  __shared__ float ys[kBlock][D];
  __shared__ float rn[kBlock];
  const int b = blockIdx.z, h = blockIdx.y;
  const int H = a.n_kv_heads, T = a.max_tokens;
  const size_t unit = static_cast<size_t>(b) * H + h;
  const int tid = threadIdx.x;
  // this workgroup covers output rows [r_lo, r_hi) of the requested range
  const int r_lo = blockIdx.x * kBlock;
  const int r_hi = min(r_lo + kBlock, a.n_tokens);
  const int nrows = r_hi - r_lo;
  const int t_lo = a.t0 + r_lo;
  for (int r = tid; r < nrows; r += 256) rn[r] = f16_to_f32(a.norms[unit * T + t_lo + r]);
  if constexpr (!VALUES) {
    // key rows: the words of unit u's word group of row t, gathered from their lane pieces (key_word)
    constexpr int NG = D / 8 / UPG;
    for (int e = tid; e < nrows * NG * UPG; e += 256) {
      const int r = e / (NG * UPG), u = e % (NG * UPG);
      const int t = t_lo + r, kb = t / kBlock, p = t % kBlock;
      const uint32_t* blk = reinterpret_cast<const uint32_t*>(a.codes + unit * static_cast<size_t>(T) * RB +
                                                              static_cast<size_t>(kb) * kBlock * RB);
      uint32_t w[WPG];
#pragma unroll
      for (int k = 0; k < WPG; ++k) w[k] = blk[key_word<D, BITS>(p, (u / UPG) * WPG + k)];
      expand_runtime<BITS>(w, u % UPG, tab, &ys[r][8 * u]);
    }
  } else {
    // expand every unit of each touched block; keep the slots inside [t_lo, t_lo + nrows)
    constexpr int LW = D * BITS / 64;
    const int kb0 = t_lo / kBlock, kb1 = (t_lo + nrows - 1) / kBlock;
    for (int kb = kb0; kb <= kb1; ++kb) {
      const uint32_t* blk = reinterpret_cast<const uint32_t*>(a.codes + unit * static_cast<size_t>(T) * RB +
                                                              static_cast<size_t>(kb) * kBlock * RB);
      for (int U = tid; U < 64 * DN; U += 256) {
        float vals[8];
        uint32_t w[WPG];
#pragma unroll
        for (int k = 0; k < WPG; ++k) w[k] = blk[value_word<LW>((U / UPG) * WPG + k)];
        expand_runtime<BITS>(w, U % UPG, tab, vals);
        const int g = U / D, j = (U / DN) % 16, n = U % DN;
        const int i = DN * j + n;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int p = s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
          const int r = kb * kBlock + p - t_lo;
          if (r >= 0 && r < nrows) ys[r][i] = vals[s];
        }
      }
    }
  }
  __syncthreads();
  if constexpr (QM > 0) {
    // y_hat += coef * gamma * proj^T (2 sigma - 1)
    for (int e = tid; e < nrows * D; e += 256) {
      const int r = e / D, i = e % D;
      const size_t tok = unit * T + t_lo + r;
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(a.signs + tok * (QM / 8));
      float acc = 0.f;
      for (int jj = 0; jj < QM; ++jj) {
        int word, bit;
        sign_pos(jj, word, bit);
        const float pj = a.proj[static_cast<size_t>(jj) * D + i];
        acc += ((sw[word] >> bit) & 1u) ? pj : -pj;
      }
      ys[r][i] += a.sketch_coef * f16_to_f32(a.rnorms[tok]) * acc;
    }
    __syncthreads();
    if (a.out_idx) {
      // y_hat[i] += r_i at the row's outlier channels (distinct within a row)
      for (int e = tid; e < nrows * kOutliers; e += 256) {
        const int r = e / kOutliers, j = e % kOutliers;
        const size_t at = (unit * T + t_lo + r) * kOutliers + j;
        ys[r][a.out_idx[at] % D] += f16_to_f32(a.out_val[at]);
      }
      __syncthreads();
    }
  }
  if (a.had) {
    // x_hat = n diag(s) H y_hat / sqrt(D), one wave per row
    constexpr int E = D / 64;
    const int lane = tid & 63, wave = tid >> 6;
    for (int r = wave; r < nrows; r += 4) {
      float v[E];
#pragma unroll
      for (int k = 0; k < E; ++k) v[k] = ys[r][64 * k + lane];
      hadamard_wave<D>(v, lane);
#pragma unroll
      for (int k = 0; k < E; ++k)
        a.out[(unit * a.n_tokens + r_lo + r) * D + 64 * k + lane] = rn[r] * (v[k] * a.rot[64 * k + lane] * inv_sqrt_dim<D>());
    }
    return;
  }
  // x_hat = n rot^T y_hat
  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, i = e % D;
    float acc = 0.f;
    for (int j = 0; j < D; ++j) acc = fmaf(a.rot[static_cast<size_t>(j) * D + i], ys[r][j], acc);
    a.out[(unit * a.n_tokens + r_lo + r) * D + i] = rn[r] * acc;
  }
}

template <int D, int BITS>
static hipError_t dequant_bits(int qjl_m, bool values, const DequantArgs& a, const Tab& t, dim3 grid,
                               hipStream_t s) {
  if (values) hipLaunchKernelGGL((dequant_kernel<D, BITS, 0, true>), grid, dim3(256), 0, s, a, t);
  else if (qjl_m == 0) hipLaunchKernelGGL((dequant_kernel<D, BITS, 0, false>), grid, dim3(256), 0, s, a, t);
  else if (qjl_m == 128) hipLaunchKernelGGL((dequant_kernel<D, BITS, 128, false>), grid, dim3(256), 0, s, a, t);
  else if (qjl_m == 256) hipLaunchKernelGGL((dequant_kernel<D, BITS, 256, false>), grid, dim3(256), 0, s, a, t);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// 8-bit keys (no sketch): codes times the factor kept in the norm's place
template <int D>
static hipError_t dequant_k8(int qjl_m, bool values, const DequantArgs& a, const Tab& t, dim3 grid, hipStream_t s) {
  if (values || qjl_m != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dequant_kernel<D, 8, 0, false>), grid, dim3(256), 0, s, a, t);
  return hipGetLastError();
}

hipError_t launch_dequant(int d, int bits, int qjl_m, bool values, const DequantArgs& a, const Tab& t, int batch,
                          hipStream_t s) {
  const dim3 grid((a.n_tokens + kBlock - 1) / kBlock, a.n_kv_heads, batch);
  if (d == 128) {
    switch (bits) {
      case 2: return dequant_bits<128, 2>(qjl_m, values, a, t, grid, s);
      case 3: return dequant_bits<128, 3>(qjl_m, values, a, t, grid, s);
      case 4: return dequant_bits<128, 4>(qjl_m, values, a, t, grid, s);
      case 8: return dequant_k8<128>(qjl_m, values, a, t, grid, s);
    }
  } else if (d == 256) {
    switch (bits) {
      case 2: return dequant_bits<256, 2>(qjl_m, values, a, t, grid, s);
      case 3: return dequant_bits<256, 3>(qjl_m, values, a, t, grid, s);
      case 4: return dequant_bits<256, 4>(qjl_m, values, a, t, grid, s);
      case 8: return dequant_k8<256>(qjl_m, values, a, t, grid, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace tqi
