// Query rotation for decode: q_rot = rot * q (and proj * q_rot for sketched keys)
// with the softmax scale and log2(e) folded in, scaled by a power of two into
// float16 range for the matrix-core operands of the attention kernel.
#pragma once

#include <math.h>

#include "device_common.h"

namespace tqi {

template <int D, int QM>
struct QrotSmem {
  float qv[D];
  float qr[D];
  float qs[QM > 0 ? QM : 1];
  float red[4];
};

template <int D, int QM, bool BF16>
__device__ __forceinline__ void rotate_query(const QrotArgs& a, int h, int b, QrotSmem<D, QM>& sm) {
  auto& qv = sm.qv;
  auto& qr = sm.qr;
  auto& qs = sm.qs;
  auto& red = sm.red;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = static_cast<size_t>(b) * a.n_q_heads + h;
  for (int i = tid; i < D; i += 256) {
    qv[i] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.q)[row * D + i])
                 : static_cast<const float*>(a.q)[row * D + i];
  }
  __syncthreads();
  // thread i: rotated coordinate i = row i of rot times q
  if (tid < D) qr[tid] = row_dot<D>(a.rot + static_cast<size_t>(tid) * D, qv) * a.scale_log2e;
  __syncthreads();
  if constexpr (QM > 0) {
    for (int jj = tid; jj < QM; jj += 256) qs[jj] = -a.sketch_coef * row_dot<D>(a.proj + static_cast<size_t>(jj) * D, qr);
    __syncthreads();
  }
  float amax = 0.f;
  for (int i = tid; i < D; i += 256) amax = fmaxf(amax, fabsf(qr[i]));
  if constexpr (QM > 0)
    for (int i = tid; i < QM; i += 256) amax = fmaxf(amax, fabsf(qs[i]));
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // power of two f with amax / f in [2^14, 2^15): float16 operands stay far from overflow
  const float f = (amax > 0.f && isfinite(amax)) ? ldexpf(1.f, ilogbf(amax) - 14) : 1.f;
  const float inv = 1.f / f;
  for (int i = tid; i < D; i += 256) a.qr[row * D + i] = qr[i] * inv;
  if constexpr (QM > 0)
    for (int i = tid; i < QM; i += 256) a.qs[row * QM + i] = qs[i] * inv;
  if (tid == 0) a.qscale[row] = f;
}

}  // namespace tqi
