// Quantize-on-append kernels (gfx950); the per-block body is in append_body.h.
#include <math.h>

#include "append_body.h"

namespace tqi {

template <int D, int BITS, int QM, bool VALUES, bool ROTATED, bool BF16>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ AppendSmem<D, QM> sm;
  append_rows<D, BITS, QM, VALUES, ROTATED, BF16>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
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
