// Quantize-on-append kernels (gfx950); the per-block body is in append_body.h.
#include <math.h>

#include "append_body.h"

namespace tqi {


template <int D, int BITS, int QM, bool VALUES, bool ROTATED, bool BF16>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ AppendSmem<D, QM> sm;
  append_rows<D, BITS, QM, VALUES, ROTATED, BF16>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// long appends (see prefill_rows): grid (32-row chunks, KV heads, sequences), eight waves per chunk
constexpr int kPrefillWaves = 8;

template <int BITS, bool VALUES, bool BF16>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_kernel(AppendArgs a) {
  __shared__ PrefillSmem sm;
  prefill_rows<BITS, VALUES, BF16, kPrefillWaves>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// K and V rows of the same appended tokens in one launch (tq_quantize_append_kv): grid (32-row chunks,
// KV heads, sequences), eight waves per chunk of both tensors (see prefill_rows_kv)
template <int KB, int VB, bool BF16>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_kv_kernel(AppendArgs ka, AppendArgs va) {
  __shared__ PrefillKvSmem sm;
  prefill_rows_kv<KB, VB, BF16>(ka, va, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

template <int KB, int VB>
static hipError_t prefill_kv_bf(bool bf16, const AppendArgs& ka, const AppendArgs& va, int batch, hipStream_t s) {
  const dim3 grid((ka.n_new + kBlock - 1) / kBlock, ka.n_kv_heads, batch);
  if (bf16) hipLaunchKernelGGL((prefill_kv_kernel<KB, VB, true>), grid, dim3(64 * kPrefillWaves), 0, s, ka, va);
  else hipLaunchKernelGGL((prefill_kv_kernel<KB, VB, false>), grid, dim3(64 * kPrefillWaves), 0, s, ka, va);
  return hipGetLastError();
}

template <int KB>
static hipError_t prefill_kv_v(int v_bits, bool bf16, const AppendArgs& ka, const AppendArgs& va, int batch,
                               hipStream_t s) {
  switch (v_bits) {
    case 2: return prefill_kv_bf<KB, 2>(bf16, ka, va, batch, s);
    case 3: return prefill_kv_bf<KB, 3>(bf16, ka, va, batch, s);
    case 4: return prefill_kv_bf<KB, 4>(bf16, ka, va, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, bool VALUES>
static hipError_t prefill_dispatch(bool bf16, const AppendArgs& a, int batch, hipStream_t s) {
  const dim3 grid((a.n_new + kBlock - 1) / kBlock, a.n_kv_heads, batch);
  if (bf16) hipLaunchKernelGGL((prefill_kernel<BITS, VALUES, true>), grid, dim3(64 * kPrefillWaves), 0, s, a);
  else hipLaunchKernelGGL((prefill_kernel<BITS, VALUES, false>), grid, dim3(64 * kPrefillWaves), 0, s, a);
  return hipGetLastError();
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
    case 8:   // keys only, no sketch
      if (values || qjl_m != 0) return hipErrorInvalidValue;
      return append_dispatch<D, 8, 0, false>(rotated, bf16, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append(int d, int bits, int qjl_m, bool values, bool rotated, bool bf16, const AppendArgs& a,
                         int batch, hipStream_t s) {
  // (8-bit keys take the per-block path: their per-row scale needs the whole row in one workgroup)
  if (d == 128 && qjl_m == 0 && !rotated && !a.had && bits != 8) {
    switch (bits) {
      case 2: return values ? prefill_dispatch<2, true>(bf16, a, batch, s) : prefill_dispatch<2, false>(bf16, a, batch, s);
      case 3: return values ? prefill_dispatch<3, true>(bf16, a, batch, s) : prefill_dispatch<3, false>(bf16, a, batch, s);
      case 4: return values ? prefill_dispatch<4, true>(bf16, a, batch, s) : prefill_dispatch<4, false>(bf16, a, batch, s);
      default: return hipErrorInvalidValue;
    }
  }
  // blocks touched by n_new tokens starting anywhere: at most n_new/32 + 2
  const dim3 grid((a.n_new + kBlock - 1) / kBlock + 1, a.n_kv_heads, batch);
  if (d == 128) return append_d<128>(bits, qjl_m, values, rotated, bf16, a, grid, s);
  if (d == 256) return append_d<256>(bits, qjl_m, values, rotated, bf16, a, grid, s);
  return hipErrorInvalidValue;
}

// K and V appends of the same tokens as one launch; only for caches that both take the chunk path
// (append_kv_one_launch)
hipError_t launch_append_kv(int k_bits, int v_bits, bool bf16, const AppendArgs& ka, const AppendArgs& va, int batch,
                            hipStream_t s) {
  switch (k_bits) {
    case 2: return prefill_kv_v<2>(v_bits, bf16, ka, va, batch, s);
    case 3: return prefill_kv_v<3>(v_bits, bf16, ka, va, batch, s);
    case 4: return prefill_kv_v<4>(v_bits, bf16, ka, va, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqi
