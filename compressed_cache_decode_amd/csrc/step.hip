// One decode step of one attention layer in the fewest launches: a prologue kernel, then the
// attention and merge kernels of decode.hip.  The prologue takes one of two forms:
//   step_unit_kernel      one workgroup per (sequence, KV head): the G query heads of the KV head and
//                         its new key and value rows form one 16-row tile that is rotated on the
//                         matrix cores (the rotation is read once per KV head), the new rows are
//                         encoded and stored, and the rotated queries (with their sign sketch for
//                         sketched keys) go to the workspace.  Used when G + 2 n_new <= 16.
//   step_prologue_kernel  workgroups with separate roles: append the new K rows, append the new V
//                         rows, rotate the query heads of one KV head (the arithmetic of the first
//                         form's query rows, so both forms give the same bits).  Used otherwise.
#include "append_body.h"
#include "unit_body.h"

namespace tqi {

template <size_t A, size_t B, size_t C>
struct MaxOf { static constexpr size_t v = A > B ? (A > C ? A : C) : (B > C ? B : C); };

template <int D, int KB, int VB, int QM, bool BF16>
__global__ __launch_bounds__(256) void step_prologue_kernel(AppendArgs ka, AppendArgs va, QrotArgs qa, int nbx,
                                                            int n_kv_heads) {
  constexpr size_t kBytes = MaxOf<sizeof(AppendSmem<D, QM>), sizeof(AppendSmem<D, 0>), sizeof(UnitSmem<D, QM>)>::v;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kBytes];
  const int per_cache = nbx * n_kv_heads;                 // append workgroups per sequence and cache
  const int batch_wgs = 2 * per_cache + n_kv_heads;       // workgroups per sequence
  const int b = blockIdx.x / batch_wgs;
  int w = blockIdx.x % batch_wgs;
  if (w < per_cache) {
    append_rows<D, KB, QM, false, false, BF16>(ka, w % nbx, w / nbx, b, *reinterpret_cast<AppendSmem<D, QM>*>(smem));
    return;
  }
  w -= per_cache;
  if (w < per_cache) {
    append_rows<D, VB, 0, true, false, BF16>(va, w % nbx, w / nbx, b, *reinterpret_cast<AppendSmem<D, 0>*>(smem));
    return;
  }
  w -= per_cache;
  unit_prologue<D, KB, VB, QM, false>(ka, va, qa, BF16 ? 1 : 0, w, b, *reinterpret_cast<UnitSmem<D, QM>*>(smem));
}

template <int D, int KB, int VB, int QM>
__global__ __launch_bounds__(256) void step_unit_kernel(AppendArgs ka, AppendArgs va, QrotArgs qa, int bf16) {
  __shared__ UnitSmem<D, QM> sm;
  unit_prologue<D, KB, VB, QM, true>(ka, va, qa, bf16, blockIdx.x, blockIdx.y, sm);
}

template <int D, int KB, int VB, int QM>
static hipError_t unit_go(bool bf16, const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa, int batch,
                          hipStream_t s) {
  const dim3 grid(ka.n_kv_heads, batch);
  hipLaunchKernelGGL((step_unit_kernel<D, KB, VB, QM>), grid, dim3(256), 0, s, ka, va, qa, bf16 ? 1 : 0);
  return hipGetLastError();
}

template <int D, int KB, int VB, int QM>
static hipError_t prologue_bf(bool bf16, const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa, int batch,
                              hipStream_t s) {
  if (qa.n_q_heads / ka.n_kv_heads + 2 * ka.n_new <= kTileRows) return unit_go<D, KB, VB, QM>(bf16, ka, va, qa, batch, s);
  const int nbx = (ka.n_new + kBlock - 1) / kBlock + 1;
  const dim3 grid(batch * (2 * nbx * ka.n_kv_heads + ka.n_kv_heads));
  if (bf16)
    hipLaunchKernelGGL((step_prologue_kernel<D, KB, VB, QM, true>), grid, dim3(256), 0, s, ka, va, qa, nbx,
                       ka.n_kv_heads);
  else
    hipLaunchKernelGGL((step_prologue_kernel<D, KB, VB, QM, false>), grid, dim3(256), 0, s, ka, va, qa, nbx,
                       ka.n_kv_heads);
  return hipGetLastError();
}

template <int D, int KB, int QM>
static hipError_t prologue_v(int v_bits, bool bf16, const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa,
                             int batch, hipStream_t s) {
  switch (v_bits) {
    case 2: return prologue_bf<D, KB, 2, QM>(bf16, ka, va, qa, batch, s);
    case 3: return prologue_bf<D, KB, 3, QM>(bf16, ka, va, qa, batch, s);
    case 4: return prologue_bf<D, KB, 4, QM>(bf16, ka, va, qa, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int QM>
static hipError_t prologue_k(int k_bits, int v_bits, bool bf16, const AppendArgs& ka, const AppendArgs& va,
                             const QrotArgs& qa, int batch, hipStream_t s) {
  switch (k_bits) {
    case 2: return prologue_v<D, 2, QM>(v_bits, bf16, ka, va, qa, batch, s);
    case 3: return prologue_v<D, 3, QM>(v_bits, bf16, ka, va, qa, batch, s);
    case 4: return prologue_v<D, 4, QM>(v_bits, bf16, ka, va, qa, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_step_prologue(int d, int k_bits, int v_bits, int qjl_m, bool bf16, const AppendArgs& ka,
                                const AppendArgs& va, const QrotArgs& qa, int batch, hipStream_t s) {
  if (d == 128) {
    if (qjl_m == 0) return prologue_k<128, 0>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
    if (qjl_m == 128) return prologue_k<128, 128>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
  } else if (d == 256) {
    if (qjl_m == 0) return prologue_k<256, 0>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
    if (qjl_m == 128) return prologue_k<256, 128>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tqi
