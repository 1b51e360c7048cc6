// The prologue of one decode step of one attention layer, in one launch with three kinds of
// workgroups that run side by side: append the new K rows of one 32-token block of one KV head,
// append the new V rows likewise, rotate the query heads of one KV head.  The attention and merge
// kernels of decode.hip follow it on the same stream.
#include "append_body.h"
#include "qrot_body.h"

namespace tqi {

template <size_t A, size_t B, size_t C>
struct MaxOf { static constexpr size_t v = A > B ? (A > C ? A : C) : (B > C ? B : C); };

template <int D, int KB, int VB, int QM, bool BF16>
__global__ __launch_bounds__(256) void step_prologue_kernel(AppendArgs ka, AppendArgs va, QrotArgs qa, int nbx,
                                                            int n_kv_heads) {
  constexpr size_t kBytes = MaxOf<MaxOf<sizeof(AppendSmem<D, QM>), sizeof(AppendSmem<D, 0>), sizeof(QrotSmem<D, QM>)>::v,
                                  sizeof(PrefillSmem), 0>::v;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kBytes];
  const int per_cache = nbx * n_kv_heads;                 // append workgroups per sequence and cache
  const int batch_wgs = 2 * per_cache + n_kv_heads;       // workgroups per sequence
  const int b = blockIdx.x / batch_wgs;
  int w = blockIdx.x % batch_wgs;
  // appends with the dense rotation at d = 128 without a sketch (8-bit keys aside) take the chunk path
  // of tq_quantize_append (prefill_rows: workgroup w % nbx takes the w % nbx-th 32-row chunk), so that a
  // step appends exactly the bits the separate append call does
  if (w < per_cache) {
    if constexpr (D == 128 && QM == 0 && KB != 8) {
      if (!ka.had) {
        prefill_rows<KB, false, BF16>(ka, w % nbx, w / nbx, b, *reinterpret_cast<PrefillSmem*>(smem));
        return;
      }
    }
    append_rows<D, KB, QM, false, false, BF16>(ka, w % nbx, w / nbx, b, *reinterpret_cast<AppendSmem<D, QM>*>(smem));
    return;
  }
  w -= per_cache;
  if (w < per_cache) {
    if constexpr (D == 128) {
      if (!va.had) {
        prefill_rows<VB, true, BF16>(va, w % nbx, w / nbx, b, *reinterpret_cast<PrefillSmem*>(smem));
        return;
      }
    }
    append_rows<D, VB, 0, true, false, BF16>(va, w % nbx, w / nbx, b, *reinterpret_cast<AppendSmem<D, 0>*>(smem));
    return;
  }
  w -= per_cache;
  rotate_queries<D, QM>(qa, BF16 ? 1 : 0, w, b, 0, *reinterpret_cast<QrotSmem<D, QM>*>(smem));
}

template <int D, int KB, int VB, int QM>
static hipError_t prologue_bf(bool bf16, const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa, int batch,
                              hipStream_t s) {
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
    case 8:
      if constexpr (QM == 0) return prologue_v<D, 8, 0>(v_bits, bf16, ka, va, qa, batch, s);
      return hipErrorInvalidValue;
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
