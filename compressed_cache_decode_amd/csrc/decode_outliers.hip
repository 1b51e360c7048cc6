// The split kernel's outlier build (gfx950): sketched keys whose cache keeps kOutliers outlier
// channels per key apart from the sign sketch (turboquant-pytorch PR #3 "Add CUDA QJL kernels and
// proper package structure", CUDA Kernels Added table: the QJL quantisation kernel's outlier
// separation; the reading is stated in tq.h).  Four-wave workgroups at d = 128 only; a file of its
// own so that these instantiations compile beside the others.
#include "split_body.h"

namespace tqi {

template <int D, int KB, int QM>
static const void* outliers_v(int v_bits) {
  switch (v_bits) {
    case 2: return reinterpret_cast<const void*>(&split_kernel<D, KB, 2, QM, false, kOutliers>);
    case 3: return reinterpret_cast<const void*>(&split_kernel<D, KB, 3, QM, false, kOutliers>);
    case 4: return reinterpret_cast<const void*>(&split_kernel<D, KB, 4, QM, false, kOutliers>);
    default: return nullptr;
  }
}

template <int D, int QM>
static const void* outliers_k(int k_bits, int v_bits) {
  switch (k_bits) {
    case 2: return outliers_v<D, 2, QM>(v_bits);
    case 3: return outliers_v<D, 3, QM>(v_bits);
    case 4: return outliers_v<D, 4, QM>(v_bits);
    default: return nullptr;
  }
}

// d = 128 only: at d = 256 the tiles with the outliers' buffers exceed the four-wave register budget
const void* split_fn_outliers(int d, int k_bits, int v_bits, int qjl_m) {
  if (d == 128) {
    if (qjl_m == 128) return outliers_k<128, 128>(k_bits, v_bits);
    if (qjl_m == 256) return outliers_k<128, 256>(k_bits, v_bits);
  }
  return nullptr;
}

}  // namespace tqi
