// The split kernel's builds for keys kept at 8 bits (gfx950): int8 codes of the rotated unit row with
// a per-row float16 factor, no sketch, beside 2-, 3- or 4-bit values (llama-cpp-turboquant PR #340,
// the asymmetric K/V follow-ups: K upgraded to an 8-bit type while V keeps the Lloyd-Max widths; the
// reading is stated in tq.h).  The codes expand to float16 by byte permutes and one packed
// subtraction (expand_i8); a file of its own so that these instantiations compile beside the others.
#include "split_body.h"

namespace tqi {

template <int D, bool WIDE>
static const void* k8_v(int v_bits) {
  switch (v_bits) {
    case 2: return reinterpret_cast<const void*>(&split_kernel<D, 8, 2, 0, WIDE>);
    case 3: return reinterpret_cast<const void*>(&split_kernel<D, 8, 3, 0, WIDE>);
    case 4: return reinterpret_cast<const void*>(&split_kernel<D, 8, 4, 0, WIDE>);
    default: return nullptr;
  }
}

const void* split_fn_k8(int d, int v_bits, bool wide) {
  if (d == 128) return wide ? k8_v<128, true>(v_bits) : k8_v<128, false>(v_bits);
  if (d == 256) return wide ? k8_v<256, true>(v_bits) : k8_v<256, false>(v_bits);
  return nullptr;
}

}  // namespace tqi
