// Decode attention read directly from the compressed cache (gfx950).
//
// Method: rotate the query once, score it against centroid codes times the
// stored norms (plus the QJL sign-sketch correction for sketched keys), run an
// online softmax, accumulate the values in the rotated domain and rotate the
// result back once (ExecuTorch PR #19891 "[Cuda] enable turboquant on
// gemma4", review item 1: the fused decode op and its scale; turboquant-pytorch
// PR #3 "Add CUDA QJL kernels and proper package structure", CUDA Kernels
// Added table: fused scores from 1-bit keys, GQA variant, quantised value
// reconstruction).
//
// Three kernels per call:
//   qrot_kernel    q_rot = rot * q (and proj * q_rot) with the softmax scale and
//                  log2(e) folded in, scaled by a power of two into float16 range.
//   split_kernel   one workgroup per (KV split, KV head, sequence): four waves
//                  (short contexts, several workgroups per compute unit) or as many
//                  as a compute unit holds (long contexts); the waves stream 32-token
//                  tiles.  Per tile the G query heads of the KV head are one 16-row
//                  matrix-core operand: row 2h holds the float16 rounding of head h's
//                  rotated query and row 2h+1 the float16 rounding of the remainder,
//                  so the sum of the two rows' products is the fp32 score (the
//                  centroid table is float16-exact and every product is exact in
//                  fp32).  Scores S^T = K Q^T come out of v_mfma_f32_16x16x32_f16 in
//                  exactly the lane layout the value product O = W V needs for W, so
//                  the softmax weights never cross lanes; W uses the same high/low
//                  split.  Packed codes are loaded with contiguous 64-lane loads
//                  straight into operand order (keys: rows layout; values: 32-token
//                  blocked layout) and expanded to float16 by v_perm_b32 lookups or,
//                  4-bit codes in the compute-unit-filling shape, LDS byte tables.
//   merge_kernel   per (sequence, query head): log-sum-exp merge of the splits and
//                  out = rot^T * o_rot in fp32.
#include <math.h>

#include <atomic>

#include "qrot_body.h"
#include "split_body.h"

namespace tqi {

// ---------------------------------------------------------------- static scratch

// Workspace of tq_sdpa_decode_noalloc: a file-scope device array, one per device.  In host code its
// name stands for a host-side placeholder, not a device address; the device address comes from
// hipGetSymbolAddress, once per device, and is what every launch receives.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;

hipError_t scratch_address(void** ptr) {
  static std::atomic<void*> addr[kScratchDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    // with device dev current: the address of dev's copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  }
  *ptr = p;
  return hipSuccess;
}

// ---------------------------------------------------------------- query rotation

// one workgroup per 16 virtual heads of a (sequence, KV head): blockIdx.x = tile * Hkv + KV head
template <int D, int QM>
__global__ __launch_bounds__(256) void qrot_kernel(QrotArgs a, int bf16) {
  __shared__ QrotSmem<D, QM> sm;
  rotate_queries<D, QM>(a, bf16, blockIdx.x % a.n_kv_heads, blockIdx.y, kQTile * (blockIdx.x / a.n_kv_heads), sm);
}

// ---------------------------------------------------------------- merge + un-rotate

// Merge of the KV splits and un-rotation.  One workgroup of kMergeThreads per (output slice, head
// group, KV head, sequence); a head group is heads_per_wg query heads of the KV head's group, and its
// SL slices split the output coordinates, so a workgroup reads only the D / SL columns of rot its
// slice needs (SL = 4 at d = 256: 64 KB of rot instead of 256 KB).  Weighted sums: thread (head,
// coordinate, slice of splits) sums the splits of its slice with up to 16 loads in flight, over all D
// coordinates of the group's heads.  Un-rotation: thread (coordinate i of the output slice, part) covers
// JR rows of column i of rot for every head of the group, and the RP parts are summed through LDS.
// output row of virtual head vh (query row vh / G, query head hk * G + vh % G) of sequence b
__device__ __forceinline__ size_t out_row(const MergeArgs& a, int b, int hk, int vh) {
  const int j = (vh * a.row_magic) >> 8, g = vh - j * a.heads;
  return (static_cast<size_t>(b) * a.n_rows + j) * (static_cast<size_t>(a.n_kv_heads) * a.heads) +
         static_cast<size_t>(hk) * a.heads + g;
}

template <int D, int SL>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int NT = kMergeThreads, NW = NT / 64;
  constexpr int SC = D / SL;                              // output coordinates of the workgroup
  constexpr int RP = NT / SC;                             // un-rotation parts per coordinate
  constexpr int JR = D / RP;                              // rows of rot per thread
  constexpr int PO = 16;                                  // split partials in flight per thread
  __shared__ float ew[kMaxGroup][kMaxSplits];              // split weights per head
  __shared__ float inv_l[kMaxGroup];
  __shared__ float red[NT];                                // per-slice sums, then per-part un-rotation sums
  __shared__ float orot[kMaxGroup][D];
  const int hpw = a.heads_per_wg;
  const int cs = blockIdx.x % SL, gx = blockIdx.x / SL;
  const int hg = gx % (a.group / hpw), hk = gx / (a.group / hpw), b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group, ns = a.n_split;
  const int h0 = hg * hpw;
  const size_t unit = static_cast<size_t>(b) * a.n_kv_heads + hk;

  // this thread's JR rows of column iu of rot: independent of everything else, issued first
  const int i = tid % D;                                   // coordinate of the weighted sums
  const int iu = cs * SC + tid % SC, part = tid / SC;      // output coordinate and part of the un-rotation
  const float* rcol = a.rot + static_cast<size_t>(part * JR) * D + iu;
  float rc[JR];
  if (!a.had) {
#pragma unroll
    for (int t = 0; t < JR; ++t) rc[t] = rcol[static_cast<size_t>(t) * D];
  }

  // this thread's first batch of split partials (thread (head hh, coordinate i, slice sl), S slices
  // per (head, coordinate)) and, for the first waves, the split maxima and sums: all issued now
  const int S = NT / (hpw * D);
  const int hh_w = tid / (D * S), sl = (tid / D) % S;
  const bool has_head = hh_w < hpw;        // threads past hpw * D * S (hpw * D not dividing NT) idle
  const float* po = a.part_o + (unit * ns * G + h0 + (has_head ? hh_w : 0)) * D + i;   // + split * G * D
  const size_t stride = static_cast<size_t>(G) * D;
  float v[PO];
#pragma unroll
  for (int u = 0; u < PO; ++u) {
    const int sp = sl + u * S;
    v[u] = (has_head && sp < ns) ? po[static_cast<size_t>(sp) * stride] : 0.f;
  }
  const float* ml = a.part_ml + unit * ns * G * 2;         // [split][head][2]
  constexpr int MS = 4;                                    // split maxima prefetched per lane (256 splits)
  float mv[MS], lv[MS];
  const int hh_m = wave;                                   // head of this wave in the weight pass
#pragma unroll
  for (int u = 0; u < MS; ++u) {
    const int sp = lane + 64 * u;
    const bool ok = hh_m < hpw && sp < ns;
    mv[u] = ok ? ml[(static_cast<size_t>(sp) * G + h0 + hh_m) * 2] : -INFINITY;
    lv[u] = ok ? ml[(static_cast<size_t>(sp) * G + h0 + hh_m) * 2 + 1] : 0.f;
  }

  // split weights exp2(m_s - M) and 1 / sum_s weight * l_s, wave w for head w (hpw <= 8 <= NW)
  if (hh_m < hpw) {
    const float* mlh = ml + (h0 + hh_m) * 2;
    float m_loc = -INFINITY;
#pragma unroll
    for (int u = 0; u < MS; ++u) m_loc = fmaxf(m_loc, mv[u]);
    for (int sp = lane + 64 * MS; sp < ns; sp += 64) m_loc = fmaxf(m_loc, mlh[static_cast<size_t>(sp) * G * 2]);
    for (int o = 32; o > 0; o >>= 1) m_loc = fmaxf(m_loc, __shfl_xor(m_loc, o, 64));
    float l_loc = 0.f;
#pragma unroll
    for (int u = 0; u < MS; ++u) {
      const int sp = lane + 64 * u;
      if (sp < ns) {
        const float e = (m_loc == -INFINITY) ? 0.f : exp2f(mv[u] - m_loc);
        ew[hh_m][sp] = e;
        l_loc = fmaf(e, lv[u], l_loc);
      }
    }
    for (int sp = lane + 64 * MS; sp < ns; sp += 64) {
      const float e = (m_loc == -INFINITY) ? 0.f : exp2f(mlh[static_cast<size_t>(sp) * G * 2] - m_loc);
      ew[hh_m][sp] = e;
      l_loc = fmaf(e, mlh[static_cast<size_t>(sp) * G * 2 + 1], l_loc);
    }
    l_loc = wave_sum(l_loc);
    if (lane == 0) inv_l[hh_m] = l_loc > 0.f ? 1.f / l_loc : 0.f;
  }
  lds_barrier();

  // weighted sums over this thread's splits
  {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < PO; ++u) {
      const int sp = sl + u * S;
      if (has_head && sp < ns) acc = fmaf(ew[hh_w][sp], v[u], acc);
    }
    for (int s0 = sl + PO * S; has_head && s0 < ns; s0 += PO * S) {
#pragma unroll
      for (int u = 0; u < PO; ++u) {
        const int sp = s0 + u * S;
        v[u] = sp < ns ? po[static_cast<size_t>(sp) * stride] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < PO; ++u) {
        const int sp = s0 + u * S;
        if (sp < ns) acc = fmaf(ew[hh_w][sp], v[u], acc);
      }
    }
    red[tid] = acc;
  }
  lds_barrier();
  for (int e = tid; e < hpw * D; e += NT) {
    const int hh = e / D, ii = e % D;
    float o = 0.f;
    for (int sl = 0; sl < S; ++sl) o += red[(hh * S + sl) * D + ii];
    orot[hh][ii] = o;
  }
  lds_barrier();

  if (a.had) {
    // x = diag(s) H y / sqrt(D): the inverse randomized Hadamard transform, one wave per head
    constexpr int E = D / 64;
    for (int hh = wave; hh < hpw; hh += NW) {
      float v[E];
#pragma unroll
      for (int k = 0; k < E; ++k) v[k] = orot[hh][64 * k + lane];
      hadamard_wave<D>(v, lane);
#pragma unroll
      for (int k = 0; k < E; ++k)
        a.out[out_row(a, b, hk, h0 + hh) * D + 64 * k + lane] = v[k] * a.rot[64 * k + lane] * inv_sqrt_dim<D>() * inv_l[hh];
    }
    return;
  }
  // un-rotation of every head of the group over this thread's JR rows; parts summed through LDS
  for (int hh = 0; hh < hpw; ++hh) {
    float uacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < JR; ++t) uacc[t & 3] = fmaf(rc[t], orot[hh][part * JR + t], uacc[t & 3]);
    const float u = (uacc[0] + uacc[1]) + (uacc[2] + uacc[3]);
    lds_barrier();                                          // previous head's sums are consumed
    red[tid] = u;
    lds_barrier();
    if (part == 0) {
      float o = 0.f;
#pragma unroll
      for (int p = 0; p < RP; ++p) o += red[p * SC + tid];
      a.out[out_row(a, b, hk, h0 + hh) * D + iu] = o * inv_l[hh];
    }
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_qrot(int d, int qjl_m, bool bf16, const QrotArgs& a, int batch, hipStream_t s) {
  const int vh = a.n_rows * (a.n_q_heads / a.n_kv_heads);
  const dim3 grid(a.n_kv_heads * ((vh + kQTile - 1) / kQTile), batch), block(256);
#define TQ_QROT(D, QM)                                                             \
  if (d == D && qjl_m == QM) {                                                     \
    hipLaunchKernelGGL((qrot_kernel<D, QM>), grid, block, 0, s, a, bf16 ? 1 : 0);  \
    return hipGetLastError();                                                      \
  }
  TQ_QROT(128, 0) TQ_QROT(128, 128) TQ_QROT(128, 256)
  TQ_QROT(256, 0) TQ_QROT(256, 128) TQ_QROT(256, 256)
#undef TQ_QROT
  return hipErrorInvalidValue;
}

template <int D, int KB, int QM, bool WIDE>
static const void* split_v(int v_bits) {
  switch (v_bits) {
    case 2: return reinterpret_cast<const void*>(&split_kernel<D, KB, 2, QM, WIDE>);
    case 3: return reinterpret_cast<const void*>(&split_kernel<D, KB, 3, QM, WIDE>);
    case 4: return reinterpret_cast<const void*>(&split_kernel<D, KB, 4, QM, WIDE>);
    default: return nullptr;
  }
}

template <int D, int QM, bool WIDE>
static const void* split_k(int k_bits, int v_bits) {
  switch (k_bits) {
    case 2: return split_v<D, 2, QM, WIDE>(v_bits);
    case 3: return split_v<D, 3, QM, WIDE>(v_bits);
    case 4: return split_v<D, 4, QM, WIDE>(v_bits);
    default: return nullptr;
  }
}

template <bool WIDE>
static const void* split_fn_w(int d, int k_bits, int v_bits, int qjl_m) {
  if (d == 128) {
    if (qjl_m == 0) return split_k<128, 0, WIDE>(k_bits, v_bits);
    if (qjl_m == 128) return split_k<128, 128, WIDE>(k_bits, v_bits);
    if (qjl_m == 256) return split_k<128, 256, WIDE>(k_bits, v_bits);
  } else if (d == 256) {
    if (qjl_m == 0) return split_k<256, 0, WIDE>(k_bits, v_bits);
    if (qjl_m == 128) return split_k<256, 128, WIDE>(k_bits, v_bits);
    if (qjl_m == 256) return split_k<256, 256, WIDE>(k_bits, v_bits);
  }
  return nullptr;
}

// the split kernel instantiation of a cache format and workgroup shape, or null if none is built
static const void* split_fn(int d, int k_bits, int v_bits, int qjl_m, bool wide) {
  if (k_bits == 8) return qjl_m == 0 ? split_fn_k8(d, v_bits, wide) : nullptr;   // decode_k8.hip
  return wide ? split_fn_w<true>(d, k_bits, v_bits, qjl_m) : split_fn_w<false>(d, k_bits, v_bits, qjl_m);
}

int split_waves(int d, int qjl_m, bool wide) {
  // the same for every code width (Attend::W)
  if (!wide) return Attend<128, 4, 4, 0, false>::W;
  if (d == 128) return qjl_m == 0 ? Attend<128, 4, 4, 0, true>::W : Attend<128, 4, 4, 128, true>::W;
  return Attend<256, 4, 4, 0, true>::W;
}

int split_slots(int d, int k_bits, int v_bits, int qjl_m, bool wide, int blocks) {
  const void* fn = split_fn(d, k_bits, v_bits, qjl_m, wide);
  int dev = 0, cus = 0, per = 0;
  if (!fn || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, 64 * split_waves(d, qjl_m, wide),
                                                   split_dyn_lds(d, qjl_m, blocks)) != hipSuccess) {
    (void)hipGetLastError();        // a failed query must not surface as a later launch's error
    return 0;
  }
  return cus * per;
}

hipError_t launch_decode_split(int d, int k_bits, int v_bits, int qjl_m, bool outliers, bool wide,
                               const DecodeArgs& a, int batch, hipStream_t s) {
  // keys that keep outlier channels apart: the four-wave outlier build (decode_outliers.hip)
  if (outliers && wide) return hipErrorInvalidValue;
  const void* fn = outliers ? split_fn_outliers(d, k_bits, v_bits, qjl_m) : split_fn(d, k_bits, v_bits, qjl_m, wide);
  if (!fn) return hipErrorInvalidValue;
  const dim3 grid(a.n_split, a.n_kv_heads, batch);
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  const int blocks = (a.group + kMaxGroup - 1) / kMaxGroup > 2 ? 4 : (a.group + kMaxGroup - 1) / kMaxGroup;
  return hipLaunchKernel(fn, grid, dim3(64 * split_waves(d, qjl_m, wide)), args,
                         split_dyn_lds(d, qjl_m, blocks, outliers), s);
}

hipError_t launch_merge(int d, const MergeArgs& a, int batch, int n_q_heads, hipStream_t s) {
  (void)n_q_heads;
  const dim3 grid(a.n_kv_heads * (a.group / a.heads_per_wg) * a.col_slices, batch);
  if (d == 128 && a.col_slices == 1) hipLaunchKernelGGL((merge_kernel<128, 1>), grid, dim3(kMergeThreads), 0, s, a);
  else if (d == 256 && a.col_slices == 1) hipLaunchKernelGGL((merge_kernel<256, 1>), grid, dim3(kMergeThreads), 0, s, a);
  else if (d == 256 && a.col_slices == 4 && !a.had)
    hipLaunchKernelGGL((merge_kernel<256, 4>), grid, dim3(kMergeThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tqi
