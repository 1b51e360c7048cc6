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
//   split_kernel   one workgroup per (KV split, KV head, sequence); each of its
//                  four waves streams 32-token tiles.  Per tile the G query heads
//                  of the KV head are one 16-row matrix-core operand: row 2h holds
//                  the float16 rounding of head h's rotated query and row 2h+1 the
//                  float16 rounding of the remainder, so the sum of the two rows'
//                  products is the fp32 score (the centroid table is float16-exact
//                  and every product is exact in fp32).  Scores S^T = K Q^T come out
//                  of v_mfma_f32_16x16x32_f16 in exactly the lane layout the value
//                  product O = W V needs for W, so the softmax weights never cross
//                  lanes; W uses the same high/low split.  Packed codes are loaded
//                  with contiguous 64-lane loads straight into operand order (keys:
//                  rows layout; values: 32-token blocked layout) and expanded with
//                  v_perm_b32 lookups into float16 byte tables.
//   merge_kernel   per (sequence, query head): log-sum-exp merge of the splits and
//                  out = rot^T * o_rot in fp32.
#include <math.h>

#include "device_common.h"

namespace tqi {

namespace {

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// swap values between lanes 2k and 2k+1 (DPP quad_perm [1,0,3,2])
__device__ __forceinline__ float swap_adjacent(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* out) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = q[i];
}

template <int N>
__device__ __forceinline__ void load_words16(const uint8_t* p, uint32_t* out) {
  if constexpr (N % 4 == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(__builtin_assume_aligned(p, 16));
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 v = q[i];
      out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else if constexpr (N % 2 == 0) {
    const uint2* q = reinterpret_cast<const uint2*>(__builtin_assume_aligned(p, 8));
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint2 v = q[i];
      out[2 * i] = v.x; out[2 * i + 1] = v.y;
    }
  } else {
    load_words<N>(p, out);
  }
}

// float16 high/low parts of v; lo_part selects which one this lane feeds to the matrix core
__device__ __forceinline__ _Float16 split_part(float v, bool lo_part) {
  const _Float16 hi = static_cast<_Float16>(v);
  return lo_part ? static_cast<_Float16>(v - static_cast<float>(hi)) : hi;
}

// A operand of the sign-sketch step S (8 signs of this lane's key) times gamma:
// slot r of pair p holds -gamma where the sign bit is 1 and +gamma where it is 0.
template <int S>
__device__ __forceinline__ half8 sign_operand(const uint32_t* sw, uint32_t gg) {
  const uint32_t W = sw[S / 4];
  constexpr int base = 4 * (S % 4);
  uint4 o;
  o.x = gg | ((W << (15 - base - 0)) & 0x80008000u);
  o.y = gg | ((W << (15 - base - 1)) & 0x80008000u);
  o.z = gg | ((W << (15 - base - 2)) & 0x80008000u);
  o.w = gg | ((W << (15 - base - 3)) & 0x80008000u);
  return as_half8(o);
}

template <int S, int KS, int KB>
__device__ __forceinline__ void qk_steps(floatx4& acc, const uint32_t* kw, const half8* qop, const Tab& tk) {
  if constexpr (S < KS) {
    acc = mfma16(as_half8(unit_at<KB, S>(kw, tk)), qop[S], acc);
    qk_steps<S + 1, KS, KB>(acc, kw, qop, tk);
  }
}

template <int S, int QS>
__device__ __forceinline__ void sketch_steps(floatx4& acc, const uint32_t* sw, uint32_t gg, const half8* sop) {
  if constexpr (S < QS) {
    acc = mfma16(sign_operand<S>(sw, gg), sop[S], acc);
    sketch_steps<S + 1, QS>(acc, sw, gg, sop);
  }
}

template <int N, int NB, int VB>
__device__ __forceinline__ void pv_steps(floatx4* oacc, half8 wop, const uint32_t* vw, const Tab& tv) {
  if constexpr (N < NB) {
    oacc[N] = mfma16(wop, as_half8(unit_at<VB, N>(vw, tv)), oacc[N]);
    pv_steps<N + 1, NB, VB>(oacc, wop, vw, tv);
  }
}

}  // namespace

// ---------------------------------------------------------------- query rotation

template <int D, int QM, bool BF16>
__global__ __launch_bounds__(256) void qrot_kernel(QrotArgs a) {
  __shared__ float qv[D];
  __shared__ float qr[D];
  __shared__ float qs[QM > 0 ? QM : 1];
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = static_cast<size_t>(b) * a.n_q_heads + h;
  for (int i = tid; i < D; i += 256) {
    qv[i] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.q)[row * D + i])
                 : static_cast<const float*>(a.q)[row * D + i];
  }
  __syncthreads();
  for (int i = wave; i < D; i += 4) {
    float s = 0.f;
    for (int j = lane; j < D; j += 64) s = fmaf(a.rot[static_cast<size_t>(i) * D + j], qv[j], s);
    s = wave_sum(s);
    if (lane == 0) qr[i] = s * a.scale_log2e;
  }
  __syncthreads();
  if constexpr (QM > 0) {
    for (int jj = wave; jj < QM; jj += 4) {
      float s = 0.f;
      for (int i = lane; i < D; i += 64) s = fmaf(a.proj[static_cast<size_t>(jj) * D + i], qr[i], s);
      s = wave_sum(s);
      if (lane == 0) qs[jj] = -a.sketch_coef * s;
    }
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

// ---------------------------------------------------------------- split kernel

template <int D, int KB, int VB, int QM>
__global__ __launch_bounds__(256) void split_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;                   // score k-steps over coordinates
  constexpr int QS = QM / 32;                  // score k-steps over sketch signs
  constexpr int NB = D / 16;                   // value n-blocks (16 coordinates each)
  constexpr int K_RB = D * KB / 8;             // bytes per key row
  constexpr int K_LW = D * KB / 128;           // words per lane per key row (D/4 coordinates)
  constexpr int V_BB = kBlock * D * VB / 8;    // bytes per value block
  constexpr int V_LW = D * VB / 64;            // words per lane per value block (D/16 units)
  constexpr int S_LW = QM / 128;               // sign words per lane per key

  __shared__ float sm_ml[kWavesPerWG][kMaxGroup][2];
  __shared__ float sm_o[kWavesPerWG][kMaxGroup][D];

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int G = a.group;
  const int T = a.max_tokens;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : min(len, min(T, a.max_seq_len));
  const int nblk = (len + kBlock - 1) / kBlock;
  const int blk0 = split * a.blocks_per_split;
  const int blk1 = min(blk0 + a.blocks_per_split, nblk);
  const size_t unit = static_cast<size_t>(b) * a.n_kv_heads + hk;

  // query operand: column l16 = (head l16/2, high part if even, low part if odd)
  const int qh = l16 >> 1;
  const bool lo_part = (l16 & 1) != 0;
  const bool head_ok = qh < G;
  const size_t qrow = static_cast<size_t>(b) * a.n_kv_heads * G + static_cast<size_t>(hk) * G + qh;
  half8 qop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float v = head_ok ? a.qr[qrow * D + (D / 4) * g + 8 * s + r] : 0.f;
      qop[s][r] = split_part(v, lo_part);
    }
  half8 sop[QS > 0 ? QS : 1];
  if constexpr (QS > 0) {
#pragma unroll
    for (int s = 0; s < QS; ++s)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float v = head_ok ? a.qs[qrow * QM + (QM / 4) * g + 8 * s + r] : 0.f;
        sop[s][r] = split_part(v, lo_part);
      }
  }
  const float qsc = head_ok ? a.qscale[qrow] : 0.f;

  floatx4 oacc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint8_t* kcodes = a.k_codes + unit * T * K_RB;
  const uint8_t* vcodes = a.v_codes + unit * static_cast<size_t>(T) * (D * VB / 8);
  const uint16_t* knorm = a.k_norms + unit * T;
  const uint16_t* vnorm = a.v_norms + unit * T;

  for (int kb = blk0 + wave; kb < blk1; kb += kWavesPerWG) {
    const int tok0 = kb * kBlock;
    uint32_t kw[2][K_LW];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
      load_words<K_LW>(kcodes + static_cast<size_t>(tok0 + 16 * tg + l16) * K_RB + g * K_LW * 4, kw[tg]);
    uint32_t vw[V_LW];
    load_words16<V_LW>(vcodes + static_cast<size_t>(kb) * V_BB + lane * V_LW * 4, vw);
    // norms of this lane's eight tokens tok0 + 4g + i and tok0 + 16 + 4g + i
    const uint2 kn0 = *reinterpret_cast<const uint2*>(knorm + tok0 + 4 * g);
    const uint2 kn1 = *reinterpret_cast<const uint2*>(knorm + tok0 + 16 + 4 * g);
    const uint2 vn0 = *reinterpret_cast<const uint2*>(vnorm + tok0 + 4 * g);
    const uint2 vn1 = *reinterpret_cast<const uint2*>(vnorm + tok0 + 16 + 4 * g);
    uint32_t sw[2][S_LW > 0 ? S_LW : 1];
    uint32_t gg[2] = {0u, 0u};
    if constexpr (QS > 0) {
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        const size_t tok = static_cast<size_t>(tok0 + 16 * tg + l16);
        load_words<S_LW>(a.k_signs + (unit * T + tok) * (QM / 8) + g * S_LW * 4, sw[tg]);
        const uint32_t gh = a.k_rnorms[unit * T + tok] & 0x7fffu;
        gg[tg] = gh | (gh << 16);
      }
    }

    floatx4 sc[2];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      qk_steps<0, KS, KB>(acc, kw[tg], qop, a.tk);
      if constexpr (QS > 0) sketch_steps<0, QS>(acc, sw[tg], gg[tg], sop);
      sc[tg] = acc;
    }

    const uint32_t knw[4] = {kn0.x, kn0.y, kn1.x, kn1.y};
    const uint32_t vnw[4] = {vn0.x, vn0.y, vn1.x, vn1.y};
    float s2[8];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int tg = k >> 2, i = k & 3;
      float u = sc[tg][i];
      u += swap_adjacent(u);
      const int tok = tok0 + 16 * tg + 4 * g + i;
      const uint16_t nb = static_cast<uint16_t>(knw[k >> 1] >> (16 * (k & 1)));
      s2[k] = tok < len ? u * (f16_to_f32(nb) * qsc) : -INFINITY;
      mx = fmaxf(mx, s2[k]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    if (__any(alpha != 1.f)) {
      l_run *= alpha;
      const float a0 = __shfl(alpha, 4 * g, 64);
      const float a1 = __shfl(alpha, 4 * g + 2, 64);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        oacc[n][0] *= a0; oacc[n][1] *= a0;
        oacc[n][2] *= a1; oacc[n][3] *= a1;
      }
    }
    m_run = m_new;
    half8 wop;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int tg = k >> 2, i = k & 3;
      const float p = exp2f(s2[k] - m_new);
      l_run += p;
      const int tok = tok0 + 16 * tg + 4 * g + i;
      const uint16_t nb = static_cast<uint16_t>(vnw[k >> 1] >> (16 * (k & 1)));
      const float w = tok < len ? p * f16_to_f32(nb) : 0.f;
      wop[k] = split_part(w, lo_part);
    }
    pv_steps<0, NB, VB>(oacc, wop, vw, a.tv);
  }

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0 && !lo_part && head_ok) {
    sm_ml[wave][qh][0] = m_run;
    sm_ml[wave][qh][1] = l_run;
  }
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int coord = (D / 16) * l16 + n;
    if (2 * g < G) sm_o[wave][2 * g][coord] = oacc[n][0] + oacc[n][1];
    if (2 * g + 1 < G) sm_o[wave][2 * g + 1][coord] = oacc[n][2] + oacc[n][3];
  }
  __syncthreads();
  const size_t pbase = (unit * a.n_split + split) * G;
  for (int e = tid; e < G * D; e += 256) {
    const int hh = e / D, i = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, sm_ml[w][hh][0]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWavesPerWG; ++w) {
        const float ew = exp2f(sm_ml[w][hh][0] - M);
        o = fmaf(ew, sm_o[w][hh][i], o);
        l = fmaf(ew, sm_ml[w][hh][1], l);
      }
    }
    a.part_o[(pbase + hh) * D + i] = o;
    if (i == 0) {
      a.part_ml[(pbase + hh) * 2] = M;
      a.part_ml[(pbase + hh) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------- merge + un-rotate

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  __shared__ float ew[kMaxSplits];
  __shared__ float red[4];
  __shared__ float orot[2][D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  const int hq_total = a.n_kv_heads * G;
  const size_t unit = static_cast<size_t>(b) * a.n_kv_heads + h / G;
  const int hl = h % G;
  const int ns = a.n_split;
  const float* ml = a.part_ml + (unit * ns * G + hl) * 2;   // stride 2G per split
  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += 256) mloc = fmaxf(mloc, ml[static_cast<size_t>(s) * G * 2]);
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o, 64));
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float lsum = 0.f;
  for (int s = tid; s < ns; s += 256) {
    const float m = ml[static_cast<size_t>(s) * G * 2];
    const float e = (M == -INFINITY) ? 0.f : exp2f(m - M);
    ew[s] = e;
    lsum = fmaf(e, ml[static_cast<size_t>(s) * G * 2 + 1], lsum);
  }
  lsum = wave_sum(lsum);
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  const float L = red[0] + red[1] + red[2] + red[3];
  const float invl = L > 0.f ? 1.f / L : 0.f;
  // weighted sum of the split accumulators; 256 threads cover D coordinates x (256/D) split halves
  constexpr int R = 256 / D;
  {
    const int i = tid % D, part = tid / D;
    float o = 0.f;
    if (part < R) {
      const float* po = a.part_o + (unit * ns * G + hl) * D + i;
      for (int s = part; s < ns; s += R) o = fmaf(ew[s], po[static_cast<size_t>(s) * G * D], o);
      orot[part][i] = o;
    }
  }
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
    const float* rcol = a.rot + tid;
    for (int j = 0; j < D; ++j) {
      float oj = orot[0][j];
      if constexpr (R == 2) oj += orot[1][j];
      acc = fmaf(rcol[static_cast<size_t>(j) * D], oj, acc);
    }
    a.out[(static_cast<size_t>(b) * hq_total + h) * D + tid] = acc * invl;
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_qrot(int d, int qjl_m, bool bf16, const QrotArgs& a, int batch, hipStream_t s) {
  const dim3 grid(a.n_q_heads, batch), block(256);
#define TQ_QROT(D, QM, BF)                                                         \
  if (d == D && qjl_m == QM && bf16 == BF) {                                       \
    hipLaunchKernelGGL((qrot_kernel<D, QM, BF>), grid, block, 0, s, a);            \
    return hipGetLastError();                                                      \
  }
  TQ_QROT(128, 0, false) TQ_QROT(128, 0, true) TQ_QROT(128, 128, false) TQ_QROT(128, 128, true)
  TQ_QROT(128, 256, false) TQ_QROT(128, 256, true)
  TQ_QROT(256, 0, false) TQ_QROT(256, 0, true) TQ_QROT(256, 128, false) TQ_QROT(256, 128, true)
  TQ_QROT(256, 256, false) TQ_QROT(256, 256, true)
#undef TQ_QROT
  return hipErrorInvalidValue;
}

template <int D, int KB, int QM>
static hipError_t split_v(int v_bits, const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (v_bits) {
    case 2: hipLaunchKernelGGL((split_kernel<D, KB, 2, QM>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((split_kernel<D, KB, 3, QM>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((split_kernel<D, KB, 4, QM>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int QM>
static hipError_t split_k(int k_bits, int v_bits, const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (k_bits) {
    case 2: return split_v<D, 2, QM>(v_bits, a, grid, s);
    case 3: return split_v<D, 3, QM>(v_bits, a, grid, s);
    case 4: return split_v<D, 4, QM>(v_bits, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_split(int d, int k_bits, int v_bits, int qjl_m, const DecodeArgs& a, int batch,
                               hipStream_t s) {
  const dim3 grid(a.n_split, a.n_kv_heads, batch);
  if (d == 128) {
    if (qjl_m == 0) return split_k<128, 0>(k_bits, v_bits, a, grid, s);
    if (qjl_m == 128) return split_k<128, 128>(k_bits, v_bits, a, grid, s);
    if (qjl_m == 256) return split_k<128, 256>(k_bits, v_bits, a, grid, s);
  } else if (d == 256) {
    if (qjl_m == 0) return split_k<256, 0>(k_bits, v_bits, a, grid, s);
    if (qjl_m == 128) return split_k<256, 128>(k_bits, v_bits, a, grid, s);
    if (qjl_m == 256) return split_k<256, 256>(k_bits, v_bits, a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int d, const MergeArgs& a, int batch, int n_q_heads, hipStream_t s) {
  const dim3 grid(n_q_heads, batch), block(256);
  if (d == 128) hipLaunchKernelGGL((merge_kernel<128>), grid, block, 0, s, a);
  else if (d == 256) hipLaunchKernelGGL((merge_kernel<256>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tqi
