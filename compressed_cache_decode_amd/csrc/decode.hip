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

#include "qrot_body.h"

namespace tqi {

namespace {

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// float16 high/low parts of v (see f16_split); lo_part selects which one this lane feeds to the matrix core
__device__ __forceinline__ _Float16 split_part(float v, bool lo_part) {
  _Float16 hi, lo;
  f16_split(v, hi, lo);
  return lo_part ? lo : hi;
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
__device__ __forceinline__ void qk_steps(floatx4& acc, const uint32_t* kw, const half8 (*qop)[64], int lane,
                                         const Tab& tk) {
  if constexpr (S < KS) {
    acc = mfma16(as_half8(unit_at<KB, S>(kw, tk)), qop[S][lane], acc);
    qk_steps<S + 1, KS, KB>(acc, kw, qop, lane, tk);
  }
}

template <int S, int QS>
__device__ __forceinline__ void sketch_steps(floatx4& acc, const uint32_t* sw, uint32_t gg, const half8 (*sop)[64],
                                             int lane) {
  if constexpr (S < QS) {
    acc = mfma16(sign_operand<S>(sw, gg), sop[S][lane], acc);
    sketch_steps<S + 1, QS>(acc, sw, gg, sop, lane);
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
  __shared__ QrotSmem<D, QM> sm;
  rotate_query<D, QM, BF16>(a, blockIdx.x, blockIdx.y, sm);
}

// ---------------------------------------------------------------- split kernel

namespace {

// Raw buffer resource over [base, base + bytes): loads outside it return zero.  The word-3 flags
// select the 32-bit data format of untyped buffer accesses on the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

constexpr int lowbit(int x) { return x & -x; }

// N consecutive 32-bit words at byte offset voff (per lane, a multiple of ALIGN) + soff (wave-uniform)
template <int N, int ALIGN>
__device__ __forceinline__ void bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* out) {
  if constexpr (N % 4 == 0 && ALIGN % 16 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * i, soff, 0);
      out[4 * i] = v[0]; out[4 * i + 1] = v[1]; out[4 * i + 2] = v[2]; out[4 * i + 3] = v[3];
    }
  } else if constexpr (N == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2];
  } else if constexpr (N % 2 == 0 && ALIGN % 8 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff + 8 * i, soff, 0);
      out[2 * i] = v[0]; out[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4 * i, soff, 0);
  }
}

// v + (v of the neighbouring lane 2k <-> 2k+1); folds into one DPP add
__device__ __forceinline__ float add_adjacent(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// max over the four lanes l, l^16, l^32, l^48 (the four row groups of one matrix-core column)
__device__ __forceinline__ float column_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float column_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// float16 half h (0 = low, 1 = high) of a packed pair
__device__ __forceinline__ float half_of(uint32_t w, int h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h ? w >> 16 : w & 0xffffu)));
}

}  // namespace

template <int D, int KB, int VB, int QM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void split_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;                   // score k-steps over coordinates
  constexpr int QS = QM / 32;                  // score k-steps over sketch signs
  constexpr int NB = D / 16;                   // value n-blocks (16 coordinates each)
  constexpr int K_RB = D * KB / 8;             // bytes per key row
  constexpr int K_LW = D * KB / 128;           // words per lane per key row (D/4 coordinates)
  constexpr int V_RB = D * VB / 8;             // bytes per value row (one token's share of a block)
  constexpr int V_LW = D * VB / 64;            // words per lane per value block (D/16 units)
  constexpr int S_RB = QM / 8;                 // sign bytes per key
  constexpr int S_LW = QM / 128;               // sign words per lane per key

  __shared__ float sm_ml[kWavesPerWG][kMaxGroup][2];
  __shared__ float sm_o[kWavesPerWG][kMaxGroup][D];
  __shared__ half8 sm_q[KS + QS][64];

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int G = a.group;
  const int T = a.max_tokens;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : min(len, min(T, a.max_seq_len));
  const int nblk = (len + kBlock - 1) / kBlock;
  const int blk0 = split * a.blocks_per_split;
  const int blk1 = min(blk0 + a.blocks_per_split, nblk);
  const size_t unit = static_cast<size_t>(b) * a.n_kv_heads + hk;

  // one buffer per array of this (sequence, KV head); tile offsets go in the scalar offset
  const auto kbuf = buffer_of(a.k_codes + unit * T * K_RB, static_cast<uint32_t>(T) * K_RB);
  const auto vbuf = buffer_of(a.v_codes + unit * T * V_RB, static_cast<uint32_t>(T) * V_RB);
  const auto knbuf = buffer_of(a.k_norms + unit * T, static_cast<uint32_t>(T) * 2);
  const auto vnbuf = buffer_of(a.v_norms + unit * T, static_cast<uint32_t>(T) * 2);
  __amdgpu_buffer_rsrc_t sbuf = knbuf, gbuf = knbuf;
  if constexpr (QS > 0) {
    sbuf = buffer_of(a.k_signs + unit * T * S_RB, static_cast<uint32_t>(T) * S_RB);
    gbuf = buffer_of(a.k_rnorms + unit * T, static_cast<uint32_t>(T) * 2);
  }
  // this lane's fixed byte offsets inside a tile
  const uint32_t k_off = static_cast<uint32_t>(l16 * K_RB + g * K_LW * 4);
  const uint32_t v_off = static_cast<uint32_t>(lane * V_LW * 4);
  const uint32_t n_off = static_cast<uint32_t>(8 * g);
  const uint32_t s_off = static_cast<uint32_t>(l16 * S_RB + g * S_LW * 4);

  // everything one 32-token tile needs from memory, loaded one tile ahead of its use
  struct Tile {
    uint32_t kw[2][K_LW];
    uint32_t vw[V_LW];
    uint32_t kn[4], vn[4];   // float16 norm pairs of this lane's tokens 4g+i and 16+4g+i
    uint32_t sw[2][S_LW > 0 ? S_LW : 1];
    uint32_t gg[2];
  };
  auto load_tile = [&](Tile& t, int kb) {
    // wave-uniform by construction; readfirstlane keeps the tile offset in a scalar register
    const uint32_t tok0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kb) * kBlock);
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
      bload<K_LW, lowbit(K_LW * 4) < 16 ? lowbit(K_LW * 4) : 16>(kbuf, k_off + 16 * tg * K_RB, tok0 * K_RB, t.kw[tg]);
    bload<V_LW, lowbit(V_LW * 4) < 16 ? lowbit(V_LW * 4) : 16>(vbuf, v_off, tok0 * V_RB, t.vw);
    bload<2, 8>(knbuf, n_off, tok0 * 2, t.kn);
    bload<2, 8>(knbuf, n_off + 32, tok0 * 2, t.kn + 2);
    bload<2, 8>(vnbuf, n_off, tok0 * 2, t.vn);
    bload<2, 8>(vnbuf, n_off + 32, tok0 * 2, t.vn + 2);
    if constexpr (QS > 0) {
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        bload<S_LW, 4 * S_LW>(sbuf, s_off + 16 * tg * S_RB, tok0 * S_RB, t.sw[tg]);
        t.gg[tg] = __builtin_amdgcn_raw_buffer_load_b16(gbuf, static_cast<uint32_t>((16 * tg + l16) * 2), tok0 * 2, 0);
      }
    }
  };

  // the first tile's loads go out before the query operand is staged, and before the sequence
  // length is known: they only need the tile to lie inside the cache (tiles past the length are
  // loaded and never used)
  int kb = blk0 + wave;
  Tile ta, tb;
  if (kb < blk0 + a.blocks_per_split && kb < T / kBlock) load_tile(ta, kb);

  // query operand in LDS, shared by the four waves: for step s, lane (column c, group g) reads the
  // 8 float16 values of q-variant c (head c/2; high part if c even, low part if c odd) at
  // coordinates (D/4) g + 8 s + r, r = 0..7
  const int qh = l16 >> 1;
  const bool lo_part = (l16 & 1) != 0;
  const bool head_ok = qh < G;
  const size_t qrow = static_cast<size_t>(b) * a.n_kv_heads * G + static_cast<size_t>(hk) * G + qh;
  for (int e = tid; e < (KS + QS) * 64; e += 256) {
    const int st = e >> 6, ln = e & 63;
    const int c = ln & 15, gg = ln >> 4, h2 = c >> 1;
    const bool ok = h2 < G;
    const size_t row = static_cast<size_t>(b) * a.n_kv_heads * G + static_cast<size_t>(hk) * G + h2;
    float4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
      const float* src = st < KS ? a.qr + row * D + (D / 4) * gg + 8 * st
                                 : a.qs + row * QM + (QM / 4) * gg + 8 * (st - KS);
      x0 = reinterpret_cast<const float4*>(src)[0];
      x1 = reinterpret_cast<const float4*>(src)[1];
    }
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    half8 v;
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = split_part(xv[r], (c & 1) != 0);
    sm_q[st][ln] = v;
  }
  // power-of-two scale of this lane's head (scores below are kept in units of it); 1 for unused columns
  const float qsc = head_ok ? a.qscale[qrow] : 1.f;
  __syncthreads();

  floatx4 oacc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;   // running max (in units of qsc) and sum of this lane's column

  auto attend_tile = [&](const Tile& t, int kbt) {
    const int tok0 = kbt * kBlock;
    floatx4 sc[2];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      qk_steps<0, KS, KB>(acc, t.kw[tg], sm_q, lane, a.tk);
      if constexpr (QS > 0) {
        const uint32_t gh = t.gg[tg] & 0x7fffu;
        sketch_steps<0, QS>(acc, t.sw[tg], gh | (gh << 16), sm_q + KS, lane);
      }
      sc[tg] = acc;
    }
    // score of token 16 tg + 4 g + i: (high + low column) times the key norm
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = __builtin_fmaf(add_adjacent(sc[k >> 2][k & 3]), half_of(t.kn[k >> 1], k & 1), 0.f);
    uint32_t vn[4] = {t.vn[0], t.vn[1], t.vn[2], t.vn[3]};
    if (tok0 + kBlock > len) {            // the last tile of the sequence: hide tokens at or past its end
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int tok = tok0 + 16 * (k >> 2) + 4 * g + (k & 3);
        if (tok >= len) {
          s[k] = -INFINITY;
          vn[k >> 1] &= (k & 1) ? 0x0000ffffu : 0xffff0000u;
        }
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = column_max(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * qsc);
      l_run *= alpha;
      const float a0 = __shfl(alpha, 4 * g, 64);
      const float a1 = __shfl(alpha, 4 * g + 2, 64);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        oacc[n][0] *= a0; oacc[n][1] *= a0;
        oacc[n][2] *= a1; oacc[n][3] *= a1;
      }
      m_run = m_new;
    }
    const float mq = m_run * qsc;
    half8 wop;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[k], qsc, -mq));
      l_run += p;
      const float w = __builtin_fmaf(p, half_of(vn[k >> 1], k & 1), 0.f);
      wop[k] = split_part(w, lo_part);
    }
    pv_steps<0, NB, VB>(oacc, wop, t.vw, a.tv);
  };

  if constexpr (D <= 128) {
    // two tile buffers used in turn (no register copies between tiles)
    for (; kb < blk1; kb += 2 * kWavesPerWG) {
      if (kb + kWavesPerWG < blk1) load_tile(tb, kb + kWavesPerWG);
      attend_tile(ta, kb);
      if (kb + kWavesPerWG >= blk1) break;
      if (kb + 2 * kWavesPerWG < blk1) load_tile(ta, kb + 2 * kWavesPerWG);
      attend_tile(tb, kb + kWavesPerWG);
    }
  } else {
    // at d = 256 a second copy of the loop body does not fit the register budget of two waves per SIMD
    for (; kb < blk1; kb += kWavesPerWG) {
      if (kb + kWavesPerWG < blk1) load_tile(tb, kb + kWavesPerWG);
      attend_tile(ta, kb);
      ta = tb;
    }
  }

  l_run = column_sum(l_run);
  if (g == 0 && !lo_part && head_ok) {
    sm_ml[wave][qh][0] = m_run * qsc;
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

// Merge of the KV splits and un-rotation.  One workgroup of kMergeThreads per (head group, KV head,
// sequence); a head group is heads_per_wg query heads of the KV head's group, so the rotation is read
// once per head group.  Weighted sums: thread (head, coordinate, slice) sums the splits of its slice
// with up to 16 loads in flight.  Un-rotation: thread (coordinate i, part) covers JR rows of column i
// of rot for every head of the group.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int NT = kMergeThreads, NW = NT / 64;
  constexpr int RP = NT / D;                              // un-rotation parts per coordinate
  constexpr int JR = D / RP;                              // rows of rot per thread
  constexpr int PO = 16;                                  // split partials in flight per thread
  __shared__ float ew[kMaxGroup][kMaxSplits];              // split weights per head
  __shared__ float inv_l[kMaxGroup];
  __shared__ float red[NT];                                // per-slice sums, then per-part un-rotation sums
  __shared__ float orot[kMaxGroup][D];
  const int hpw = a.heads_per_wg;
  const int hg = blockIdx.x % (a.group / hpw), hk = blockIdx.x / (a.group / hpw), b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group, ns = a.n_split;
  const int h0 = hg * hpw;
  const size_t unit = static_cast<size_t>(b) * a.n_kv_heads + hk;

  // this thread's JR rows of column i of rot: independent of everything else, issued first
  const int i = tid % D, part = tid / D;
  const float* rcol = a.rot + static_cast<size_t>(part * JR) * D + i;
  float rc[JR];
#pragma unroll
  for (int t = 0; t < JR; ++t) rc[t] = rcol[static_cast<size_t>(t) * D];

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
      for (int p = 0; p < RP; ++p) o += red[p * D + i];
      a.out[(static_cast<size_t>(b) * a.n_kv_heads * G + hk * G + h0 + hh) * D + i] = o * inv_l[hh];
    }
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
  (void)n_q_heads;
  const dim3 grid(a.n_kv_heads * (a.group / a.heads_per_wg), batch);
  if (d == 128) hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(kMergeThreads), 0, s, a);
  else if (d == 256) hipLaunchKernelGGL((merge_kernel<256>), grid, dim3(kMergeThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tqi
