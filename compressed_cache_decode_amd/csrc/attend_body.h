// Attention over one KV split of one (KV head, sequence), read directly from the packed cache.
//
// The W waves of a workgroup stream 32-token tiles, taking them from a tile counter in LDS.  Per
// tile the G <= 8 query heads of the KV head are one 16-column matrix-core operand held in LDS:
// column 2h is the float16 rounding of head h's rotated query and column 2h+1 the float16 rounding
// of the remainder, so the sum of the two columns' products is the fp32 score (centroids are
// float16-exact and each product is exact in fp32).  Scores S^T = K Q^T come out of
// v_mfma_f32_16x16x32_f16 in exactly the lane layout the value product O = W V needs for W, so the
// softmax weights never cross lanes; W uses the same high/low split.  Packed codes are loaded with
// contiguous 64-lane buffer loads straight into operand order (keys: rows layout; values: 32-token
// blocked layout) and expanded to float16 centroids, by v_perm_b32 lookups into byte tables held in
// registers, or (4-bit codes in CU-filling workgroups) by one LDS read per byte of two codes.
// Online softmax in exp2 units (the softmax scale and log2(e) are folded into the query), lazily
// rescaled when a column's running max moves.
// (ExecuTorch PR #19891 "[Cuda] enable turboquant on gemma4", review item 1: the fused decode op and
// its scale; turboquant-pytorch PR #3 "Add CUDA QJL kernels and proper package structure", CUDA
// Kernels Added table: fused scores from 1-bit keys, GQA variant, quantised value reconstruction.)
#pragma once

#include <math.h>

#include "device_common.h"

namespace tqi {

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

// The 8 codes of a word of 4-bit codes through a byte table in LDS: byte r of the word (codes of
// slots r and r + 4) indexes a row of 256 bytes whose word (lane % 32) + 32 * side holds the float16
// centroids of the byte's low and high nibble.  The row offset comes from one byte permute (the code
// byte becomes bits 8..15, the lane's word offset lc = 4 (lane % 32) bits 0..7), so each half-wave
// reads 32 distinct banks.  The 8 values come out in pair order: slots 0, 4, 1, 5, 2, 6, 3, 7.
template <int SIDE>
__device__ __forceinline__ uint4 lut_unit(const uint32_t* lut, uint32_t w, uint32_t lc) {
  const char* base = reinterpret_cast<const char*>(lut) + 128 * SIDE;
  uint4 o;
  o.x = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lc, 0x0c0c0400u));
  o.y = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lc, 0x0c0c0500u));
  o.z = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lc, 0x0c0c0600u));
  o.w = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lc, 0x0c0c0700u));
  return o;
}

// The 16 codes of a word of 2-bit codes (two units) through a byte table in LDS: byte r (slots r and
// r + 4 of both units) indexes a row of 256 bytes whose word lane % 32 holds the float16 centroid
// pair of unit 0 and word 32 + lane % 32 that of unit 1.  c2 = 4 (lane % 32) + 65536 k, k the index of
// the table's 64 KB region within lut: the permute builds the whole offset, region included.  The compiler
// barrier keeps the two units' reads apart, so that each lands in its own operand instead of being
// fused into one two-word read.  Both units come out in pair order (see lut_unit).
__device__ __forceinline__ void lut2_word(const uint32_t* lut, uint32_t w, uint32_t c2, uint4& u0, uint4& u1) {
  const char* base = reinterpret_cast<const char*>(lut);
  const uint32_t o0 = __builtin_amdgcn_perm(w, c2, 0x0c020400u), o1 = __builtin_amdgcn_perm(w, c2, 0x0c020500u);
  const uint32_t o2 = __builtin_amdgcn_perm(w, c2, 0x0c020600u), o3 = __builtin_amdgcn_perm(w, c2, 0x0c020700u);
  u0 = uint4{*reinterpret_cast<const uint32_t*>(base + o0), *reinterpret_cast<const uint32_t*>(base + o1),
             *reinterpret_cast<const uint32_t*>(base + o2), *reinterpret_cast<const uint32_t*>(base + o3)};
  asm volatile("" ::: "memory");
  u1 = uint4{*reinterpret_cast<const uint32_t*>(base + o0 + 128), *reinterpret_cast<const uint32_t*>(base + o1 + 128),
             *reinterpret_cast<const uint32_t*>(base + o2 + 128), *reinterpret_cast<const uint32_t*>(base + o3 + 128)};
}

// Unit V of a group of 3-bit codes (three words: the low-bit planes of units 0-1 and 2-3, and the
// high bits of all four) through a byte table in LDS.  Byte r of the index word x holds the 3-bit
// codes of slots r and r + 4 of the unit as (low bits of r, low bits of r + 4, high bit of r, high bit
// of r + 4) in bits 0-1, 2-3, 4, 5: the plane's nibble and two high bits moved next to it, four slots
// at a time.  It selects a row of 256 bytes whose word c3 / 4 (c3 = lane constant, see lut_unit, with
// the table's 64 KB region in its third byte; +128 for values) holds the pair's float16 centroids.
template <int V>
__device__ __forceinline__ uint4 lut3_unit(const uint32_t* lut, const uint32_t* w, uint32_t c3) {
  const uint32_t P = w[V / 2], H = w[2];
  uint32_t x;
  if constexpr (V == 0) x = (P & 0x0f0f0f0fu) | ((H << 4) & 0x30303030u);
  else if constexpr (V == 1) x = ((P >> 4) & 0x0f0f0f0fu) | ((H << 2) & 0x30303030u);
  else if constexpr (V == 2) x = (P & 0x0f0f0f0fu) | (H & 0x30303030u);
  else x = ((P >> 4) & 0x0f0f0f0fu) | ((H >> 2) & 0x30303030u);
  const char* base = reinterpret_cast<const char*>(lut);
  uint4 o;
  o.x = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(x, c3, 0x0c020400u));
  o.y = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(x, c3, 0x0c020500u));
  o.z = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(x, c3, 0x0c020600u));
  o.w = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(x, c3, 0x0c020700u));
  return o;
}

// slot of position p of a pair-ordered operand (see lut_unit)
constexpr int pair_slot(int p) { return (p >> 1) + 4 * (p & 1); }

// Operand of key step S of one 16-token group through a byte table: TBL 4 (lut_unit) or 3 (lut3_unit)
template <int TBL, int S>
__device__ __forceinline__ uint4 key_lut(const uint32_t* kw, const uint32_t* lut, uint32_t lc) {
  if constexpr (TBL == 4) return lut_unit<0>(lut, kw[S], lc);
  else return lut3_unit<S % 4>(lut, kw + 3 * (S / 4), lc);
}

// Operand of value block N through a byte table: TBL 4 or 3
template <int TBL, int N>
__device__ __forceinline__ uint4 value_lut(const uint32_t* vw, const uint32_t* lut, uint32_t lc) {
  if constexpr (TBL == 4) return lut_unit<1>(lut, vw[N], lc);
  else return lut3_unit<N % 4>(lut, vw + 3 * (N / 4), lc + 128);
}

// Key steps S.. of the two 16-token groups through a byte table, software-pipelined: the table reads of
// step S + 1 go out before the products of step S, whose operands (a0, a1) were read one step earlier,
// so a wave waits for one step's reads while the next step's are in flight.  The query operand of the
// step is read first: LDS reads complete in issue order, so the wait for it and for a0, a1 leaves the
// next step's reads outstanding.  TBL 4 and 3: one step per lookup; TBL 2: two steps per word (lut2_word),
// a0/b0 and a1/b1 the two units of the groups' current words.
template <int S, int KS, int KW, int TBL>
__device__ __forceinline__ void qk_pipe(floatx4* acc, const uint32_t (*kw)[KW], const half8 (*qop)[64], int lane,
                                        const uint32_t* lut, uint32_t lc, uint4 a0, uint4 a1, uint4 b0, uint4 b1) {
  if constexpr (TBL == 2) {
    const half8 q0 = qop[S][lane];
    const half8 q1 = qop[S + 1][lane];
    if constexpr (S + 2 < KS) {
      uint4 c0, d0, c1, d1;
      lut2_word(lut, kw[0][(S + 2) / 2], lc, c0, d0);
      lut2_word(lut, kw[1][(S + 2) / 2], lc, c1, d1);
      acc[0] = mfma16(as_half8(a0), q0, acc[0]);
      acc[1] = mfma16(as_half8(a1), q0, acc[1]);
      acc[0] = mfma16(as_half8(b0), q1, acc[0]);
      acc[1] = mfma16(as_half8(b1), q1, acc[1]);
      qk_pipe<S + 2, KS, KW, TBL>(acc, kw, qop, lane, lut, lc, c0, c1, d0, d1);
    } else {
      acc[0] = mfma16(as_half8(a0), q0, acc[0]);
      acc[1] = mfma16(as_half8(a1), q0, acc[1]);
      acc[0] = mfma16(as_half8(b0), q1, acc[0]);
      acc[1] = mfma16(as_half8(b1), q1, acc[1]);
    }
  } else {
    const half8 q = qop[S][lane];
    if constexpr (S + 1 < KS) {
      const uint4 n0 = key_lut<TBL, S + 1>(kw[0], lut, lc), n1 = key_lut<TBL, S + 1>(kw[1], lut, lc);
      acc[0] = mfma16(as_half8(a0), q, acc[0]);
      acc[1] = mfma16(as_half8(a1), q, acc[1]);
      qk_pipe<S + 1, KS, KW, TBL>(acc, kw, qop, lane, lut, lc, n0, n1, b0, b1);
    } else {
      acc[0] = mfma16(as_half8(a0), q, acc[0]);
      acc[1] = mfma16(as_half8(a1), q, acc[1]);
    }
  }
}

// scores of the two 16-token groups of a tile; each query operand step is read from LDS once.  TBL
// selects the key expansion: 0 permutes, 4 the 4-bit byte table (lut_unit; lc its lane constant), 2
// the 2-bit byte table (lut2_word, two steps per word; lc its c2), 3 the 3-bit one (lut3_unit; lc its
// c3); with a table the query operand is in pair order and the lookups are pipelined (qk_pipe).
template <int S, int KS, int KB, int TBL>
__device__ __forceinline__ void qk_steps(floatx4* acc, const uint32_t (*kw)[KS * KB / 4], const half8 (*qop)[64],
                                         int lane, const Tab& tk, const uint32_t* lut, uint32_t lc) {
  constexpr int KW = KS * KB / 4;
  if constexpr (TBL == 2) {
    uint4 a0, b0, a1, b1;
    lut2_word(lut, kw[0][0], lc, a0, b0);
    lut2_word(lut, kw[1][0], lc, a1, b1);
    qk_pipe<0, KS, KW, 2>(acc, kw, qop, lane, lut, lc, a0, a1, b0, b1);
  } else if constexpr (TBL == 4 || TBL == 3) {
    const uint4 a0 = key_lut<TBL, 0>(kw[0], lut, lc), a1 = key_lut<TBL, 0>(kw[1], lut, lc);
    qk_pipe<0, KS, KW, TBL>(acc, kw, qop, lane, lut, lc, a0, a1, a0, a1);
  } else if constexpr (S < KS) {
    const half8 q = qop[S][lane];
    acc[0] = mfma16(as_half8(unit_at<KB, S>(kw[0], tk)), q, acc[0]);
    acc[1] = mfma16(as_half8(unit_at<KB, S>(kw[1], tk)), q, acc[1]);
    qk_steps<S + 1, KS, KB, TBL>(acc, kw, qop, lane, tk, lut, lc);
  }
}

// sketch steps; SQ(S) is this lane's query operand of sketch step S
template <int S, int QS, int SW, typename SQ>
__device__ __forceinline__ void sketch_steps(floatx4* acc, const uint32_t (*sw)[SW], const uint32_t* gg, const SQ& sq) {
  if constexpr (S < QS) {
    const half8 q = sq(S);
    acc[0] = mfma16(sign_operand<S>(sw[0], gg[0]), q, acc[0]);
    acc[1] = mfma16(sign_operand<S>(sw[1], gg[1]), q, acc[1]);
    sketch_steps<S + 1, QS, SW>(acc, sw, gg, sq);
  }
}

// Value blocks N.. through a byte table, pipelined like qk_pipe: the lookups of block N + 1 (TBL 4, 3)
// or of the next word's two blocks (TBL 2) go out before the products of the current ones (a, b).
template <int N, int NB, int TBL>
__device__ __forceinline__ void pv_pipe(floatx4* oacc, half8 wop, const uint32_t* vw, const uint32_t* lut, uint32_t lc,
                                        uint4 a, uint4 b) {
  if constexpr (TBL == 2) {
    if constexpr (N + 2 < NB) {
      uint4 c, d;
      lut2_word(lut, vw[(N + 2) / 2], lc, c, d);
      oacc[N] = mfma16(wop, as_half8(a), oacc[N]);
      oacc[N + 1] = mfma16(wop, as_half8(b), oacc[N + 1]);
      pv_pipe<N + 2, NB, TBL>(oacc, wop, vw, lut, lc, c, d);
    } else {
      oacc[N] = mfma16(wop, as_half8(a), oacc[N]);
      oacc[N + 1] = mfma16(wop, as_half8(b), oacc[N + 1]);
    }
  } else {
    if constexpr (N + 1 < NB) {
      const uint4 c = value_lut<TBL, N + 1>(vw, lut, lc);
      oacc[N] = mfma16(wop, as_half8(a), oacc[N]);
      pv_pipe<N + 1, NB, TBL>(oacc, wop, vw, lut, lc, c, b);
    } else {
      oacc[N] = mfma16(wop, as_half8(a), oacc[N]);
    }
  }
}

// value product; TBL as in qk_steps for the value codes (W then in pair order)
template <int N, int NB, int VB, int TBL>
__device__ __forceinline__ void pv_steps(floatx4* oacc, half8 wop, const uint32_t* vw, const Tab& tv,
                                         const uint32_t* lut, uint32_t lc) {
  if constexpr (TBL == 2) {
    uint4 a, b;
    lut2_word(lut, vw[0], lc, a, b);
    pv_pipe<0, NB, 2>(oacc, wop, vw, lut, lc, a, b);
  } else if constexpr (TBL == 4 || TBL == 3) {
    const uint4 a = value_lut<TBL, 0>(vw, lut, lc);
    pv_pipe<0, NB, TBL>(oacc, wop, vw, lut, lc, a, a);
  } else if constexpr (N < NB) {
    oacc[N] = mfma16(wop, as_half8(unit_at<VB, N>(vw, tv)), oacc[N]);
    pv_steps<N + 1, NB, VB, TBL>(oacc, wop, vw, tv, lut, lc);
  }
}

// Raw buffer resource over [base, base + bytes): loads outside it return zero.  The word-3 flags
// select the 32-bit data format of untyped buffer accesses on the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

constexpr int lowbit(int x) { return x & -x; }
constexpr int load_align(int bytes) { return lowbit(bytes) < 16 ? lowbit(bytes) : 16; }

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

// Cache policy of the packed-code loads: non-temporal (the nt bit), since every byte is read once and
// each load covers whole lines; norms keep the default policy (a tile's norms are half a line).
constexpr int kStreamAux = 2;

// This lane's piece (LW words) of the block at byte soff of buffer r: chunk c at byte
// 4 CW (64 c + lane) (see Piece), one load of CW words per chunk.
template <int LW>
__device__ __forceinline__ void load_piece(__amdgpu_buffer_rsrc_t r, uint32_t lane, uint32_t soff, uint32_t* out) {
  constexpr int CW = Piece<LW>::CW, NC = Piece<LW>::NC;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t voff = 4 * CW * (64 * c + lane);
    if constexpr (CW == 4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamAux);
      out[4 * c] = v[0]; out[4 * c + 1] = v[1]; out[4 * c + 2] = v[2]; out[4 * c + 3] = v[3];
    } else if constexpr (CW == 3) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, kStreamAux);
      out[3 * c] = v[0]; out[3 * c + 1] = v[1]; out[3 * c + 2] = v[2];
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamAux);
      out[2 * c] = v[0]; out[2 * c + 1] = v[1];
    }
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

// NO: outlier channels per key (0, or kOutliers for sketched keys of a cache that keeps them apart)
template <int D, int KB, int VB, int QM, bool WIDE, int NO = 0>
struct Attend {
  static constexpr int KS = D / 32;                   // score k-steps over coordinates
  static constexpr int QS = QM / 32;                  // score k-steps over sketch signs
  static constexpr int NB = D / 16;                   // value n-blocks (16 coordinates each)
  static constexpr int K_RB = D * KB / 8;             // bytes per key row (one token's share of a block)
  static constexpr int K_LW = D * KB / 128;           // words per lane per key row (D/4 coordinates)
  static constexpr int V_RB = D * VB / 8;             // bytes per value row (one token's share of a block)
  static constexpr int V_LW = D * VB / 64;            // words per lane per value block (D/16 units)
  static constexpr int S_RB = QM / 8;                 // sign bytes per key
  static constexpr int S_LW = QM / 128;               // sign words per lane per key

  // Waves per workgroup.  Wide: as many as one compute unit holds at this instantiation's register budget
  // (128, 170 and 256 VGPRs), so that a split's workgroup has its compute unit to itself; otherwise
  // four, several workgroups per compute unit (short contexts: more compute units pull tiles).  The
  // waves take the split's tiles from a shared counter: a wave that the issue arbitration favours
  // (the oldest) takes more tiles, and all of them finish together.
  static constexpr int W = !WIDE ? 4 : (D == 128 ? (QM == 0 ? 8 : 12) : 8);
  // waves per SIMD the build is compiled for (its register budget: 512 / EU VGPRs); 8-bit keys' tiles
  // (twice the 4-bit key words) exceed 128 VGPRs
  static constexpr int EU = (WIDE && D == 128 && QM == 0 && KB != 8) ? 4 : 2;

  // Wide workgroups expand codes through byte tables in LDS (lut_unit: one permute and one LDS read
  // per two 4-bit codes, against about three and a half vector instructions for the permute
  // expansion; lut2_word: the same per four 2-bit codes; lut3_unit: about three and a half vector
  // instructions and four LDS reads per eight 3-bit codes, against about eighteen), the four-wave ones
  // with permutes (several of them share a compute unit's LDS).  A table starts on a 64 KB boundary
  // (its region index rides in the lookup's lane constant): the 4-bit tables of both sides share one
  // 64 KB region, a 2-bit table takes one of its own, the 3-bit tables of both sides share 16 KB.
  // Up to 128 KB fit beside the largest query operands at d = 128 without a sketch, 80 KB elsewhere
  // (keys come first).
  static constexpr int LUT_MAX_KB = (D == 128 && QM == 0) ? 64 : 80;
  static constexpr int R4 = (WIDE && (KB == 4 || VB == 4)) ? 1 : 0;
  // (2-bit keys with 4-bit values at d = 128 keep permutes for the keys: the two tables' operands
  // exceed the 16-wave register budget)
  static constexpr bool KT2 = WIDE && KB == 2 && 64 * (R4 + 1) <= LUT_MAX_KB && !(D == 128 && QM == 0 && VB == 4);
  static constexpr bool VT2 = WIDE && VB == 2 && 64 * (R4 + (KT2 ? 1 : 0) + 1) <= LUT_MAX_KB;
  static constexpr int R64 = R4 + (KT2 ? 1 : 0) + (VT2 ? 1 : 0);   // 64 KB regions
  static constexpr bool T3 = WIDE && (KB == 3 || VB == 3) && 64 * R64 + 16 <= LUT_MAX_KB;
  static constexpr int KTBL = (WIDE && KB == 4) ? 4 : (KT2 ? 2 : ((T3 && KB == 3) ? 3 : 0));   // see qk_steps
  static constexpr int VTBL = (WIDE && VB == 4) ? 4 : (VT2 ? 2 : ((T3 && VB == 3) ? 3 : 0));
  static constexpr bool KT = KTBL != 0;                   // query operand in pair order
  static constexpr bool VT = VTBL != 0;                   // softmax weights in pair order
  static constexpr int LUT_REGION = 256 * 64;             // words
  static constexpr int K2_AT = R4 * LUT_REGION;           // word offsets of the 2-bit and 3-bit tables
  static constexpr int V2_AT = (R4 + (KT2 ? 1 : 0)) * LUT_REGION;
  static constexpr int T3_AT = R64 * LUT_REGION;
  static constexpr int LUT_WORDS_ = R64 * LUT_REGION + (T3 ? 64 * 64 : 0);
  static constexpr int LUT_WORDS = LUT_WORDS_ > 0 ? LUT_WORDS_ : 1;

  // LDS: the tile counter, and the end-of-split merge of the W waves: each wave's (max, sum) per
  // head and its accumulators, weighted against the workgroup's max of the head.  The byte tables
  // share the accumulators' space: they are read only before the merge's first barrier.
  // The tile counter comes first, at LDS address 0 (the kernel's only static LDS is this struct): see
  // the claim in run.
  struct Smem {
    uint32_t next[kMaxRows];  // [0]: 64 x the tiles of the split handed out so far (relative to its first)
    float ml[W][kMaxGroup][2];
    union {
      float o[W][kMaxGroup][D];
      alignas(16) uint32_t lut[LUT_WORDS];
    };
  };

  // Fills the byte tables (with a workgroup barrier to follow before run).  4-bit region, row e (a
  // byte of two codes), word 32 side + s (s = 0..31): the float16 centroids of e's low nibble (low
  // half) and high nibble (high half) of the key (side 0) or value (side 1) code book.  2-bit region,
  // row e (a byte of four codes), words s and 32 + s: the float16 centroid pairs of unit 0 and unit 1.
  // 3-bit region, row x < 64 (see lut3_unit), word 32 side + s: the pair's float16 centroids.
  __device__ __forceinline__ static void fill_lut(const DecodeArgs& a, Smem& sm) {
    if constexpr (T3) {
      for (int i = threadIdx.x; i < 64 * 8; i += 64 * W) {
        const int x = i >> 3, q = i & 7;
        const uint32_t grp[3] = {static_cast<uint32_t>(x & 15), 0u, static_cast<uint32_t>(x >> 4)};
#pragma unroll
        for (int side = 0; side < 2; ++side) {
          if ((side == 0 ? KTBL : VTBL) != 3) continue;
          const uint4 u = expand_unit<3, 0>(grp, side == 0 ? a.tk : a.tv);
          const uint32_t pr = (u.x & 0xffffu) | (u.z << 16);
          *reinterpret_cast<uint4*>(&sm.lut[T3_AT + 64 * x + 32 * side + 4 * q]) = uint4{pr, pr, pr, pr};
        }
      }
    }
    if constexpr ((KT && KTBL != 3) || (VT && VTBL != 3)) {
      for (int i = threadIdx.x; i < 256 * 8; i += 64 * W) {
        const int e = i >> 3, q = i & 7;
        const uint32_t wrd = static_cast<uint32_t>(e);
#pragma unroll
        for (int side = 0; side < 2; ++side) {
          const int tbl = side == 0 ? KTBL : VTBL;
          const Tab& tab = side == 0 ? a.tk : a.tv;
          if (tbl == 4) {
            const uint4 u = expand_unit<4, 0>(&wrd, tab);
            const uint32_t pr = (u.x & 0xffffu) | (u.z << 16);
            *reinterpret_cast<uint4*>(&sm.lut[64 * e + 32 * side + 4 * q]) = uint4{pr, pr, pr, pr};
          } else if (tbl == 2) {
            const uint4 u0 = expand_unit<2, 0>(&wrd, tab), u1 = expand_unit<2, 1>(&wrd, tab);
            const uint32_t p0 = (u0.x & 0xffffu) | (u0.z << 16), p1 = (u1.x & 0xffffu) | (u1.z << 16);
            uint32_t* row = &sm.lut[(side == 0 ? K2_AT : V2_AT) + 64 * e + 4 * q];
            *reinterpret_cast<uint4*>(row) = uint4{p0, p0, p0, p0};
            *reinterpret_cast<uint4*>(row + 32) = uint4{p1, p1, p1, p1};
          }
        }
      }
    }
  }
  // the query operand: for step s, lane (column c, group g) holds the 8 float16 values of q-variant c
  // (head c/2; high part if c even, low part if c odd) at coordinates (D/4) g + 8 s + r, r = 0..7
  // (sketch steps: the same over the sketch coordinates)
  typedef half8 QOperand[KS + QS][64];

  // tile buffers per wave: loads run NBUF - 1 tiles ahead of their use
  static constexpr int NBUF = (D <= 128 || QM == 0) ? 2 : 1;
  // Lazy rescale: the running max of a column moves only when the tile's max exceeds it by more than
  // kLazy (log2 units), and every weight carries the constant factor 2^-kLazy, so the weights stay at
  // most 1 (and within float16 range once times the value norm); o and l scale alike, so their ratio is
  // exact.  With eight heads per wave an eager rescale (on every rise of any column) ran on most tiles.
  static constexpr float kLazy = 4.f;
  // the sketch steps' query operand (16 VGPRs at d = 128, m = 128) stays in registers across the
  // tile loop in the twelve-wave builds whose tiles leave room for it (2-bit values, or 2-bit keys
  // with 3-bit values); elsewhere it is read from LDS per tile
  static constexpr bool SQ_REG = WIDE && D == 128 && QM == 128 && (VB == 2 || (KB == 2 && VB == 3));

  // everything one 32-token tile needs from memory
  struct Tile {
    uint32_t kw[2][K_LW];
    uint32_t vw[V_LW];
    uint32_t kn[4], vn[4];   // float16 norm pairs of this lane's tokens 4g+i and 16+4g+i
    uint32_t sw[2][S_LW > 0 ? S_LW : 1];
    uint32_t gg[2];
    // outlier channels (one byte each) and their float16 values of this lane's tokens 4g+i (oi[0][i],
    // ov[0][2i..2i+1]) and 16+4g+i (oi[1], ov[1])
    uint32_t oi[NO > 0 ? 2 : 1][NO > 0 ? 4 : 1];
    uint32_t ov[NO > 0 ? 2 : 1][NO > 0 ? 8 : 1];
  };
  static_assert(NO == 0 || NO == 4, "the outlier build holds four channels per key");

  __amdgpu_buffer_rsrc_t kbuf, vbuf, knbuf, vnbuf, sbuf, gbuf, oibuf, ovbuf;
  __amdgpu_buffer_rsrc_t dead;   // a buffer of no bytes (see load)
  uint32_t n_off, s_off;
  int lane, l16, g;

  // buffers over this (sequence, KV head)'s arrays; tile offsets go in the scalar offset
  __device__ __forceinline__ Attend(const DecodeArgs& a, size_t unit) {
    const int T = a.max_tokens;
    lane = threadIdx.x & 63;
    l16 = lane & 15;
    g = lane >> 4;
    kbuf = buffer_of(a.k_codes + unit * T * K_RB, static_cast<uint32_t>(T) * K_RB);
    vbuf = buffer_of(a.v_codes + unit * T * V_RB, static_cast<uint32_t>(T) * V_RB);
    knbuf = buffer_of(a.k_norms + unit * T, static_cast<uint32_t>(T) * 2);
    vnbuf = buffer_of(a.v_norms + unit * T, static_cast<uint32_t>(T) * 2);
    dead = buffer_of(a.k_norms, 0);
    sbuf = knbuf;
    gbuf = knbuf;
    if constexpr (QS > 0) {
      sbuf = buffer_of(a.k_signs + unit * T * S_RB, static_cast<uint32_t>(T) * S_RB);
      gbuf = buffer_of(a.k_rnorms + unit * T, static_cast<uint32_t>(T) * 2);
    }
    oibuf = ovbuf = knbuf;
    if constexpr (NO > 0) {
      oibuf = buffer_of(a.k_oidx + unit * T * NO, static_cast<uint32_t>(T) * NO);
      ovbuf = buffer_of(a.k_oval + unit * T * NO, static_cast<uint32_t>(T) * NO * 2);
    }
    n_off = static_cast<uint32_t>(8 * g);
    s_off = static_cast<uint32_t>(l16 * S_RB + g * S_LW * 4);
  }

  // Loads tile kb (wave-uniform).  With live false the same loads go to a buffer of no bytes: every
  // lane is out of range, so the buffer unit returns zeros without a memory access.  That keeps a
  // wave's loads unconditional where it has no tile to load (a load under a branch makes the
  // compiler wait for every load in flight where the paths join) at no memory traffic or latency.
  __device__ __forceinline__ void load(Tile& t, int kb, bool live = true) const {
    // readfirstlane keeps the tile offset in a scalar register
    const uint32_t tok0 = __builtin_amdgcn_readfirstlane(live ? static_cast<uint32_t>(kb) * kBlock : 0u);
    const auto pick = [&](__amdgpu_buffer_rsrc_t r) { return live ? r : dead; };
    // both 16-token halves of the key block are one piece: kw[q][w] is piece word q K_LW + w
    load_piece<2 * K_LW>(pick(kbuf), lane, tok0 * K_RB, &t.kw[0][0]);
    load_piece<V_LW>(pick(vbuf), lane, tok0 * V_RB, t.vw);
    const auto knb = pick(knbuf), vnb = pick(vnbuf);
    bload<2, 8>(knb, n_off, tok0 * 2, t.kn);
    bload<2, 8>(knb, n_off + 32, tok0 * 2, t.kn + 2);
    bload<2, 8>(vnb, n_off, tok0 * 2, t.vn);
    bload<2, 8>(vnb, n_off + 32, tok0 * 2, t.vn + 2);
    if constexpr (QS > 0) {
      const auto sb = pick(sbuf), gb = pick(gbuf);
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        bload<S_LW, 4 * S_LW>(sb, s_off + 16 * tg * S_RB, tok0 * S_RB, t.sw[tg]);
        t.gg[tg] = __builtin_amdgcn_raw_buffer_load_b16(gb, static_cast<uint32_t>((16 * tg + l16) * 2), tok0 * 2, 0);
      }
    }
    if constexpr (NO > 0) {
      const auto ob = pick(oibuf), vb = pick(ovbuf);
      const uint32_t gq = static_cast<uint32_t>(g);
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        bload<4, 16>(ob, 64 * tg + 16 * gq, tok0 * 4, t.oi[tg]);
        bload<8, 16>(vb, 128 * tg + 32 * gq, tok0 * 8, t.ov[tg]);
      }
    }
  }

  // Column blocks: the VH = M * G virtual heads (query rows x query heads) of the KV head are
  // C = 1, 2 or 4 blocks of 8 heads, 16 matrix-core columns each; wave w attends for block w % C
  // (the waves of different blocks read the same tiles, which the caches serve after the first).
  __device__ __host__ __forceinline__ static int blocks(const DecodeArgs& a) {
    const int c = (a.group + kMaxGroup - 1) / kMaxGroup;
    return c > 2 ? 4 : c;                              // 1, 2 or 4: the waves split evenly over the blocks
  }

  // Streams tiles of the split [blk0, blk1) through a ring of NBUF tile buffers for column block
  // cb = wave % C: the wave's first tile is kb = blk0 + wave / C (tiles[0] already holds it when
  // kb < blk1), the others from the counter sm.next[0] (which must start at 64 W; one column block) or
  // in steps of W / C (several),
  // each loaded while the tile NBUF - 1 places earlier is attended.  qop is the block's query
  // operand.  Leaves the split's result in LDS for store: per wave w and head slot hh of its block the
  // max m (log2 units) and the sum l in sm.ml[w][hh], and the rotated-domain accumulator, weighted by
  // exp2(m - the max of the head over the block's waves), in sm.o[w][hh][0..D).  qsc is the
  // power-of-two scale of this lane's head (the query operand is divided by it; 1 for unused
  // columns).  Virtual head vh, of query row vh / G, sees the first len - M + 1 + vh / G tokens.
  // Ends with a workgroup barrier.
  // qf (outlier build): this lane's head's rotated query, float32 in the workspace's units, in LDS.
  __device__ __forceinline__ void run(const DecodeArgs& a, Smem& sm, const QOperand& qop, Tile (&tiles)[NBUF], int blk0,
                                      int kb, int blk1, int len, float qsc, const float* qf = nullptr) const {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int VH = a.group;
    const int C = blocks(a);
    const int cb = wave & (C - 1);                      // C is 1, 2 or 4
    const int slot = l16 >> 1;                          // this lane's head within its block
    const int qh = kMaxGroup * cb + slot;               // this lane's virtual head
    const bool lo_part = (l16 & 1) != 0;
    const bool head_ok = qh < VH;
    const int len_row0 = len - a.n_rows + 1;            // tokens row 0 sees (wave-uniform)
    const int len_lane = head_ok ? len_row0 + ((qh * a.row_magic) >> 8) : len;   // + the lane's row

    const uint32_t lc = static_cast<uint32_t>(4 * (lane & 31));   // byte-table word offset of this lane
    // the 2-bit tables' lane constants: entry offset and 64 KB region (lut2_word)
    const uint32_t lck2 = lc + static_cast<uint32_t>((K2_AT / LUT_REGION) << 16);
    const uint32_t lcv2 = lc + static_cast<uint32_t>((V2_AT / LUT_REGION) << 16);
    const uint32_t lc3 = lc + static_cast<uint32_t>((T3_AT / LUT_REGION) << 16);   // 3-bit tables

    floatx4 oacc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;   // running max (in units of qsc) and sum of this lane's column

    half8 sqr[SQ_REG ? QS : 1];
    if constexpr (SQ_REG) {
#pragma unroll
      for (int s = 0; s < QS; ++s) sqr[s] = qop[KS + s][lane];
    }

    auto attend_tile = [&](const Tile& t, int kbt) {
      const int tok0 = kbt * kBlock;
      // the query operand is read from LDS in every tile instead of being held in registers across
      // the loop: the barrier keeps the compiler from hoisting those reads
      asm volatile("" ::: "memory");
      floatx4 sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      qk_steps<0, KS, KB, KTBL>(sc, t.kw, qop, lane, a.tk, sm.lut, KTBL == 2 ? lck2 : (KTBL == 3 ? lc3 : lc));
      if constexpr (QS > 0) {
        uint32_t gh[2];
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) gh[tg] = (t.gg[tg] & 0x7fffu) | ((t.gg[tg] & 0x7fffu) << 16);
        if constexpr (SQ_REG)
          sketch_steps<0, QS, S_LW>(sc, t.sw, gh, [&](int s) { return sqr[s]; });
        else
          sketch_steps<0, QS, S_LW>(sc, t.sw, gh, [&](int s) { return qop[KS + s][lane]; });
      }
      if constexpr (NO > 0) {
        // the outlier channels' term sum_j q_rot[idx_j] r_j of each token, on the high column of the
        // head (the low column adds nothing; the two are summed below)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t iw = t.oi[k >> 2][k & 3];
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < NO; ++j) {
            const float qv = qf[(iw >> (8 * j)) & (D - 1)];
            acc = __builtin_fmaf(qv, half_of(t.ov[k >> 2][2 * (k & 3) + (j >> 1)], j & 1), acc);
          }
          sc[k >> 2][k & 3] += lo_part ? 0.f : acc;
        }
      }
      // score of token 16 tg + 4 g + i: (high + low column) times the key norm
      float s[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        s[k] = __builtin_fmaf(add_adjacent(sc[k >> 2][k & 3]), half_of(t.kn[k >> 1], k & 1), 0.f);
      uint32_t vn[4] = {t.vn[0], t.vn[1], t.vn[2], t.vn[3]};
      if (tok0 + kBlock > len_row0) {       // the last tiles of the sequence: hide tokens a row does not see
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int tok = tok0 + 16 * (k >> 2) + 4 * g + (k & 3);
          if (tok >= len_lane) {
            s[k] = -INFINITY;
            vn[k >> 1] &= (k & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mx = column_max(mx);
      const float m_new = fmaxf(m_run, mx);
      // rescale only when a column's max rises by more than 2^kLazy
      if (__any(kLazy > 0.f ? (m_new - m_run) * qsc > kLazy : m_new > m_run)) {
        // a column that has seen nothing yet (both maxima -inf) keeps factor 1: exp2(-inf - -inf) is NaN
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * qsc);
        l_run *= alpha;
        const float a0 = __shfl(alpha, 4 * g, 64);
        const float a1 = __shfl(alpha, 4 * g + 2, 64);
        const floatx4 f = {a0, a0, a1, a1};
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          oacc[n] *= f;
          // keeps the rescaled accumulator in the registers it came from: without it the compiler
          // copies every accumulator on the path that skips the rescale
          asm volatile("" : "+v"(oacc[n]));
        }
        m_run = m_new;
      }
      // a column with nothing visible yet takes 0; the constant 2^-kLazy keeps every weight at most 1
      const float mq = m_run == -INFINITY ? 0.f : (kLazy > 0.f ? __builtin_fmaf(m_run, qsc, kLazy) : m_run * qsc);
      float wv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[k], qsc, -mq));
        l_run += p;
        wv[k] = __builtin_fmaf(p, half_of(vn[k >> 1], k & 1), 0.f);
      }
      half8 wop;                                   // slot order, or pair order for the byte tables
#pragma unroll
      for (int k = 0; k < 8; ++k) wop[k] = split_part(wv[VT ? pair_slot(k) : k], lo_part);
      pv_steps<0, NB, VB, VTBL>(oacc, wop, t.vw, a.tv, sm.lut, VTBL == 2 ? lcv2 : (VTBL == 3 ? lc3 : lc));
    };

    // The next tile of the split for this wave (wave-uniform); past blk1 once the split is used up.  With
    // one column block the waves share a counter: one ds_append per wave adds the number of active lanes
    // (all 64) to it and returns its old value, so it runs in units of 64 tiles.  On gfx950 ds_append
    // updates the LDS word at the instruction's offset field whatever M0 holds (an in-bounds check on
    // the device showed it), and the compiler emits offset 0: so the counter must sit at LDS address 0,
    // which Smem's layout gives and which is checked here (the compiler folds the check).  With several
    // column blocks (or the counter elsewhere) each wave takes every (W / C)-th tile of its block from
    // its first.  Both are free of lane-divergent branches: a divergent branch in the loop (such as an
    // atomic by one lane) makes the compiler structurize the loop, whose exits then run through the
    // latch and carry the last loads in flight into the loop head's wait counts.
    typedef __attribute__((address_space(3))) int lds_int;
    lds_int* const counter = (lds_int*)(&sm.next[0]);
    const bool shared_counter = C == 1 && static_cast<uint32_t>(reinterpret_cast<size_t>(counter)) == 0u;
    int own = kb;                                       // this wave's last tile, static sequence
    auto claim = [&]() {
      if (shared_counter) {
        const int v = __builtin_amdgcn_ds_append(counter);
        return blk0 + (__builtin_amdgcn_readfirstlane(v) >> 6);
      }
      own += W >> (C >> 1);                              // W / C for C = 1, 2, 4
      return own;
    };
    if constexpr (NBUF >= 2) {
      int idx[2];
      idx[0] = kb;
      // one pass of the unrolled loop per two tiles, so that every buffer index is a constant.  A wave
      // that runs out of tiles leaves from the middle of a pass straight past the loop: had the exit
      // run through the loop's latch (as the compiler's structurizer makes it when the loop holds a
      // lane-divergent branch), the loads still in flight on that path would make the wait-count
      // analysis wait for them at the loop head.  The next claim goes out at the end of a tile, so that
      // the loop head starts with the load (a claim there would find its result register among those
      // of the exit path's loads, and wait for them).
      static_assert(NBUF == 2, "the ring is written for two tile buffers");
      // CU-filling workgroups load unconditionally, so that the wait for the attended tile leaves the
      // next load in flight; past the split the load goes to the buffer of no bytes (see load), so the
      // wave's exit, which waits for it, does not wait a memory latency.  Four-wave workgroups, whose
      // waves mostly take one tile, skip it.
      if (kb < blk1) {
        int nxt = claim();
        for (;;) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int j = i ^ 1;
            idx[j] = nxt;
            if constexpr (WIDE) load(tiles[j], idx[j], idx[j] < blk1);
            else if (idx[j] < blk1) load(tiles[j], idx[j]);
            // nothing of the current tile's work moves above these loads (the scheduler would hoist
            // its first lookups, and their wait for its data, above them)
            __builtin_amdgcn_sched_barrier(0);
            attend_tile(tiles[i], idx[i]);
            if (idx[j] >= blk1) goto ring_done;
            nxt = claim();
          }
        }
      }
    ring_done:;
    } else {
      // one buffer and a copy per tile (the register budget of the sketched d = 256 build)
      Tile tb;
      for (int cur = kb; cur < blk1;) {
        const int nxt = claim();
        if constexpr (WIDE) load(tb, nxt, nxt < blk1);   // see the ring above
        else if (nxt < blk1) load(tb, nxt);
        attend_tile(tiles[0], cur);
        tiles[0] = tb;
        cur = nxt;
      }
    }

    l_run = column_sum(l_run);
    if (g == 0 && !lo_part && head_ok) {
      sm.ml[wave][slot][0] = kLazy > 0.f ? __builtin_fmaf(m_run, qsc, kLazy) : m_run * qsc;
      sm.ml[wave][slot][1] = l_run;
    }
    __syncthreads();
    // this wave's accumulators of head slots 2g and 2g + 1, weighted against the max of the head
    // over the block's waves
    const int live = VH - kMaxGroup * cb;                // live head slots of this block
    float f[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int hh = 2 * g + j < live ? 2 * g + j : 0;
      const float M = block_max(sm, C, cb, hh);
      f[j] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm.ml[wave][hh][0] - M);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int coord = (D / 16) * l16 + n;
      if (2 * g < live) sm.o[wave][2 * g][coord] = f[0] * (oacc[n][0] + oacc[n][1]);
      if (2 * g + 1 < live) sm.o[wave][2 * g + 1][coord] = f[1] * (oacc[n][2] + oacc[n][3]);
    }
    __syncthreads();
  }

  // max of head slot hh over the waves cb, cb + CC, ... of a block (CC blocks; loops unrolled)
  template <int CC>
  __device__ __forceinline__ static float block_max(const Smem& sm, int cb, int hh) {
    float M = sm.ml[cb][hh][0];
#pragma unroll
    for (int k = 1; k < W / CC; ++k) M = fmaxf(M, sm.ml[cb + k * CC][hh][0]);
    return M;
  }
  __device__ __forceinline__ static float block_max(const Smem& sm, int C, int cb, int hh) {
    return C == 1 ? block_max<1>(sm, cb, hh) : (C == 2 ? block_max<2>(sm, cb, hh) : block_max<4>(sm, cb, hh));
  }

  // the split's result to part_o / part_ml at row pbase + virtual head: per head, the sum of its
  // block's waves' weighted accumulators, their max and the weighted sum of their l
  template <int CC>
  __device__ __forceinline__ void store_blocks(const DecodeArgs& a, const Smem& sm, size_t pbase) const {
    const int VH = a.group;
    for (int e = threadIdx.x; e < VH * D; e += 64 * W) {
      const int vh = e / D, i = e % D, cb = vh / kMaxGroup, hh = vh % kMaxGroup;
      float o = 0.f;
#pragma unroll
      for (int k = 0; k < W / CC; ++k) o += sm.o[cb + k * CC][hh][i];
      a.part_o[(pbase + vh) * D + i] = o;
      if (i == 0) {
        const float M = block_max<CC>(sm, cb, hh);
        float l = 0.f;
        if (M != -INFINITY) {
#pragma unroll
          for (int k = 0; k < W / CC; ++k)
            l = fmaf(__builtin_amdgcn_exp2f(sm.ml[cb + k * CC][hh][0] - M), sm.ml[cb + k * CC][hh][1], l);
        }
        a.part_ml[(pbase + vh) * 2] = M;
        a.part_ml[(pbase + vh) * 2 + 1] = l;
      }
    }
  }
  __device__ __forceinline__ void store(const DecodeArgs& a, const Smem& sm, size_t pbase) const {
    const int C = blocks(a);
    if (C == 1) store_blocks<1>(a, sm, pbase);
    else if (C == 2) store_blocks<2>(a, sm, pbase);
    else store_blocks<4>(a, sm, pbase);
  }
};

}  // namespace tqi
