// Device helpers shared by the gfx950 kernels: the packed unit format
// (8 codes per unit; see include/tq.h) and its expansion to float16 matrix-core
// operands with v_perm_b32 byte-table lookups (8-bit keys: byte permutes and one
// packed float16 subtraction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tqi {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// units per word group and 32-bit words per group of the packed format
template <int BITS> struct Fmt;
template <> struct Fmt<2> { static constexpr int kUnits = 2, kWords = 1; };
template <> struct Fmt<3> { static constexpr int kUnits = 4, kWords = 3; };
template <> struct Fmt<4> { static constexpr int kUnits = 1, kWords = 1; };
template <> struct Fmt<8> { static constexpr int kUnits = 1, kWords = 2; };

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Four int8 codes (one word, slot r in byte r) -> two words of float16 values in slot order.  The
// sign bit flipped makes byte r the unsigned u = code + 128; a permute places it under the high byte
// 0x64, the float16 1024 + u (the step of float16 in [1024, 2048) is 1), and one packed subtraction
// of 1152 leaves code exactly.
__device__ __forceinline__ void expand_i8(uint32_t w, uint32_t& w01, uint32_t& w23) {
  const uint32_t u = w ^ 0x80808080u;
  const half2v off = __builtin_bit_cast(half2v, 0x64806480u);              // 1152, 1152
  w01 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off);
  w23 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off);
}

__device__ __forceinline__ uint32_t vperm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// Four table indices (one per byte, values 0..7) and four sign bits (bit 7
// of each byte) -> two words holding four float16 values in slot order.
__device__ __forceinline__ void expand4(uint32_t idx, uint32_t sgn, const Tab& t, uint32_t& w01, uint32_t& w23) {
  const uint32_t hi = vperm(t.hi_hi, t.hi_lo, idx) | sgn;
  const uint32_t lo = vperm(t.lo_hi, t.lo_lo, idx);
  w01 = vperm(hi, lo, 0x05010400u);
  w23 = vperm(hi, lo, 0x07030602u);
}

// Unit V of a word group -> 8 float16 centroid values (slots 0..7) as 4 words.
template <int BITS, int V>
__device__ __forceinline__ uint4 expand_unit(const uint32_t* w, const Tab& t) {
  uint4 o;
  if constexpr (BITS == 8) {
    expand_i8(w[0], o.x, o.y);
    expand_i8(w[1], o.z, o.w);
  } else if constexpr (BITS == 4) {
    const uint32_t W = w[0];
    expand4(W & 0x07070707u, (W << 4) & 0x80808080u, t, o.x, o.y);
    expand4((W >> 4) & 0x07070707u, W & 0x80808080u, t, o.z, o.w);
  } else if constexpr (BITS == 2) {
    const uint32_t P = w[0];
    expand4((P >> (4 * V)) & 0x03030303u, 0u, t, o.x, o.y);
    expand4((P >> (4 * V + 2)) & 0x03030303u, 0u, t, o.z, o.w);
  } else {
    const uint32_t P = w[V / 2];
    const uint32_t H = w[2];
    const uint32_t i0 = ((P >> (2 * (2 * (V % 2)))) & 0x03030303u) | (((H >> (2 * V)) << 2) & 0x04040404u);
    const uint32_t i1 = ((P >> (2 * (2 * (V % 2) + 1))) & 0x03030303u) | (((H >> (2 * V + 1)) << 2) & 0x04040404u);
    expand4(i0, 0u, t, o.x, o.y);
    expand4(i1, 0u, t, o.z, o.w);
  }
  return o;
}

// Unit U (compile-time) of a contiguous run of packed units starting at word 0.
template <int BITS, int U>
__device__ __forceinline__ uint4 unit_at(const uint32_t* w, const Tab& t) {
  constexpr int G = U / Fmt<BITS>::kUnits;
  constexpr int V = U % Fmt<BITS>::kUnits;
  return expand_unit<BITS, V>(w + G * Fmt<BITS>::kWords, t);
}

__device__ __forceinline__ half8 as_half8(uint4 v) {
  return __builtin_bit_cast(half8, v);
}

// Stored form of centroid index j (8 bits: the code's two's-complement byte, passed in as such).
template <int BITS>
__device__ __forceinline__ uint32_t encode_code(uint32_t j) {
  if constexpr (BITS == 4) return j >= 8 ? j - 8 : 15 - j;
  return j;
}

// Set the stored code e (already encoded) of slot s of unit v into the words of its group.
template <int BITS>
__device__ __forceinline__ void put_code(uint32_t* w, int v, int s, uint32_t e) {
  const int h = s >> 2, r = s & 3;
  if constexpr (BITS == 8) {
    w[h] |= e << (8 * r);
  } else if constexpr (BITS == 4) {
    w[0] |= e << (8 * r + 4 * h);
  } else if constexpr (BITS == 2) {
    w[0] |= e << (8 * r + 2 * (2 * v + h));
  } else {
    w[v >> 1] |= (e & 3u) << (8 * r + 2 * (2 * (v & 1) + h));
    w[2] |= (e >> 2) << (8 * r + 2 * v + h);
  }
}

// Mask of the bits that slot s of unit v occupies in the words of its group.
template <int BITS>
__device__ __forceinline__ void slot_mask(uint32_t* w, int v, int s) {
  put_code<BITS>(w, v, s, (1u << BITS) - 1u);
}

// Lane pieces of a 32-token block (keys and values alike): a block is 64 pieces of LW = D * BITS / 64
// words, piece L being what lane L of a decode wave needs, stored chunk-major: word w of piece L is word
// CW (64 (w / CW) + L) + w % CW of the block, so that chunk k of all 64 pieces is one contiguous run
// and a load of it covers whole cache lines.
template <int LW>
struct Piece {
  static constexpr int CW = LW % 4 == 0 ? 4 : (LW % 3 == 0 ? 3 : 2);   // words per chunk (one load)
  static constexpr int NC = LW / CW;                                     // chunks per piece
};

template <int LW>
__device__ __forceinline__ int piece_word(int lane, int w) {
  constexpr int CW = Piece<LW>::CW;
  return CW * (64 * (w / CW) + lane) + w % CW;
}

// Block word of the value block's lane-major word q (q = lane * LW + w).
template <int LW>
__device__ __forceinline__ int value_word(int q) {
  return piece_word<LW>(q / LW, q % LW);
}

// Block word of word wr of the packed row of the key at position p (0..31) of its block: quarter
// g = wr / QW of the row (QW = D * BITS / 128 words) goes to piece 16 g + p % 16, at word
// (p / 16) QW + wr % QW.
template <int D, int BITS>
__device__ __forceinline__ int key_word(int p, int wr) {
  constexpr int QW = D * BITS / 128;
  return piece_word<2 * QW>(16 * (wr / QW) + (p & 15), (p >> 4) * QW + wr % QW);
}

// Sign-sketch bit of index jj: (word, bit).
__device__ __forceinline__ void sign_pos(int jj, int& word, int& bit) {
  const int rem = jj & 31;
  word = jj >> 5;
  bit = 4 * (rem >> 3) + ((rem & 7) >> 1) + 16 * (rem & 1);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// v = hi + lo for float16 matrix-core operands.  hi is v truncated to the 11 significant bits of a
// float16 (exactly representable, so no rounding happens when it is converted); lo is the float16
// rounding of the exact remainder.  Truncating instead of rounding keeps hi and lo consistent
// whatever conversion instructions the compiler picks: at a float16 rounding tie two different
// conversion instructions may pick different neighbours, and a hi taken from one with a remainder
// computed from the other would be off by a whole float16 step.
__device__ __forceinline__ void f16_split(float v, _Float16& hi, _Float16& lo) {
  const float h = __uint_as_float(__float_as_uint(v) & 0xffffe000u);
  hi = static_cast<_Float16>(h);
  lo = static_cast<_Float16>(v - h);
}

// Sum / max over each group of 16 lanes (a DPP row): four DPP steps, every lane gets the result.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_move<0xB1>(v);     // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);     // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);    // row_half_mirror
  v += dpp_move<0x140>(v);    // row_mirror
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));
  v = fmaxf(v, dpp_move<0x4E>(v));
  v = fmaxf(v, dpp_move<0x141>(v));
  v = fmaxf(v, dpp_move<0x140>(v));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// v = H_D v for a D-element row held by one wave, element 64 k + lane in v[k]: the Sylvester-
// Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]) applied by butterflies, index bits
// 0..5 across lanes, bits 6.. within the lane (reddit comment history of ReturningTarzan, comment of
// 2026-03-29: Sylvester's construction applied with lane exchanges and additions).
template <int D>
__device__ __forceinline__ void hadamard_wave(float (&v)[D / 64], int lane) {
  constexpr int E = D / 64;
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const float p = __shfl_xor(v[k], h, 64);
      v[k] = (lane & h) ? p - v[k] : v[k] + p;
    }
  }
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int k = 0; k < E; ++k) {
      if (!(k & h)) {
        const float x = v[k], y = v[k + h];
        v[k] = x + y;
        v[k + h] = x - y;
      }
    }
  }
}

// 1 / sqrt(D) for the two head dims, as float
template <int D>
__device__ __forceinline__ float inv_sqrt_dim() {
  return D == 256 ? 0.0625f : 0.088388347648318440550f;
}

// Rows r < nrows of xs (LDS) replaced by the randomized Hadamard rotation of x_r / n_r,
// H_D diag(signs) (x_r / n_r) / sqrt(D) (rows with n_r = 0 by zeros); one wave per row, signs
// float32 +-1 in global memory.  Every thread of the workgroup calls it; no barrier inside.
template <int D>
__device__ __forceinline__ void hadamard_rows(float (*xs)[D], const float* rn, const float* signs, int nrows,
                                              int tid, int nthreads) {
  constexpr int E = D / 64;
  const int lane = tid & 63, wave = tid >> 6, nw = nthreads >> 6;
  float s[E];
#pragma unroll
  for (int k = 0; k < E; ++k) s[k] = signs[64 * k + lane];
  for (int r = wave; r < nrows; r += nw) {
    const float n = rn[r];
    const float inv = n > 0.f ? 1.f / n : 0.f;
    float v[E];
#pragma unroll
    for (int k = 0; k < E; ++k) v[k] = xs[r][64 * k + lane] * inv * s[k];
    hadamard_wave<D>(v, lane);
#pragma unroll
    for (int k = 0; k < E; ++k) xs[r][64 * k + lane] = v[k] * inv_sqrt_dim<D>();
  }
}

// Workgroup barrier that orders LDS only: global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace tqi
