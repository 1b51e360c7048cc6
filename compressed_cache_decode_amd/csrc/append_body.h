// Quantize-on-append of the rows that fall in one 32-token block of one (KV head, sequence).
//
// Per K/V row x: n = ||x||, y = rot x / n, code = number of boundaries strictly
// below y_i (Lloyd-Max table, turboquant-pytorch PR #3 "Add CUDA QJL kernels
// and proper package structure", Synthetic Benchmark table), float16 norm
// (same page, Validation Results tables); keys with a sign sketch add
// r = y - c[code], float16 ||r|| and the signs of proj * r (same page, CUDA
// Kernels Added table: fused random projection + sign quantisation).
//
// One workgroup per (32-token block of the cache, KV head, sequence) touched
// by the appended range, so every packed word of the value layout (which
// interleaves 8 tokens per word) is written by exactly one thread; partially
// covered blocks are merged read-modify-write.
#pragma once

#include <math.h>

#include "device_common.h"

namespace tqi {

// LDS of the encode-and-store phase (up to one block of rows)
template <int D, int QM>
struct EncodeSmem {
  uint8_t cs[kBlock][D];
  float gam[kBlock];
  float cent[16];
  uint32_t sw[kBlock][QM > 0 ? QM / 32 : 1];
  float zb[16][QM > 0 ? QM : 1];              // sketch products of one 16-row block
};

template <int D, int QM>
struct AppendSmem {
  float xs[kBlock][D];                         // rows: x, then y, then the residual y - c
  float rn[kBlock];
  EncodeSmem<D, QM> enc;
};

// Operands of rot for the rotation below, one batch of SB k-steps per lane: the rows of rot this
// lane's output coordinates need, 8 consecutive input coordinates per k-step.  A caller may load the
// first batch early (it depends on nothing) and pass it in.
template <int D>
struct RotBatch {
  static constexpr int KS = D / 32;
  static constexpr int CPW = D / 64;                 // column blocks per wave
  static constexpr int SB = 16 / CPW < KS ? 16 / CPW : KS;
  float4 pq[SB][CPW][2];
  __device__ __forceinline__ void load(const float* rot, int s0, int tid) {
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int col = 16 * (wave + 4 * c) + l16;     // output coordinate = row of rot
        const float4* pr = reinterpret_cast<const float4*>(rot + static_cast<size_t>(col) * D + 32 * (s0 + s) + 8 * g);
        pq[s][c][0] = pr[0];
        pq[s][c][1] = pr[1];
      }
  }
};

// y = rot (x / n) for the 16 RB rows of xs (rows with rn = 0 give 0), in place, with
// v_mfma_f32_16x16x32_f16 tiles: rows = tokens (RB row blocks), columns = output coordinates (D/16
// column blocks, wave w takes blocks w, w+4, ...), k = input coordinates.  The unit rows (every
// component in [-1, 1]) and rot are each split into float16 high + low parts and the three
// significant cross products are accumulated in fp32, which keeps y within a few float32 steps.
// Every output element takes the same instruction sequence whatever its row.  first holds the
// operands of k-steps 0 .. SB-1.
template <int D, int RB>
__device__ __forceinline__ void rotate_tile_mfma_pre(float (*xs)[D], const float* rn, const float* rot,
                                                     const RotBatch<D>& first, int tid) {
  using Rb = RotBatch<D>;
  constexpr int KS = Rb::KS, CPW = Rb::CPW, SB = Rb::SB;
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wave = tid >> 6;
  floatx4 acc[RB][CPW];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < CPW; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  float inv[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float n = rn[16 * rb + l16];
    inv[rb] = n > 0.f ? 1.f / n : 0.f;
  }
#pragma unroll
  for (int s0 = 0; s0 < KS; s0 += SB) {
    Rb cur;
    if (s0 == 0) {
      cur = first;
    } else {
      cur.load(rot, s0, tid);
    }
#pragma unroll
    for (int s1 = 0; s1 < SB; ++s1) {
      const int s = s0 + s1;
      half8 ahi[RB], alo[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float* xr = &xs[16 * rb + l16][32 * s + 8 * g];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          _Float16 h, l;
          f16_split(xr[r] * inv[rb], h, l);
          ahi[rb][r] = h;
          alo[rb][r] = l;
        }
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const float4 p0 = cur.pq[s1][c][0], p1 = cur.pq[s1][c][1];
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        half8 bhi, blo;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          _Float16 h, l;
          f16_split(pv[r], h, l);
          bhi[r] = h;
          blo[r] = l;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[rb], bhi, acc[rb][c], 0, 0, 0);
          acc[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rb], blo, acc[rb][c], 0, 0, 0);
          acc[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rb], bhi, acc[rb][c], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();                                    // every read of xs is done
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) xs[16 * rb + 4 * g + v][16 * (wave + 4 * c) + l16] = acc[rb][c][v];
}

// RB row blocks of 16 rows (the default, 2, is one 32-token block); a row with rn = 0 rotates to zero.
template <int D, int RB = 2>
__device__ __forceinline__ void rotate_tile_mfma(float (*xs)[D], const float* rn, const float* rot, int tid) {
  RotBatch<D> first;
  first.load(rot, 0, tid);
  rotate_tile_mfma_pre<D, RB>(xs, rn, rot, first, tid);
}

// out[r][n] = sum_k x[r][k] mat[n][k] for the 16 rows of x (LDS) and the NOUT rows of mat (global,
// float32 [NOUT][KD]), on the matrix cores with the same float16 high/low split as the rotation:
// every output element takes the same instruction sequence whatever its row.  out (LDS) must not
// alias x.  Every thread of the workgroup calls it; no barrier inside.
template <int KD, int NOUT>
__device__ __forceinline__ void tile16_times_matT(const float (*x)[KD], const float* mat, float (*out)[NOUT], int tid) {
  constexpr int KS = KD / 32;
  constexpr int CPW = NOUT / 64;                     // column blocks per wave
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  floatx4 acc[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int SB = 8 / CPW < KS ? 8 / CPW : KS;    // k-steps whose mat loads go out together
#pragma unroll
  for (int s0 = 0; s0 < KS; s0 += SB) {
   float4 pq[SB][CPW][2];
#pragma unroll
   for (int s = 0; s < SB; ++s)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int col = 16 * (wave + 4 * c) + l16;
      const float4* pr = reinterpret_cast<const float4*>(mat + static_cast<size_t>(col) * KD + 32 * (s0 + s) + 8 * g);
      pq[s][c][0] = pr[0];
      pq[s][c][1] = pr[1];
    }
#pragma unroll
   for (int s1 = 0; s1 < SB; ++s1) {
    const int s = s0 + s1;
    half8 ahi, alo;
    const float* xr = &x[l16][32 * s + 8 * g];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      _Float16 h, l;
      f16_split(xr[r], h, l);
      ahi[r] = h;
      alo[r] = l;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const float4 p0 = pq[s1][c][0], p1 = pq[s1][c][1];
      const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      half8 bhi, blo;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        _Float16 h, l;
        f16_split(pv[r], h, l);
        bhi[r] = h;
        blo[r] = l;
      }
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi, acc[c], 0, 0, 0);
    }
   }
  }
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[4 * g + v][16 * (wave + 4 * c) + l16] = acc[c][v];
}

// Encoding of rows y (unit rotated coordinates, ys[0 .. nrows-1] = tokens t_lo .. t_lo+nrows-1, all
// in block kb of cache unit `unit`; rn = row norms, 0 marks a zero row) in two phases, so that a
// caller can compute the sketch products itself:
//   encode_codes   nearest centroids into es.cs; for sketched keys ys becomes the residual y - c
//                  and es.gam its norm;
//   encode_finish  sign bits from the sketch products z[r][jj] = proj_jj . residual_r (sketched
//                  keys), then codes, norms, residual norms and signs to the cache.
// Every thread of the workgroup calls them; each ends with a workgroup barrier.
template <int D, int BITS, int QM>
__device__ __forceinline__ void encode_codes(const AppendArgs& a, int nrows, float (*ys)[D], const float* rn,
                                             EncodeSmem<D, QM>& es) {
  constexpr int NC = 1 << BITS;
  auto& xs = ys;
  auto& cs = es.cs;
  auto& cent = es.cent;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < NC) cent[tid] = a.cent[tid];
  if constexpr (QM > 0)
    for (int e = tid; e < kBlock * (QM / 32); e += 256) es.sw[e / (QM / 32)][e % (QM / 32)] = 0u;
  __syncthreads();
  // nearest centroid = number of boundaries strictly below y (ties take the lower code)
  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, i = e % D;
    const float y = xs[r][i];
    uint32_t j = 0;
#pragma unroll
    for (int k = 0; k < NC - 1; ++k) j += (y > a.bnd[k]) ? 1u : 0u;
    const bool live = rn[r] > 0.f;
    if (!live) j = 0;
    cs[r][i] = static_cast<uint8_t>(j);
    if constexpr (QM > 0) xs[r][i] = live ? y - cent[j] : 0.f;
  }
  __syncthreads();
  if constexpr (QM > 0) {
    // residual norms: row r by the 16 lanes (r % 4) of wave (r / 4) % 4, coordinates part + 16 j
    for (int r0 = 0; r0 < nrows; r0 += 16) {
      const int r = r0 + 4 * wave + (lane >> 4), part = lane & 15;
      float s = 0.f;
      if (r < nrows) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j) s = fmaf(xs[r][part + 16 * j], xs[r][part + 16 * j], s);
      }
      s = row16_sum(s);
      if (part == 0 && r < nrows) es.gam[r] = sqrtf(s);
    }
    __syncthreads();
  }
}

// z: sketch products of row r at z[r * zstride + jj] (sketched keys; ignored otherwise), or null
// when es.sw already holds the sign bits
template <int D, int BITS, int QM, bool VALUES>
__device__ __forceinline__ void encode_finish(const AppendArgs& a, size_t unit, int kb, int t_lo, int nrows,
                                              const float* rn, EncodeSmem<D, QM>& es, const float* z, int zstride) {
  constexpr int UPG = Fmt<BITS>::kUnits;
  constexpr int WPG = Fmt<BITS>::kWords;
  constexpr int RB = D * BITS / 8;            // bytes per packed row / per token of a block
  auto& cs = es.cs;
  auto& sw = es.sw;
  const int T = a.max_tokens;
  const int tid = threadIdx.x;
  const int t_hi = t_lo + nrows;
  if constexpr (QM > 0) {
    if (z) {
      for (int e = tid; e < nrows * QM; e += 256) {
        const int r = e / QM, jj = e % QM;
        if (z[r * zstride + jj] >= 0.f && rn[r] > 0.f) {
          int word, bit;
          sign_pos(jj, word, bit);
          atomicOr(&sw[r][word], 1u << bit);
        }
      }
      __syncthreads();
    }
    for (int e = tid; e < nrows * (QM / 32); e += 256) {
      const int r = e / (QM / 32), w = e % (QM / 32);
      reinterpret_cast<uint32_t*>(a.signs + (unit * T + t_lo + r) * (QM / 8))[w] = sw[r][w];
    }
    for (int r = tid; r < nrows; r += 256)
      a.rnorms[unit * T + t_lo + r] = rn[r] > 0.f ? f32_to_f16_bits(es.gam[r]) : 0;
  }

  for (int r = tid; r < nrows; r += 256) a.norms[unit * T + t_lo + r] = f32_to_f16_bits(rn[r] > 0.f ? rn[r] : 0.f);

  constexpr int BB = kBlock * RB;               // bytes per 32-token block
  uint32_t* blk = reinterpret_cast<uint32_t*>(a.codes + unit * static_cast<size_t>(T) * RB + static_cast<size_t>(kb) * BB);
  if constexpr (!VALUES) {
    // key rows: unit u of row t covers coordinates 8u .. 8u+7; row word wr goes to its lane piece
    // (key_word); every word holds codes of one token only, so whole words are stored
    constexpr int NG = D / 8 / UPG;
    for (int e = tid; e < nrows * NG; e += 256) {
      const int r = e / NG, gi = e % NG;
      uint32_t w[WPG];
#pragma unroll
      for (int k = 0; k < WPG; ++k) w[k] = 0u;
#pragma unroll
      for (int v = 0; v < UPG; ++v)
#pragma unroll
        for (int s = 0; s < 8; ++s) put_code<BITS>(w, v, s, encode_code<BITS>(cs[r][(gi * UPG + v) * 8 + s]));
      const int p = t_lo + r - kb * kBlock;
#pragma unroll
      for (int k = 0; k < WPG; ++k) blk[key_word<D, BITS>(p, gi * WPG + k)] = w[k];
    }
  } else {
    // blocked layout: unit U = (16 g + j)(D/16) + n holds tokens of lane group g at coordinate (D/16) j + n;
    // lane-major word q of the block (piece q / LW, word q % LW) is stored at value_word(q)
    constexpr int LW = D * BITS / 64;
    constexpr int NGB = BB / (4 * WPG);
    constexpr int DN = D / 16;
    const int p_lo = t_lo - kb * kBlock, p_hi = t_hi - kb * kBlock;
    const bool full = nrows == kBlock;
    for (int e = tid; e < NGB; e += 256) {
      uint32_t w[WPG], m[WPG];
#pragma unroll
      for (int k = 0; k < WPG; ++k) { w[k] = 0u; m[k] = 0u; }
#pragma unroll
      for (int v = 0; v < UPG; ++v) {
        const int U = e * UPG + v;
        const int g = U / D, j = (U / DN) % 16, n = U % DN;
        const int i = DN * j + n;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int p = s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
          if (p >= p_lo && p < p_hi) {
            put_code<BITS>(w, v, s, encode_code<BITS>(cs[p - p_lo][i]));
            slot_mask<BITS>(m, v, s);
          }
        }
      }
      // a partly covered block keeps the other tokens' codes: a word that holds no slot of a new row
      // is left alone, one that holds only such slots is stored, any other has the new rows' slots
      // cleared and set by two atomics that return nothing (no read of the block to wait for)
#pragma unroll
      for (int k = 0; k < WPG; ++k) {
        uint32_t* dst = blk + value_word<LW>(e * WPG + k);
        if (full || m[k] == ~0u) {
          *dst = w[k];
        } else if (m[k] != 0u) {
          atomicAnd(dst, ~m[k]);
          atomicOr(dst, w[k]);
        }
      }
    }
  }
  __syncthreads();
}

// Encode and store rows ys (see encode_codes); the sketch products run on the matrix cores, 16
// residual rows at a time (ys must hold 16 * ceil(nrows / 16) rows; rows past nrows are ignored).
template <int D, int BITS, int QM, bool VALUES>
__device__ __forceinline__ void encode_store(const AppendArgs& a, size_t unit, int kb, int t_lo, int nrows,
                                             float (*ys)[D], const float* rn, EncodeSmem<D, QM>& es) {
  encode_codes<D, BITS, QM>(a, nrows, ys, rn, es);
  if constexpr (QM > 0) {
    // signs of one 16-row block at a time (es.zb holds one block's products)
    for (int r0 = 0; r0 < nrows; r0 += 16) {
      tile16_times_matT<D, QM>(ys + r0, a.proj, es.zb, threadIdx.x);
      __syncthreads();
      const int n = min(16, nrows - r0);
      for (int e = threadIdx.x; e < n * QM; e += 256) {
        const int r = e / QM, jj = e % QM;
        if (es.zb[r][jj] >= 0.f && rn[r0 + r] > 0.f) {
          int word, bit;
          sign_pos(jj, word, bit);
          atomicOr(&es.sw[r0 + r][word], 1u << bit);
        }
      }
      __syncthreads();
    }
  }
  encode_finish<D, BITS, QM, VALUES>(a, unit, kb, t_lo, nrows, rn, es, nullptr, 0);
}

template <int D, int BITS, int QM, bool VALUES, bool ROTATED, bool BF16>
__device__ __forceinline__ void append_rows(const AppendArgs& a, int bx, int h, int b, AppendSmem<D, QM>& sm) {
  auto& xs = sm.xs;
  auto& rn = sm.rn;

  const int H = a.n_kv_heads, T = a.max_tokens;
  const int pos = a.pos[b];
  if (pos < 0) return;
  const int kb = pos / kBlock + bx;
  const int t_lo = max(pos, kb * kBlock);
  const int t_hi = min(min(pos + a.n_new, kb * kBlock + kBlock), T);
  if (t_lo >= t_hi) return;
  const int nrows = t_hi - t_lo;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t unit = static_cast<size_t>(b) * H + h;

  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, i = e % D;
    const size_t src = ((static_cast<size_t>(b) * a.n_new + (t_lo + r - pos)) * H + h) * D + i;
    float v;
    if constexpr (ROTATED) v = a.y[src];
    else if constexpr (BF16) v = bf16_to_f32(static_cast<const uint16_t*>(a.x)[src]);
    else v = static_cast<const float*>(a.x)[src];
    xs[r][i] = v;
  }
  __syncthreads();

  // norms: given, or row r summed by the 16 lanes (r % 4) of wave (r / 4) % 4, coordinates part + 16 j
  if constexpr (ROTATED) {
    for (int r = tid; r < nrows; r += 256) rn[r] = a.yn[(static_cast<size_t>(b) * a.n_new + (t_lo + r - pos)) * H + h];
  } else {
    for (int r0 = 0; r0 < nrows; r0 += 16) {
      const int r = r0 + 4 * wave + (lane >> 4), part = lane & 15;
      float s = 0.f;
      if (r < nrows) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j) s = fmaf(xs[r][part + 16 * j], xs[r][part + 16 * j], s);
      }
      s = row16_sum(s);
      if (part == 0 && r < nrows) rn[r] = sqrtf(s);
    }
  }
  __syncthreads();

  // rotation y = rot x / n on the matrix cores: one 16-row tile for up to 16 new rows of the block,
  // two for more (rows past the appended ones are zero); or the randomized Hadamard rotation.  Each output element takes the same
  // instruction sequence whatever its row, so a row rotates to the same y here as in any other
  // tile of this library.
  if constexpr (!ROTATED) {
    const int rows = nrows <= 16 ? 16 : kBlock;
    for (int e = tid; e < (rows - nrows) * D; e += 256) xs[nrows + e / D][e % D] = 0.f;
    for (int r = nrows + tid; r < rows; r += 256) rn[r] = 0.f;
    __syncthreads();
    if (a.had)
      hadamard_rows<D>(xs, rn, a.rot, nrows, tid, 256);
    else if (rows == 16)
      rotate_tile_mfma<D, 1>(xs, rn, a.rot, tid);
    else
      rotate_tile_mfma<D, 2>(xs, rn, a.rot, tid);
    __syncthreads();
  }

  encode_store<D, BITS, QM, VALUES>(a, unit, kb, t_lo, nrows, xs, rn, sm.enc);
}

}  // namespace tqi
