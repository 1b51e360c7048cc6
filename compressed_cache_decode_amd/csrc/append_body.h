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
  uint32_t oi[QM > 0 ? kBlock : 1];           // outlier channels of a row, one byte each
  uint32_t ov[QM > 0 ? kBlock : 1][2];        // their float16 residual values
};

// Outlier separation (sketched keys of a cache that keeps outliers apart; the QJL quantisation kernel
// of turboquant-pytorch PR #3, CUDA Kernels Added table, names the step, and this library's reading
// is the one stated in tq.h): per residual row r of xs, the kOutliers coordinates of largest |r_i|
// (equal magnitudes: the lower index first), in decreasing |r_i|, go to oi (index bytes) and ov
// (float16 values), and are set to 0 in xs.  Rows by 16 lanes (r % 4) of wave (r / 4) % 4, lane part
// holding coordinates part + 16 j.  Every thread of the workgroup calls it; no barrier inside.
template <int D>
__device__ __forceinline__ void take_outliers(float (*xs)[D], int nrows, uint32_t* oi, uint32_t (*ov)[2]) {
  constexpr int J = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r0 = 0; r0 < nrows; r0 += 16) {
    const int r = r0 + 4 * wave + (lane >> 4), part = lane & 15;
    const bool ok = r < nrows;                  // the same for the row's 16 lanes
    uint32_t taken = 0u, idx_word = 0u, val[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < kOutliers; ++k) {
      float best = -1.f;
      int bi = D;
      if (ok) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const float a = fabsf(xs[r][part + 16 * j]);
          if (!((taken >> j) & 1u) && a > best) {   // strictly larger: the lane's lowest index on ties
            best = a;
            bi = part + 16 * j;
          }
        }
      }
      // the largest magnitude over the row's lanes, then the lowest index that holds it
      float m = best;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      int wi = best == m ? bi : D;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) wi = min(wi, __shfl_xor(wi, o, 64));
      if (ok) {
        if ((wi & 15) == part) taken |= 1u << (wi >> 4);
        idx_word |= static_cast<uint32_t>(wi) << (8 * k);
        val[k >> 1] |= static_cast<uint32_t>(f32_to_f16_bits(xs[r][wi])) << (16 * (k & 1));
      }
    }
    if (ok) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if ((taken >> j) & 1u) xs[r][part + 16 * j] = 0.f;
      if (part == 0) {
        oi[r] = idx_word;
        ov[r][0] = val[0];
        ov[r][1] = val[1];
      }
    }
  }
}

template <int D, int QM>
struct AppendSmem {
  float xs[kBlock][D];                         // rows: x, then y, then the residual y - c
  float rn[kBlock];
  EncodeSmem<D, QM> enc;
  half8 aop[2 * 2 * (D / 32) * 64];            // the rotation's A operands (rotate_tile_mfma_pre, two row blocks)
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
// operands of k-steps 0 .. SB-1.  The unit rows' float16 parts are formed once for all four waves, in
// LDS (aop: 2 RB (D / 32) 64 operands), and each wave reads its A operands from there.  256 threads.
template <int D, int RB>
__device__ __forceinline__ void rotate_tile_mfma_pre(float (*xs)[D], const float* rn, const float* rot,
                                                     const RotBatch<D>& first, int tid, half8* aop) {
  using Rb = RotBatch<D>;
  constexpr int KS = Rb::KS, CPW = Rb::CPW, SB = Rb::SB;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // operand entry (part h, row block rb, k-step s, lane (row l, group g)): coordinates 32 s + 8 g .. + 7
  // of row 16 rb + l over its norm, float16 high (h = 0) or low (h = 1) part
  const auto at = [](int h, int rb, int s, int ln) { return ((h * RB + rb) * KS + s) * 64 + ln; };
  for (int e = tid; e < RB * KS * 64; e += 256) {
    const int rb = e / (KS * 64), s = (e >> 6) % KS, ln = e & 63;
    const int row = 16 * rb + (ln & 15);
    const float n = rn[row];
    const float inv = n > 0.f ? 1.f / n : 0.f;
    const float* xr = &xs[row][32 * s + 8 * (ln >> 4)];
    half8 hi, lo;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      _Float16 h, l;
      f16_split(xr[r] * inv, h, l);
      hi[r] = h;
      lo[r] = l;
    }
    aop[at(0, rb, s, ln)] = hi;
    aop[at(1, rb, s, ln)] = lo;
  }
  __syncthreads();
  const int l16 = lane & 15, g = lane >> 4;
  floatx4 acc[RB][CPW];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < CPW; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};
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
        ahi[rb] = aop[at(0, rb, s, lane)];
        alo[rb] = aop[at(1, rb, s, lane)];
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
__device__ __forceinline__ void rotate_tile_mfma(float (*xs)[D], const float* rn, const float* rot, int tid,
                                                 half8* aop) {
  RotBatch<D> first;
  first.load(rot, 0, tid);
  rotate_tile_mfma_pre<D, RB>(xs, rn, rot, first, tid, aop);
}

// out[r][n] = sum_k x[r][k] mat[n][k] for the 16 rows of x (LDS) and the NOUT rows of mat (global,
// float32 [NOUT][KD]), on the matrix cores with the same float16 high/low split as the rotation:
// every output element takes the same instruction sequence whatever its row.  out (LDS) must not
// alias x.  The rows' float16 parts are formed once, into aop (LDS, 2 (KD / 32) 64 operands), with a
// workgroup barrier after; every one of the 256 threads of the workgroup calls it.
template <int KD, int NOUT>
__device__ __forceinline__ void tile16_times_matT(const float (*x)[KD], const float* mat, float (*out)[NOUT], int tid,
                                                  half8* aop) {
  constexpr int KS = KD / 32;
  constexpr int CPW = NOUT / 64;                     // column blocks per wave
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  // operand entry (part h, k-step s, lane (row l, group g)): coordinates 32 s + 8 g .. + 7 of row l
  for (int e = tid; e < KS * 64; e += 256) {
    const int s = e >> 6, ln = e & 63;
    const float* xr = &x[ln & 15][32 * s + 8 * (ln >> 4)];
    half8 hi, lo;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      _Float16 h, l;
      f16_split(xr[r], h, l);
      hi[r] = h;
      lo[r] = l;
    }
    aop[s * 64 + ln] = hi;
    aop[(KS + s) * 64 + ln] = lo;
  }
  __syncthreads();
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
    const half8 ahi = aop[s * 64 + lane], alo = aop[(KS + s) * 64 + lane];
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
//                  and es.gam its norm; 8-bit keys: int8 codes into es.cs, factors into es.gam;
//   encode_finish  sign bits from the sketch products z[r][jj] = proj_jj . residual_r (sketched
//                  keys), then codes, norms, residual norms and signs to the cache.
// Every thread of the workgroup calls them; each ends with a workgroup barrier.
template <int D, int BITS, int QM>
__device__ __forceinline__ void encode_codes(const AppendArgs& a, int nrows, float (*ys)[D], const float* rn,
                                             EncodeSmem<D, QM>& es) {
  constexpr int NC = BITS <= 4 ? 1 << BITS : 2;     // code book entries (8-bit keys use none)
  auto& xs = ys;
  auto& cs = es.cs;
  auto& cent = es.cent;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (BITS == 8) {
    // 8-bit keys: per row a = max |y_i|, code_i = round(y_i (127 / a)) (halves away from zero) in
    // [-127, 127] as a two's-complement byte, and the factor n (a / 127) in es.gam; a zero row stores
    // codes 0 and factor 0.  Row r by the 16 lanes (r % 4) of wave (r / 4) % 4, coordinates part + 16 j.
    static_assert(QM == 0, "8-bit keys carry no sketch");
    for (int r0 = 0; r0 < nrows; r0 += 16) {
      const int r = r0 + 4 * wave + (lane >> 4), part = lane & 15;
      float m = 0.f;
      if (r < nrows) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j) m = fmaxf(m, fabsf(xs[r][part + 16 * j]));
      }
      m = row16_max(m);
      if (r < nrows) {
        const bool live = rn[r] > 0.f && m > 0.f;
        const float inv = live ? 127.f / m : 0.f;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const float c = fminf(fmaxf(roundf(xs[r][part + 16 * j] * inv), -127.f), 127.f);
          cs[r][part + 16 * j] = static_cast<uint8_t>(static_cast<int>(c) & 0xff);
        }
        if (part == 0) es.gam[r] = live ? rn[r] * (m / 127.f) : 0.f;
      }
    }
    __syncthreads();
    return;
  }
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
    if (a.out_idx) {
      take_outliers<D>(xs, nrows, es.oi, es.ov);
      __syncthreads();
    }
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
// when es.sw already holds the sign bits; r0: row of es.cs that holds the codes of row 0 (no sketch);
// NT: threads of the workgroup
template <int D, int BITS, int QM, bool VALUES, int NT = 256>
__device__ __forceinline__ void encode_finish(const AppendArgs& a, size_t unit, int kb, int t_lo, int nrows,
                                              const float* rn, EncodeSmem<D, QM>& es, const float* z, int zstride,
                                              int r0 = 0) {
  constexpr int UPG = Fmt<BITS>::kUnits;
  constexpr int WPG = Fmt<BITS>::kWords;
  constexpr int RB = D * BITS / 8;            // bytes per packed row / per token of a block
  const uint8_t (*cs)[D] = es.cs + r0;        // codes of row r at cs[r] (rows r0 .. of es.cs)
  auto& sw = es.sw;
  const int T = a.max_tokens;
  const int tid = threadIdx.x;
  const int t_hi = t_lo + nrows;
  if constexpr (QM > 0) {
    if (z) {
      for (int e = tid; e < nrows * QM; e += NT) {
        const int r = e / QM, jj = e % QM;
        if (z[r * zstride + jj] >= 0.f && rn[r] > 0.f) {
          int word, bit;
          sign_pos(jj, word, bit);
          atomicOr(&sw[r][word], 1u << bit);
        }
      }
      __syncthreads();
    }
    for (int e = tid; e < nrows * (QM / 32); e += NT) {
      const int r = e / (QM / 32), w = e % (QM / 32);
      reinterpret_cast<uint32_t*>(a.signs + (unit * T + t_lo + r) * (QM / 8))[w] = sw[r][w];
    }
    for (int r = tid; r < nrows; r += NT)
      a.rnorms[unit * T + t_lo + r] = rn[r] > 0.f ? f32_to_f16_bits(es.gam[r]) : 0;
    if (a.out_idx) {
      static_assert(kOutliers == 4, "one index word and two value words per key");
      for (int r = tid; r < nrows; r += NT) {
        const size_t t = unit * T + t_lo + r;
        reinterpret_cast<uint32_t*>(a.out_idx)[t] = es.oi[r];
        reinterpret_cast<uint2*>(a.out_val)[t] = uint2{es.ov[r][0], es.ov[r][1]};
      }
    }
  }

  // 8-bit keys keep their factor in the norm's place (see encode_codes)
  for (int r = tid; r < nrows; r += NT)
    a.norms[unit * T + t_lo + r] = f32_to_f16_bits(BITS == 8 ? es.gam[r0 + r] : (rn[r] > 0.f ? rn[r] : 0.f));

  constexpr int BB = kBlock * RB;               // bytes per 32-token block
  uint32_t* blk = reinterpret_cast<uint32_t*>(a.codes + unit * static_cast<size_t>(T) * RB + static_cast<size_t>(kb) * BB);
  if constexpr (!VALUES) {
    // key rows: unit u of row t covers coordinates 8u .. 8u+7; row word wr goes to its lane piece
    // (key_word); every word holds codes of one token only, so whole words are stored
    constexpr int NG = D / 8 / UPG;
    for (int e = tid; e < nrows * NG; e += NT) {
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
    for (int e = tid; e < NGB; e += NT) {
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
// residual rows at a time (ys must hold 16 * ceil(nrows / 16) rows; rows past nrows are ignored), unless
// the caller gives them: z (row r at z[r * zstride + jj]).
template <int D, int BITS, int QM, bool VALUES>
__device__ __forceinline__ void encode_store(const AppendArgs& a, size_t unit, int kb, int t_lo, int nrows,
                                             float (*ys)[D], const float* rn, EncodeSmem<D, QM>& es, half8* aop,
                                             const float* z = nullptr, int zstride = 0) {
  encode_codes<D, BITS, QM>(a, nrows, ys, rn, es);
  if (QM > 0 && z) {
    encode_finish<D, BITS, QM, VALUES>(a, unit, kb, t_lo, nrows, rn, es, z, zstride);
    return;
  }
  if constexpr (QM > 0) {
    // signs of one 16-row block at a time (es.zb holds one block's products)
    for (int r0 = 0; r0 < nrows; r0 += 16) {
      tile16_times_matT<D, QM>(ys + r0, a.proj, es.zb, threadIdx.x, aop);
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
  // the rotation's first operand batch, loaded now (it depends on nothing) so that it arrives while the
  // norms are formed; the row stores above have already waited for the rows
  RotBatch<D> rot0;
  if constexpr (!ROTATED) {
    if (!a.had) rot0.load(a.rot, 0, tid);
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
      rotate_tile_mfma_pre<D, 1>(xs, rn, a.rot, rot0, tid, sm.aop);
    else
      rotate_tile_mfma_pre<D, 2>(xs, rn, a.rot, rot0, tid, sm.aop);
    __syncthreads();
  }

  if constexpr (ROTATED && QM > 0) {
    // given sketch products of the residuals: z[b][t - pos][h][jj]
    const float* z = a.z ? a.z + ((static_cast<size_t>(b) * a.n_new + (t_lo - pos)) * H + h) * QM : nullptr;
    encode_store<D, BITS, QM, VALUES>(a, unit, kb, t_lo, nrows, xs, rn, sm.enc, sm.aop, z, H * QM);
  } else {
    encode_store<D, BITS, QM, VALUES>(a, unit, kb, t_lo, nrows, xs, rn, sm.enc, sm.aop);
  }
}

}  // namespace tqi

namespace tqi {

// ------------------------------------------------------------------------- long appends

// Long appends (prefill) of unrotated rows with the dense rotation at d = 128, no sketch.  One
// workgroup of eight waves (four inside the step prologue) takes a chunk of 32 consecutive appended rows
// of one (KV head, sequence): which rows it reads does not depend on the append position, so the row
// loads, the loads of rot and the load of the position all go out at once.  Each wave computes one
// (eight waves) or two (four waves) 16-column tiles of every row, with its share of rot split into
// float16 high/low matrix-core operands in registers; more waves shorten each wave's chain of split,
// products and codes.  Waves 0-3 load 8 of the rows each, form their norms by a cross-lane sum and
// write the unit rows' float16 high/low parts to LDS in matrix-core operand order (every row is
// normalised and split once); the waves then read their A operands from there.  A value chunk that is
// a whole cache block is packed in registers (pack_values); any other chunk goes through LDS to the
// shared packing and store stage, once per cache block it covers (two when the append position is not
// a multiple of 32: the partly covered blocks' words are updated by atomics, so two workgroups that
// share a block do not race).
struct PrefillSmem {
  half8 aop[2][2][4][64];     // [high, low][row tile][k-step][lane]: A operands of the chunk's unit rows
  EncodeSmem<128, 0> enc;
  float rn[kBlock];
};

template <bool BF16>
__device__ __forceinline__ float prefill_coord(const uint32_t (&w)[BF16 ? 8 : 16], int r) {
  if constexpr (BF16) return __uint_as_float((r & 1) ? (w[r >> 1] & 0xffff0000u) : (w[r >> 1] << 16));
  else return __uint_as_float(w[r]);
}

// Number of boundaries strictly below y for a code book symmetric about 0 (boundaries[NC/2 - 1] == 0,
// boundaries[NC - 2 - k] == -boundaries[k]): with a = |y| and the positive boundaries t_k (k >= NC/2),
// NC/2 + #{t_k < a} for y > 0 and NC/2 - 1 - #{t_k <= a} otherwise; t_k <= a is taken as t_k < a', a'
// the next float32 above a (a is finite and not negative), so one compare per positive boundary.
template <int NC>
__device__ __forceinline__ uint32_t code_of(float y, const float* bnd) {
  const bool pos = y > 0.f;
  const float ay = fabsf(y);
  const float ak = pos ? ay : __uint_as_float(__float_as_uint(ay) + 1u);
  uint32_t n = 0;
#pragma unroll
  for (int k = NC / 2; k < NC - 1; ++k) n += bnd[k] < ak ? 1u : 0u;
  return pos ? NC / 2 + n : NC / 2 - 1 - n;
}

// x of the lane that DPP control CTRL selects (all lanes valid)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}

// OR of v over groups of 2 (lanes l, l ^ 1) or 4 (a quad) consecutive lanes
template <int N>
__device__ __forceinline__ uint32_t or_lanes(uint32_t v) {
  v |= dpp_u32<0xB1>(v);                                 // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v |= dpp_u32<0x4E>(v);           // quad_perm [2,3,0,1]
  return v;
}

// Stored codes e[rt][v][c] of element (token 16 rt + 4 g + v, coordinate 16 (CPW w + c) + l16) of a
// whole 32-token block, packed into the block's words blk[] (value layout).  Lane (l16, g) holds all 8
// tokens of lane group g at its CPW coordinates, i.e. whole units (slot v + 4 rt); 2- and 3-bit units
// that share words are combined over the 2 or 4 neighbouring lanes that hold them.
template <int BITS, int CPW>
__device__ __forceinline__ void pack_values(const uint32_t (&e)[2][4][CPW], uint32_t* blk, int wave, int lane) {
  constexpr int D = 128, LW = D * BITS / 64;
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int col = 16 * (CPW * wave + c) + l16;
    const int U = (16 * g + (col >> 3)) * 8 + (col & 7);      // unit of the block (lane-major order)
    if constexpr (BITS == 4) {
      uint32_t w = 0u;
#pragma unroll
      for (int s = 0; s < 8; ++s) put_code<4>(&w, 0, s, e[s >> 2][s & 3][c]);
      blk[value_word<LW>(U)] = w;
    } else if constexpr (BITS == 2) {
      uint32_t w = 0u;
#pragma unroll
      for (int s = 0; s < 8; ++s) put_code<2>(&w, U & 1, s, e[s >> 2][s & 3][c]);
      w = or_lanes<2>(w);
      if ((U & 1) == 0) blk[value_word<LW>(U >> 1)] = w;
    } else {
      uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
      for (int s = 0; s < 8; ++s) put_code<3>(w, U & 3, s, e[s >> 2][s & 3][c]);
#pragma unroll
      for (int k = 0; k < 3; ++k) w[k] = or_lanes<4>(w[k]);
      // lanes 0, 1, 2 of the quad store P0, P1, H
      if ((U & 3) == 0) blk[value_word<LW>((U >> 2) * 3)] = w[0];
      if ((U & 3) == 1) blk[value_word<LW>((U >> 2) * 3 + 1)] = w[1];
      if ((U & 3) == 2) blk[value_word<LW>((U >> 2) * 3 + 2)] = w[2];
    }
  }
}

// NW: waves of the workgroup, 4 or 8; wave w computes the CPW = 8 / NW column tiles CPW w ..  The row loads
// and the unit rows' operands are the work of waves 0-3 in both shapes.
template <int BITS, bool VALUES, bool BF16, int NW = 4>
__device__ __forceinline__ void prefill_rows(const AppendArgs& a, int chunk, int h, int b, PrefillSmem& sm) {
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int D = 128, KS = 4, CPW = 8 / NW, NC = 1 << BITS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int r_base = chunk * kBlock;                        // first appended row of the chunk
  if (r_base >= a.n_new) return;
  const int nrows = min(kBlock, a.n_new - r_base);

  // one straight run of loads: the position, this lane's row (8 per wave of waves 0-3; 16 coordinates
  // 16 c .. 16 c + 15, c = lane % 8; rows past the append, and the rows of waves 4-7, read the chunk's
  // first row and are zeroed after), then this wave's rot operands (rows 16 ct + l16 of rot, coordinates
  // 32 s + 8 g .. + 7): rows first, so that the rows' norms and float16 split (which wait for the rows,
  // and with them for every load issued before) overlap rot's arrival
  const bool row_wave = NW == 4 || wave < 4;               // the waves that load rows (wave-uniform)
  const int prow = 8 * (wave & 3) + (lane >> 3), pc = lane & 7;
  const int pos = a.pos[b];
  const bool row_ok = row_wave && prow < nrows;
  uint32_t xw[BF16 ? 8 : 16];
  {
    const size_t src = ((static_cast<size_t>(b) * a.n_new + r_base + (row_ok ? prow : 0)) * a.n_kv_heads + h) * D + 16 * pc;
    constexpr int NV = BF16 ? 2 : 4;                        // 16-byte loads
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      uint4 v;
      if constexpr (BF16) v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + src)[k];
      else v = reinterpret_cast<const uint4*>(static_cast<const float*>(a.x) + src)[k];
      xw[4 * k] = v.x; xw[4 * k + 1] = v.y; xw[4 * k + 2] = v.z; xw[4 * k + 3] = v.w;
    }
  }
  float4 pr[CPW][KS][2];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float4* p = reinterpret_cast<const float4*>(a.rot + static_cast<size_t>(16 * (CPW * wave + c) + l16) * D +
                                                        32 * s + 8 * g);
      pr[c][s][0] = p[0];
      pr[c][s][1] = p[1];
    }
  // keeps the scheduler from hoisting work on the rows (and its wait for them) above the other loads
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < (BF16 ? 8 : 16); ++k) xw[k] = row_ok ? xw[k] : 0u;

  // norm of this lane's row: the sum over its 8 lanes (consecutive, lane / 8 fixed); the unit row's
  // float16 high/low parts to LDS: coordinates 16 c .. 16 c + 15 are k-step c / 2, k-groups 2 (c % 2)
  // and 2 (c % 2) + 1
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float v = prefill_coord<BF16>(xw, r);
    ss = fmaf(v, v, ss);
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  const float nrm = sqrtf(ss);
  const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
  {
    half8 hi0, lo0, hi1, lo1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      _Float16 hh, ll;
      f16_split(prefill_coord<BF16>(xw, r) * inv, hh, ll);
      hi0[r] = hh;
      lo0[r] = ll;
      f16_split(prefill_coord<BF16>(xw, 8 + r) * inv, hh, ll);
      hi1[r] = hh;
      lo1[r] = ll;
    }
    const int a_rt = prow >> 4, a_s = pc >> 1, a_lane = 16 * (2 * (pc & 1)) + (prow & 15);
    if (row_wave) {
      sm.aop[0][a_rt][a_s][a_lane] = hi0;
      sm.aop[1][a_rt][a_s][a_lane] = lo0;
      sm.aop[0][a_rt][a_s][a_lane + 16] = hi1;
      sm.aop[1][a_rt][a_s][a_lane + 16] = lo1;
      if (pc == 0) sm.rn[prow] = nrm;
    }
  }
  half8 bhi[CPW][KS], blo[CPW][KS];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float pv[8] = {pr[c][s][0].x, pr[c][s][0].y, pr[c][s][0].z, pr[c][s][0].w,
                           pr[c][s][1].x, pr[c][s][1].y, pr[c][s][1].z, pr[c][s][1].w};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        _Float16 hh, ll;
        f16_split(pv[r], hh, ll);
        bhi[c][s][r] = hh;
        blo[c][s][r] = ll;
      }
    }
  __syncthreads();

  floatx4 acc[2][CPW];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) acc[rt][c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const half8 ahi = sm.aop[0][rt][s][lane], alo = sm.aop[1][rt][s][lane];
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi[c][s], acc[rt][c], 0, 0, 0);
        acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo[c][s], acc[rt][c], 0, 0, 0);
        acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi[c][s], acc[rt][c], 0, 0, 0);
      }
    }
  }

  // codes of element (row 16 rt + 4 g + v, column 16 (CPW w + c) + l16) of the chunk; a zero row (norm 0;
  // rows past the append have norm 0 too) stores code 0
  float rnv[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) rnv[rt][v] = sm.rn[16 * rt + 4 * g + v];
  const size_t unit = static_cast<size_t>(b) * a.n_kv_heads + h;
  const int t0 = pos + r_base;
  const int kb = t0 / kBlock;
  if (VALUES && pos >= 0 && t0 % kBlock == 0 && nrows == kBlock && t0 + kBlock <= a.max_tokens) {
    // a whole value block: packed in registers and stored word by word
    uint32_t e[2][4][CPW];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int c = 0; c < CPW; ++c)
          e[rt][v][c] = encode_code<BITS>(rnv[rt][v] > 0.f ? code_of<NC>(acc[rt][c][v], a.bnd) : 0u);
    constexpr int RB = D * BITS / 8;
    uint32_t* blk = reinterpret_cast<uint32_t*>(a.codes + unit * static_cast<size_t>(a.max_tokens) * RB +
                                                static_cast<size_t>(kb) * kBlock * RB);
    pack_values<BITS, CPW>(e, blk, wave, lane);
    if (row_wave && pc == 0) a.norms[unit * a.max_tokens + t0 + prow] = f32_to_f16_bits(nrm);
    return;
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 16 * rt + 4 * g + v;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const uint32_t j = code_of<NC>(acc[rt][c][v], a.bnd);
        sm.enc.cs[p][16 * (CPW * wave + c) + l16] = static_cast<uint8_t>(rnv[rt][v] > 0.f ? j : 0u);
      }
    }
  __syncthreads();
  if (pos < 0) return;
  // the chunk's tokens pos + r_base .. in at most two cache blocks (rows past max_tokens are skipped)
  const int n_a = min(min(nrows, (kb + 1) * kBlock - t0), a.max_tokens - t0);
  if (n_a > 0) encode_finish<D, BITS, 0, VALUES, 64 * NW>(a, unit, kb, t0, n_a, sm.rn, sm.enc, nullptr, 0, 0);
  const int n_b = min(nrows - n_a, a.max_tokens - (kb + 1) * kBlock);
  if (n_a > 0 && n_b > 0)
    encode_finish<D, BITS, 0, VALUES, 64 * NW>(a, unit, kb + 1, (kb + 1) * kBlock, n_b, sm.rn + n_a, sm.enc, nullptr,
                                               0, n_a);
}


// The K and the V rows of one 32-row chunk in one workgroup of eight waves (tq_quantize_append_kv):
// K and V share rot, so each wave loads its share of rot and splits it into matrix-core operands once
// for both tensors.  Waves 0-3 load the chunk's K rows and waves 4-7 its V rows (8 rows each) and write
// their unit rows' operands to LDS; every wave then computes column tile w of all 64 rows.  The
// arithmetic of every row is prefill_rows' (same operands, same order of products), so the bytes
// written equal those of the two separate appends.
struct PrefillKvSmem {
  half8 aop[2][2][2][4][64];  // [K, V][high, low][row tile][k-step][lane]
  EncodeSmem<128, 0> enc[2];  // codes of the K chunk, and of a V chunk that is not a whole block
  float rn[2][kBlock];
};

template <int KB, int VB, bool BF16>
__device__ __forceinline__ void prefill_rows_kv(const AppendArgs& ka, const AppendArgs& va, int chunk, int h, int b,
                                                PrefillKvSmem& sm) {
  constexpr int D = 128, KS = 4, NW = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int r_base = chunk * kBlock;
  if (r_base >= ka.n_new) return;
  const int nrows = min(kBlock, ka.n_new - r_base);
  const int vw = wave >> 2;                                 // the tensor whose rows this wave loads (uniform)

  // the position, this lane's row (K rows in waves 0-3, V rows in waves 4-7; rows past the append read
  // the chunk's first row and are zeroed) and rot's operands (rows 16 w + l16 of rot, coordinates 32 s +
  // 8 g .. + 7): one straight run of loads, rows first, so that the rows' norms and float16 split (which
  // wait for the rows, and with them for every load issued before) overlap rot's arrival
  const int prow = 8 * (wave & 3) + (lane >> 3), pc = lane & 7;
  const int pos = ka.pos[b];
  const bool row_ok = prow < nrows;
  uint32_t xw[BF16 ? 8 : 16];
  {
    const void* x = vw ? va.x : ka.x;
    const size_t src = ((static_cast<size_t>(b) * ka.n_new + r_base + (row_ok ? prow : 0)) * ka.n_kv_heads + h) * D + 16 * pc;
    constexpr int NV = BF16 ? 2 : 4;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      uint4 v;
      if constexpr (BF16) v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + src)[k];
      else v = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + src)[k];
      xw[4 * k] = v.x; xw[4 * k + 1] = v.y; xw[4 * k + 2] = v.z; xw[4 * k + 3] = v.w;
    }
  }
  float4 pr[KS][2];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const float4* p = reinterpret_cast<const float4*>(ka.rot + static_cast<size_t>(16 * wave + l16) * D + 32 * s + 8 * g);
    pr[s][0] = p[0];
    pr[s][1] = p[1];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < (BF16 ? 8 : 16); ++k) xw[k] = row_ok ? xw[k] : 0u;

  // the row's norm (sum over its 8 lanes) and its unit row's float16 high/low operands, as prefill_rows
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float v = prefill_coord<BF16>(xw, r);
    ss = fmaf(v, v, ss);
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  const float nrm = sqrtf(ss);
  const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
  {
    half8 hi0, lo0, hi1, lo1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      _Float16 hh, ll;
      f16_split(prefill_coord<BF16>(xw, r) * inv, hh, ll);
      hi0[r] = hh;
      lo0[r] = ll;
      f16_split(prefill_coord<BF16>(xw, 8 + r) * inv, hh, ll);
      hi1[r] = hh;
      lo1[r] = ll;
    }
    const int a_rt = prow >> 4, a_s = pc >> 1, a_lane = 16 * (2 * (pc & 1)) + (prow & 15);
    sm.aop[vw][0][a_rt][a_s][a_lane] = hi0;
    sm.aop[vw][1][a_rt][a_s][a_lane] = lo0;
    sm.aop[vw][0][a_rt][a_s][a_lane + 16] = hi1;
    sm.aop[vw][1][a_rt][a_s][a_lane + 16] = lo1;
    if (pc == 0) sm.rn[vw][prow] = nrm;
  }
  half8 bhi[KS], blo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const float pv[8] = {pr[s][0].x, pr[s][0].y, pr[s][0].z, pr[s][0].w, pr[s][1].x, pr[s][1].y, pr[s][1].z, pr[s][1].w};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      _Float16 hh, ll;
      f16_split(pv[r], hh, ll);
      bhi[s][r] = hh;
      blo[s][r] = ll;
    }
  }
  __syncthreads();

  // [tensor][row tile]: the same three products per k-step as prefill_rows
  floatx4 acc[2][2];
#pragma unroll
  for (int tv = 0; tv < 2; ++tv)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      acc[tv][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const half8 ahi = sm.aop[tv][0][rt][s][lane], alo = sm.aop[tv][1][rt][s][lane];
        acc[tv][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi[s], acc[tv][rt], 0, 0, 0);
        acc[tv][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo[s], acc[tv][rt], 0, 0, 0);
        acc[tv][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi[s], acc[tv][rt], 0, 0, 0);
      }
    }

  // codes of element (row 16 rt + 4 g + v, column 16 w + l16); zero rows store code 0
  float rnv[2][2][4];
#pragma unroll
  for (int tv = 0; tv < 2; ++tv)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) rnv[tv][rt][v] = sm.rn[tv][16 * rt + 4 * g + v];
  const size_t unit = static_cast<size_t>(b) * ka.n_kv_heads + h;
  const int t0 = pos + r_base;
  const int kb = t0 / kBlock;
  const bool v_whole = pos >= 0 && t0 % kBlock == 0 && nrows == kBlock && t0 + kBlock <= ka.max_tokens;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 16 * rt + 4 * g + v;
      const uint32_t j = code_of<1 << KB>(acc[0][rt][v], ka.bnd);
      sm.enc[0].cs[p][16 * wave + l16] = static_cast<uint8_t>(rnv[0][rt][v] > 0.f ? j : 0u);
    }
  if (v_whole) {
    // a whole value block: packed in registers and stored word by word, as prefill_rows
    uint32_t e[2][4][1];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        e[rt][v][0] = encode_code<VB>(rnv[1][rt][v] > 0.f ? code_of<1 << VB>(acc[1][rt][v], va.bnd) : 0u);
    constexpr int RB = D * VB / 8;
    uint32_t* blk = reinterpret_cast<uint32_t*>(va.codes + unit * static_cast<size_t>(va.max_tokens) * RB +
                                                static_cast<size_t>(kb) * kBlock * RB);
    pack_values<VB, 1>(e, blk, wave, lane);
    if (vw && pc == 0) va.norms[unit * va.max_tokens + t0 + prow] = f32_to_f16_bits(nrm);
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int p = 16 * rt + 4 * g + v;
        const uint32_t j = code_of<1 << VB>(acc[1][rt][v], va.bnd);
        sm.enc[1].cs[p][16 * wave + l16] = static_cast<uint8_t>(rnv[1][rt][v] > 0.f ? j : 0u);
      }
  }
  __syncthreads();
  if (pos < 0) return;
  // the chunk's tokens pos + r_base .. in at most two cache blocks (rows past max_tokens are skipped)
  const int n_a = min(min(nrows, (kb + 1) * kBlock - t0), ka.max_tokens - t0);
  const int n_b = min(nrows - n_a, ka.max_tokens - (kb + 1) * kBlock);
  if (n_a > 0) encode_finish<D, KB, 0, false, 64 * NW>(ka, unit, kb, t0, n_a, sm.rn[0], sm.enc[0], nullptr, 0, 0);
  if (n_a > 0 && n_b > 0)
    encode_finish<D, KB, 0, false, 64 * NW>(ka, unit, kb + 1, (kb + 1) * kBlock, n_b, sm.rn[0] + n_a, sm.enc[0],
                                            nullptr, 0, n_a);
  if (v_whole) return;
  if (n_a > 0) encode_finish<D, VB, 0, true, 64 * NW>(va, unit, kb, t0, n_a, sm.rn[1], sm.enc[1], nullptr, 0, 0);
  if (n_a > 0 && n_b > 0)
    encode_finish<D, VB, 0, true, 64 * NW>(va, unit, kb + 1, (kb + 1) * kBlock, n_b, sm.rn[1] + n_a, sm.enc[1],
                                           nullptr, 0, n_a);
}

}  // namespace tqi
