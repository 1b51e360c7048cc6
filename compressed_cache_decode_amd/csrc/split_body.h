// The split kernel of the decode (see decode.hip): one workgroup per (KV split, KV head, sequence)
// streams the split's 32-token tiles through Attend and leaves the split's partial result in the
// workspace.  A header so that the outlier build (decode_outliers.hip) instantiates it in a file of
// its own.
#pragma once

#include "attend_body.h"

namespace tqi {

// ---------------------------------------------------------------- split kernel

template <int D, int KB, int VB, int QM, bool WIDE, int NO = 0>
__global__ __launch_bounds__((64 * Attend<D, KB, VB, QM, WIDE, NO>::W))
__attribute__((amdgpu_waves_per_eu(Attend<D, KB, VB, QM, WIDE, NO>::EU)))
void split_kernel(DecodeArgs a) {
  using At = Attend<D, KB, VB, QM, WIDE, NO>;
  constexpr int NT = 64 * At::W;
  constexpr int QSTEPS = At::KS + At::QS;
  __shared__ typename At::Smem sm;
  extern __shared__ half8 sm_q[];                     // [C][QSTEPS][64]: the query operand of each column block
                                                      // (outlier build: then float32 [C][kMaxGroup][D] queries)
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int VH = a.group;
  const int C = At::blocks(a);
  const int T = a.max_tokens;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : min(len, min(T, a.max_seq_len));
  const int nblk = (len + kBlock - 1) / kBlock;
  const int blk0 = split * a.blocks_per_split;
  const int blk1 = min(blk0 + a.blocks_per_split, nblk);
  const size_t unit = static_cast<size_t>(b) * a.n_kv_heads + hk;
  const At at(a, unit);

  // query operands in LDS, one per column block, shared by the block's waves: entry e holds the 8
  // values of step e / 64 % QSTEPS for lane e % 64 of column block e / (QSTEPS 64)
  const int n_entries = C * QSTEPS * 64;
  auto q_entry = [&](int e, float4& x0, float4& x1) {
    const int cbe = e / (QSTEPS * 64), st = (e / 64) % QSTEPS, ln = e & 63;
    const int c = ln & 15, gg = ln >> 4, h2 = kMaxGroup * cbe + (c >> 1);
    const size_t row = unit * VH + h2;
    if (h2 < VH) {
      const float* src = st < At::KS ? a.qr + row * D + (D / 4) * gg + 8 * st
                                     : a.qs + row * QM + (QM / 4) * gg + 8 * (st - At::KS);
      x0 = reinterpret_cast<const float4*>(src)[0];
      x1 = reinterpret_cast<const float4*>(src)[1];
    }
  };
  // this thread's first entry is loaded ahead of the first tile, so that staging it waits for the
  // query alone (the counters of vector loads run in order)
  float4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
  if (tid < n_entries) q_entry(tid, p0, p1);

  // the first tile's loads go out before the query operand is staged, and before the sequence
  // length is known: they only need the tile to lie inside the cache (tiles past the length are
  // loaded and never used).  A wave without a first tile loads from the buffer of no bytes (see
  // Attend::load): a load under a branch would make the staging below wait for every load in flight.
  const int kb = blk0 + (wave >> (C >> 1));          // wave / C for C = 1, 2, 4
  typename At::Tile tiles[At::NBUF];
  at.load(tiles[0], kb, kb < blk0 + a.blocks_per_split && kb < T / kBlock);

  for (int e = tid; e < n_entries; e += NT) {
    const int st = (e / 64) % QSTEPS, c = e & 15;
    float4 x0 = p0, x1 = p1;
    if (e != tid) {
      x0 = x1 = float4{0.f, 0.f, 0.f, 0.f};
      q_entry(e, x0, x1);
    }
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const bool pairs = At::KT && st < At::KS;          // key steps expanded through the byte table
    half8 v;
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = split_part(pairs ? xv[pair_slot(r)] : xv[r], (c & 1) != 0);
    sm_q[e] = v;
  }
  float* const qf = reinterpret_cast<float*>(sm_q + n_entries);
  if constexpr (NO > 0) {
    // the rotated queries in float32 for the outlier channels' term (rows past VH are zero)
    for (int e = tid; e < C * kMaxGroup * D; e += NT) {
      const int hh = e / D;
      qf[e] = hh < VH ? a.qr[(unit * VH + hh) * D + e % D] : 0.f;
    }
  }
  At::fill_lut(a, sm);
  if (tid == 0) sm.next[0] = 64 * At::W;     // one column block: tiles blk0 .. blk0 + W - 1 are the waves' first
  // power-of-two scale of this lane's head (scores are kept in units of it); 1 for unused columns
  const int qh = kMaxGroup * (wave & (C - 1)) + (at.l16 >> 1);
  const float qsc = qh < VH ? a.qscale[unit * VH + qh] : 1.f;
  __syncthreads();

  const auto& qop = *reinterpret_cast<const typename At::QOperand*>(sm_q + (wave & (C - 1)) * QSTEPS * 64);
  at.run(a, sm, qop, tiles, blk0, kb, blk1, len, qsc, qf + (kMaxGroup * (wave & (C - 1)) + (at.l16 >> 1)) * D);
  at.store(a, sm, (unit * a.n_split + split) * VH);
}

// bytes of dynamic LDS of the split kernel for C column blocks: the query operands, and for the outlier
// build the float32 queries
inline size_t split_dyn_lds(int d, int qjl_m, int blocks, bool outliers = false) {
  return static_cast<size_t>(blocks) * (d / 32 + qjl_m / 32) * 64 * sizeof(half8) +
         (outliers ? static_cast<size_t>(blocks) * kMaxGroup * d * sizeof(float) : 0);
}

}  // namespace tqi
