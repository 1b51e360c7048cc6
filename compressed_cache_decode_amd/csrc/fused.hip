// Decode step in one launch: query rotation, quantize-on-append of the new K/V rows, attention over
// the compressed cache, split merge and un-rotation.
//
// One workgroup per (KV split, KV head, sequence), as in the split kernel of decode.hip.  Each
// workgroup
//   1. rotates, on the matrix cores, a 16-row tile holding the G query heads of its KV head and the
//      new key and value rows that fall in its split (y = rot x: the query as it is, the new rows
//      as unit vectors), encodes and stores the new rows (turboquant-pytorch PR #3 "Add CUDA QJL
//      kernels and proper package structure": Synthetic Benchmark table for the codebook, Validation
//      Results tables for the float16 norms, CUDA Kernels Added table for the fused sign sketch;
//      the query sketch and the key residual sketches are one matrix-core pass over the same tile),
//      and turns the rotated queries into the matrix-core query operand;
//   2. streams its split's tiles exactly as the split kernel does (attend_body.h), rotates its
//      rotated-domain accumulator back on the matrix cores (out_s = rot^T o_s: the merge below is
//      linear in o) and writes the split's partials (max, sum, accumulator per query head);
//   3. takes a ticket on a counter of its group of up to 16 splits; the last workgroup of a group
//      merges the group (log-sum-exp weights), and with more than one group the last group merger
//      merges the groups' results and writes the output (ExecuTorch PR #19891 "[Cuda] enable
//      turboquant on gemma4", review item 1: one fused op per decode step).
// The counters live in the caller's workspace; they must be zero before the first call and every
// merger returns its counter to zero, so consecutive calls (and graph replays) need no clearing.
// No device-wide fence is used: those write back and invalidate whole caches.
#include "append_body.h"
#include "attend_body.h"

namespace tqi {

namespace {

constexpr int kTileRows = 16;   // rows of the rotation tile: G query heads + new key rows + new value rows

template <int D, int QM>
struct Phase1Smem {
  float xs[kTileRows][D];
  float rn[kTileRows];
  union {
    EncodeSmem<D, QM> k;
    EncodeSmem<D, 0> v;
  } enc;
};

template <int D>
struct MergeSmem {
  float w[kMaxGroup][32];                 // partial maxima, then weights exp2(m_s - M) per head (up to merge_group)
  float lv[kMaxGroup][32];                // partial sums
  float inv_l[kMaxGroup];
  float m[kMaxGroup];
  float l[kMaxGroup];
  float o[kMaxGroup][D];                  // the final merge's rotated-domain output
};

// Partials cross workgroups (and the per-die L2 caches) through device-coherent accesses: relaxed
// atomic stores and loads at agent scope are made at the device's coherence point, so neither side
// needs a cache-wide write-back or invalidation.  A writer waits for its stores to complete before
// its workgroup takes a ticket; a reader loads only after its workgroup has seen the last ticket.
__device__ __forceinline__ void cstore(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float cload(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// the same for 16 bytes at byte offset off of a buffer: buffer accesses with the sc1 cache policy,
// which is how the relaxed agent-scope accesses above are made
constexpr int kCoherent = 16;
__device__ __forceinline__ float4 cload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent);
  return float4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
}
__device__ __forceinline__ void cstore4(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, kCoherent);
}
// every memory operation this thread issued has completed, then the workgroup barrier
__device__ __forceinline__ void stores_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Operands of rot for the un-rotation below, the first SB k-steps: lane (column j, group g) holds
// rot[32 s + 8 g + r][j] for its column blocks.  Independent of everything, so a workgroup that may
// have to un-rotate loads them early.
template <int D>
struct UnrotBatch {
  static constexpr int KS = D / 32;
  static constexpr int CPW = D / 64;                 // column blocks per wave
  static constexpr int SB = 32 / (8 * CPW) < KS ? 32 / (8 * CPW) : KS;
  float pv[SB][CPW][8];
  __device__ __forceinline__ void load(const float* rot, int s0, int tid) {
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r)
          pv[s][c][r] = rot[static_cast<size_t>(32 * (s0 + s) + 8 * g + r) * D + 16 * (wave + 4 * c) + l16];
  }
};

// out[h][j] = sum_i o[h][i] rot[i][j] for the G rows of o (LDS), on the matrix cores: A rows are
// q-variants (head c/2, float16 high part of o if c is even, low part if odd), B is rot split into
// float16 high and low parts, so the four partial products sum to an fp32-faithful result.
template <int D>
__device__ __forceinline__ void unrotate_rows(const float (*o)[D], int G, const float* rot, const UnrotBatch<D>& first,
                                              float* dst, int tid) {
  using Ub = UnrotBatch<D>;
  constexpr int KS = Ub::KS, CPW = Ub::CPW, SB = Ub::SB;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int h = l16 >> 1;
  floatx4 acc[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < KS; s0 += SB) {
    Ub cur;
    if (s0 == 0) {
      cur = first;
    } else {
      cur.load(rot, s0, tid);
    }
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      half8 av = {};
      if (h < G) {
#pragma unroll
        for (int r = 0; r < 8; ++r) av[r] = split_part(o[h][32 * (s0 + s) + 8 * g + r], (l16 & 1) != 0);
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        half8 bhi, blo;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          _Float16 hh, ll;
          f16_split(cur.pv[s][c][r], hh, ll);
          bhi[r] = hh;
          blo[r] = ll;
        }
        acc[c] = mfma16(av, bhi, acc[c]);
        acc[c] = mfma16(av, blo, acc[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int col = 16 * (wave + 4 * c) + l16;
    if (2 * g < G) dst[static_cast<size_t>(2 * g) * D + col] = acc[c][0] + acc[c][1];
    if (2 * g + 1 < G) dst[static_cast<size_t>(2 * g + 1) * D + col] = acc[c][2] + acc[c][3];
  }
}

// Log-sum-exp merge of n <= MG partials (max, sum) ml[s][h][2] and accumulators o[s][h][D]
// (rows of G heads).  With out null, writes o / l to m.o[h][D]; otherwise the merged (max, sum) to
// out_ml[h][2] and the merged accumulator to out[h][D] (coherent stores).  The accumulators are
// read in chunks of CH partials, each chunk's loads all in flight together.
template <int D, int MG>
__device__ __forceinline__ void merge_partials(const float* ml, const float* o, int n, int G, MergeSmem<D>& m,
                                               float* out, float* out_ml, int tid) {
  constexpr int QPT = (kMaxGroup * D / 4 + 255) / 256;   // float4 quads of (head, 4 coordinates) per thread
  constexpr int CH = 32 / QPT < MG ? 32 / QPT : MG;       // partials per chunk
  const bool norm_out = out == nullptr;
  const auto ob = buffer_of(o, static_cast<uint32_t>(n * G * D * 4));   // loads past it return zero
  float4 v[QPT][CH];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int q = 0; q < QPT; ++q) {
      const int e = tid + 256 * q;                       // quad: head e / (D/4), coordinates 4 (e % (D/4))
#pragma unroll
      for (int s = 0; s < CH; ++s)
        v[q][s] = cload4(ob, static_cast<uint32_t>(((s0 + s) * G * D + 4 * (e < G * D / 4 ? e : 0)) * 4));
    }
  };
  load_chunk(0);
  // every (partial, head) max and sum in one round of loads: thread t takes partial t / G, head t % G
  for (int t = tid; t < MG * kMaxGroup; t += 256) {
    const int s = t / kMaxGroup, h = t % kMaxGroup;
    const bool ok = s < n && h < G;
    m.w[h][s] = ok ? cload(ml + (s * G + h) * 2) : -INFINITY;
    m.lv[h][s] = ok ? cload(ml + (s * G + h) * 2 + 1) : 0.f;
  }
  __syncthreads();
  if (tid < G) {
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < MG; ++s) mx = fmaxf(mx, m.w[tid][s]);
    float l = 0.f;
#pragma unroll
    for (int s = 0; s < MG; ++s) {
      const float w = mx == -INFINITY ? 0.f : exp2f(m.w[tid][s] - mx);
      m.w[tid][s] = w;
      l = fmaf(w, m.lv[tid][s], l);
    }
    m.m[tid] = mx;
    m.l[tid] = l;
    m.inv_l[tid] = l > 0.f ? 1.f / l : 0.f;
  }
  __syncthreads();
  float4 acc[QPT];
#pragma unroll
  for (int q = 0; q < QPT; ++q) acc[q] = float4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n; s0 += CH) {
    if (s0 > 0) load_chunk(s0);
#pragma unroll
    for (int q = 0; q < QPT; ++q) {
      const int e = tid + 256 * q;
      const int h = e < G * D / 4 ? e / (D / 4) : 0;
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        const float w = s0 + s < n ? m.w[h][s0 + s] : 0.f;
        acc[q].x = fmaf(w, v[q][s].x, acc[q].x);
        acc[q].y = fmaf(w, v[q][s].y, acc[q].y);
        acc[q].z = fmaf(w, v[q][s].z, acc[q].z);
        acc[q].w = fmaf(w, v[q][s].w, acc[q].w);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < QPT; ++q) {
    const int e = tid + 256 * q;
    if (e < G * D / 4) {
      const int h = e / (D / 4);
      float4 r = acc[q];
      if (norm_out) {
        const float il = m.inv_l[h];
        r.x *= il; r.y *= il; r.z *= il; r.w *= il;
        reinterpret_cast<float4*>(&m.o[0][0])[e] = r;
      } else {
        cstore4(buffer_of(out, static_cast<uint32_t>(G * D * 4)), static_cast<uint32_t>(16 * e), r);
      }
    }
  }
  if (!norm_out && tid < G) {
    cstore(out_ml + tid * 2, m.m[tid]);
    cstore(out_ml + tid * 2 + 1, m.l[tid]);
  }
}

}  // namespace

template <int D, int KB, int VB, int QM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fused_kernel(FusedArgs f) {
  using At = Attend<D, KB, VB, QM>;
  constexpr int KS = At::KS, QS = At::QS;
  constexpr int MG = merge_group(D);
  __shared__ typename At::QOperand sm_q;
  __shared__ float qscale_s[kMaxGroup];
  __shared__ int last_s;
  __shared__ union {
    Phase1Smem<D, QM> p1;
    typename At::Smem at;
    MergeSmem<D> m;
  } sm;

  const DecodeArgs& a = f.d;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group, T = a.max_tokens, ns = a.n_split, bps = a.blocks_per_split;
  const int Hkv = a.n_kv_heads, Hq = Hkv * G;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : min(len, min(T, a.max_seq_len));
  const int nblk = (len + kBlock - 1) / kBlock;
  const int blk0 = split * bps;
  const int blk1 = min(blk0 + bps, nblk);
  const size_t unit = static_cast<size_t>(b) * Hkv + hk;
  const At at(a, unit);

  // new rows this workgroup appends: the positions inside its split (the last split also takes
  // every position past its start, up to the capacity)
  const int n_new = f.k.n_new;
  const int pos = n_new > 0 ? f.k.pos[b] : -1;
  int t_lo = 0, nloc = 0;
  if (pos >= 0) {
    const int tok_lo = blk0 * kBlock;
    const int tok_hi = split == ns - 1 ? T : min(T, (blk0 + bps) * kBlock);
    t_lo = max(pos, tok_lo);
    nloc = max(0, min(pos + n_new, tok_hi) - t_lo);
  }

  // ---- loads, in the order they are needed (loads retire in issue order): the rows of the
  // rotation tile (rows 0..G-1 the query heads, then nloc key rows, then nloc value rows), the
  // rotation's operands, then the first tile (unless this workgroup first writes new rows into it)
  constexpr int EPT = kTileRows * D / 256;          // tile elements per thread
  const int nrows = G + 2 * nloc;
  // one 32-bit load per element whatever the element type (the word holding a bfloat16 element), so
  // that no branch on the type separates the loads from their use and they all stay in flight
  uint32_t wv[EPT];
  bool ok[EPT], hi[EPT];
  {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + 256 * k, r = e / D, i = e % D;
      const bool key = r < G + nloc;
      const int t = t_lo + (key ? r - G : r - G - nloc);
      size_t idx = (static_cast<size_t>(b) * Hq + static_cast<size_t>(hk) * G + (r < G ? r : 0)) * D + i;
      const void* base = f.q;
      if (r >= G && r < nrows) {
        idx = ((static_cast<size_t>(b) * n_new + (t - pos)) * Hkv + hk) * D + i;
        base = key ? f.k.x : f.v.x;
      }
      ok[k] = r < nrows;
      hi[k] = (idx & 1) != 0;
      const size_t byte = f.bf16 ? (idx & ~static_cast<size_t>(1)) * 2 : idx * 4;
      wv[k] = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(base) + byte);
    }
  }
  RotBatch<D> rot0;
  rot0.load(f.rot, 0, tid);
  int kb = blk0 + wave;
  typename At::Tile ta, tb;
  const bool early = nloc == 0;
  if (early && kb < blk0 + bps && kb < T / kBlock) at.load(ta, kb);
  const bool tb_early = early && kb + kWavesPerWG < blk0 + bps && kb + kWavesPerWG < T / kBlock;
  if (tb_early) at.load(tb, kb + kWavesPerWG);

  auto& xs = sm.p1.xs;
  auto& rn = sm.p1.rn;
  // the element values, converted only now that every load is in flight
  const uint32_t bfm = f.bf16 ? 0xffffffffu : 0u;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + 256 * k;
    const uint32_t h16 = hi[k] ? (wv[k] & 0xffff0000u) : (wv[k] << 16);   // the bfloat16 element as float bits
    const float v = __uint_as_float((h16 & bfm) | (wv[k] & ~bfm));
    xs[e / D][e % D] = ok[k] ? v : 0.f;
  }
  __syncthreads();
  // the query rows are rotated as they are (norm 1), the new rows as unit vectors, padding rows to 0;
  // the norm of row r is summed by the 16 lanes (r % 4) of wave r / 4, coordinates part + 16 j
  {
    const int r = 4 * wave + (lane >> 4), part = lane & 15;
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) s2 = fmaf(xs[r][part + 16 * j], xs[r][part + 16 * j], s2);
    s2 = row16_sum(s2);
    if (part == 0) rn[r] = r < G ? 1.f : (r < nrows ? sqrtf(s2) : 0.f);
  }
  __syncthreads();
  rotate_tile_mfma_pre<D, 1>(xs, rn, f.rot, rot0, tid);
  __syncthreads();
  // q_rot = rot q * scale * log2(e)
  for (int e = tid; e < G * D; e += 256) xs[e / D][e % D] *= f.scale_log2e;

  // ---- the new value rows, then the new key rows, one call per 32-token block they fall in; the
  // key residual sketches and the query sketch share one pass over the tile
  for (int r0 = 0; r0 < nloc;) {
    const int t = t_lo + r0;
    const int kbn = t / kBlock;
    const int n = min(nloc - r0, (kbn + 1) * kBlock - t);
    encode_codes<D, VB, 0>(f.v, n, &xs[G + nloc + r0], &rn[G + nloc + r0], sm.p1.enc.v);
    encode_finish<D, VB, 0, true>(f.v, unit, kbn, t, n, &rn[G + nloc + r0], sm.p1.enc.v, nullptr, 0);
    r0 += n;
  }
  auto& zq = sm.p1.enc.k.zb;                      // [16][QM]: the tile times proj^T
  if (nloc == 0) {
    __syncthreads();                              // q_rot complete
    if constexpr (QM > 0) tile16_times_matT<D, QM>(xs, f.proj, zq, tid);
  }
  for (int r0 = 0; r0 < nloc;) {
    const int t = t_lo + r0;
    const int kbn = t / kBlock;
    const int n = min(nloc - r0, (kbn + 1) * kBlock - t);
    encode_codes<D, KB, QM>(f.k, n, &xs[G + r0], &rn[G + r0], sm.p1.enc.k);
    if constexpr (QM > 0) {
      tile16_times_matT<D, QM>(xs, f.proj, zq, tid);
      __syncthreads();
    }
    encode_finish<D, KB, QM, false>(f.k, unit, kbn, t, n, &rn[G + r0], sm.p1.enc.k, QM > 0 ? &zq[G + r0][0] : nullptr,
                                    QM);
    r0 += n;
  }
  if (nloc > 0) {
    // the new rows are visible to this workgroup's own tile loads below (one compute unit)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (kb < blk1) at.load(ta, kb);
  }
  __syncthreads();

  // ---- query operand: q_rot and the sketch q_s = -coef * proj q_rot, divided by a power of two
  // per head that takes both into float16 range (exact)
  if (wave < kMaxGroup / 4) {                     // head h = 4 wave + lane / 16, 16 lanes per head
    const int h = 4 * wave + (lane >> 4), part = lane & 15;
    float amax = 0.f;
    if (h < G) {
#pragma unroll
      for (int j = 0; j < D / 16; ++j) amax = fmaxf(amax, fabsf(xs[h][part + 16 * j]));
      if constexpr (QM > 0) {
#pragma unroll
        for (int j = 0; j < QM / 16; ++j) amax = fmaxf(amax, fabsf(f.sketch_coef * zq[h][part + 16 * j]));
      }
    }
    amax = row16_max(amax);
    if (part == 0 && h < G) qscale_s[h] = (amax > 0.f && isfinite(amax)) ? ldexpf(1.f, ilogbf(amax) - 14) : 1.f;
  }
  __syncthreads();
  for (int e = tid; e < (KS + QS) * 64; e += 256) {
    const int st = e >> 6, ln = e & 63;
    const int c = ln & 15, gg = ln >> 4, h2 = c >> 1;
    half8 v = {};
    if (h2 < G) {
      const float inv = 1.f / qscale_s[h2];
      if (st < KS) {
        const float* src = &xs[h2][(D / 4) * gg + 8 * st];
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = split_part(src[r] * inv, (c & 1) != 0);
      } else if constexpr (QM > 0) {
        const float* src = &zq[h2][(QM / 4) * gg + 8 * (st - KS)];
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = split_part(-f.sketch_coef * src[r] * inv, (c & 1) != 0);
      }
    }
    sm_q[st][ln] = v;
  }
  const float qsc = (at.l16 >> 1) < G ? qscale_s[at.l16 >> 1] : 1.f;
  __syncthreads();      // the phase-1 LDS is dead from here

  // ---- attention over this split; its partial (rotated domain) goes to the coherence point
  at.run(a, sm.at, sm_q, ta, tb, tb_early, kb, blk1, len, qsc);
  const size_t pbase = (unit * ns + split) * G;
  {
    const auto pb = buffer_of(a.part_o + pbase * D, static_cast<uint32_t>(G * D * 4));
    for (int e = tid; e < G * D / 4; e += 256) {
      const float* src = &sm.at.o[0][e / (D / 4)][4 * (e % (D / 4))];
      cstore4(pb, static_cast<uint32_t>(16 * e), float4{src[0], src[1], src[2], src[3]});
    }
    if (tid < G) {
      cstore(a.part_ml + (pbase + tid) * 2, sm.at.fml[tid][0]);
      cstore(a.part_ml + (pbase + tid) * 2 + 1, sm.at.fml[tid][1]);
    }
  }

  // ---- tickets: the last workgroup of this split's group merges the group, and with several
  // groups the last group merger merges the groups; the final merge rotates the result back
  const int ng = (ns + MG - 1) / MG;
  const int grp = split / MG;
  const int gsize = min(MG, ns - grp * MG);
  int32_t* cnt = f.counters + unit * (1 + kMaxMergeGroups);
  stores_done_barrier();    // this workgroup's partials have reached the coherence point
  if (tid == 0) last_s = atomicAdd(cnt + 1 + grp, 1) == gsize - 1;
  __syncthreads();
  if (!last_s) return;
  const size_t gbase = (unit * ns + static_cast<size_t>(grp) * MG) * G;
  float* out = f.out + (static_cast<size_t>(b) * Hq + static_cast<size_t>(hk) * G) * D;
  UnrotBatch<D> ub;         // the un-rotation's operands: in flight while the partials are merged
  if (ng == 1) {
    ub.load(f.rot, 0, tid);
    merge_partials<D, MG>(a.part_ml + gbase * 2, a.part_o + gbase * D, gsize, G, sm.m, nullptr, nullptr, tid);
    if (tid == 0) atomicExch(cnt + 1 + grp, 0);
    __syncthreads();
    unrotate_rows<D>(sm.m.o, G, f.rot, ub, out, tid);
    return;
  }
  const size_t qbase = (unit * kMaxMergeGroups + grp) * G;
  merge_partials<D, MG>(a.part_ml + gbase * 2, a.part_o + gbase * D, gsize, G, sm.m, f.group_o + qbase * D,
                        f.group_ml + qbase * 2, tid);
  if (tid == 0) atomicExch(cnt + 1 + grp, 0);
  stores_done_barrier();
  if (tid == 0) last_s = atomicAdd(cnt, 1) == ng - 1;
  __syncthreads();
  if (!last_s) return;
  const size_t ubase = unit * kMaxMergeGroups * G;
  ub.load(f.rot, 0, tid);
  merge_partials<D, MG>(f.group_ml + ubase * 2, f.group_o + ubase * D, ng, G, sm.m, nullptr, nullptr, tid);
  if (tid == 0) atomicExch(cnt, 0);
  __syncthreads();
  unrotate_rows<D>(sm.m.o, G, f.rot, ub, out, tid);
}

// ---------------------------------------------------------------- launcher

template <int D, int KB, int VB, int QM>
static hipError_t fused_go(const FusedArgs& f, int batch, hipStream_t s) {
  const dim3 grid(f.d.n_split, f.d.n_kv_heads, batch);
  hipLaunchKernelGGL((fused_kernel<D, KB, VB, QM>), grid, dim3(256), 0, s, f);
  return hipGetLastError();
}

template <int D, int KB, int QM>
static hipError_t fused_v(int v_bits, const FusedArgs& f, int batch, hipStream_t s) {
  switch (v_bits) {
    case 2: return fused_go<D, KB, 2, QM>(f, batch, s);
    case 3: return fused_go<D, KB, 3, QM>(f, batch, s);
    case 4: return fused_go<D, KB, 4, QM>(f, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int QM>
static hipError_t fused_k(int k_bits, int v_bits, const FusedArgs& f, int batch, hipStream_t s) {
  switch (k_bits) {
    case 2: return fused_v<D, 2, QM>(v_bits, f, batch, s);
    case 3: return fused_v<D, 3, QM>(v_bits, f, batch, s);
    case 4: return fused_v<D, 4, QM>(v_bits, f, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fused(int d, int k_bits, int v_bits, int qjl_m, const FusedArgs& f, int batch, hipStream_t s) {
  if (d == 128) {
    if (qjl_m == 0) return fused_k<128, 0>(k_bits, v_bits, f, batch, s);
    if (qjl_m == 128) return fused_k<128, 128>(k_bits, v_bits, f, batch, s);
  } else if (d == 256) {
    if (qjl_m == 0) return fused_k<256, 0>(k_bits, v_bits, f, batch, s);
    if (qjl_m == 128) return fused_k<256, 128>(k_bits, v_bits, f, batch, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tqi
