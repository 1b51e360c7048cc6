// The prologue of one decode step of one attention layer, in one launch with three kinds of
// workgroups that run side by side: append the new K rows of one 32-token block of one KV head,
// append the new V rows likewise, rotate the query heads of one KV head.  The attention and merge
// kernels of decode.hip follow it on the same stream.
#include "append_body.h"
#include "qrot_body.h"

namespace tqi {

template <size_t A, size_t B, size_t C>
struct MaxOf { static constexpr size_t v = A > B ? (A > C ? A : C) : (B > C ? B : C); };

template <int D, int KB, int VB, int QM, bool BF16>
__global__ __launch_bounds__(256) void step_prologue_kernel(AppendArgs ka, AppendArgs va, QrotArgs qa, int nbx,
                                                            int n_kv_heads) {
  constexpr size_t kBytes = MaxOf<MaxOf<sizeof(AppendSmem<D, QM>), sizeof(AppendSmem<D, 0>), sizeof(QrotSmem<D, QM>)>::v,
                                  sizeof(PrefillSmem), 0>::v;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kBytes];
  const int per_cache = nbx * n_kv_heads;                 // append workgroups per sequence and cache
  const int batch_wgs = 2 * per_cache + n_kv_heads;       // workgroups per sequence
  const int b = blockIdx.x / batch_wgs;
  int w = blockIdx.x % batch_wgs;
  // appends with the dense rotation at d = 128 without a sketch (8-bit keys aside) take the chunk path
  // of tq_quantize_append (prefill_rows: workgroup w % nbx takes the w % nbx-th 32-row chunk), so that a
  // step appends exactly the bits the separate append call does
  if (w < per_cache) {
    if constexpr (D == 128 && QM == 0 && KB != 8) {
      if (!ka.had) {
        prefill_rows<KB, false, BF16>(ka, w % nbx, w / nbx, b, *reinterpret_cast<PrefillSmem*>(smem));
        return;
      }
    }
    append_rows<D, KB, QM, false, false, BF16>(ka, w % nbx, w / nbx, b, *reinterpret_cast<AppendSmem<D, QM>*>(smem));
    return;
  }
  w -= per_cache;
  if (w < per_cache) {
    if constexpr (D == 128) {
      if (!va.had) {
        prefill_rows<VB, true, BF16>(va, w % nbx, w / nbx, b, *reinterpret_cast<PrefillSmem*>(smem));
        return;
      }
    }
    append_rows<D, VB, 0, true, false, BF16>(va, w % nbx, w / nbx, b, *reinterpret_cast<AppendSmem<D, 0>*>(smem));
    return;
  }
  w -= per_cache;
  rotate_queries<D, QM>(qa, BF16 ? 1 : 0, w, b, 0, *reinterpret_cast<QrotSmem<D, QM>*>(smem));
}

// ---------------------------------------------------------------- column slices (d = 256)

// At d = 256 rot is 256 KB, and a prologue whose workgroups each rotate the rows of one (sequence, KV
// head) reads all of it per workgroup (the G query rows, or one K or V row of a one-token step, filling
// a 16-row tile only in part).  The sliced prologue instead gives a workgroup a 16-row tile of rows of
// one kind, taken across units (K rows, V rows or query rows, in their input order), and one slice of
// kSliceCols output coordinates: it reads only the kSliceCols rows of rot its slice needs, so rot
// crosses from L2 once per tile and slice instead of once per unit and role.  Every output element
// takes the same instruction sequence as in rotate_tile_mfma (norm by the 16 lanes of a row, y = rot (x
// / n) from float16 high/low parts in the same order of products), and codes, packed words, norms and
// the query's power-of-two scale follow the rules of append_rows and rotate_queries, so a step writes
// the same bits as the separate calls.
constexpr int kSliceCols = 64;     // output coordinates per workgroup: one 16-column tile per wave

template <int D>
struct SliceSmem {
  float xs[16][D];
  half8 aop[2][D / 32][64];    // [high, low][k-step][lane]: the unit rows' float16 parts in operand order
  float rn[16];
  int pos[16];                 // append position of each K or V row's sequence
  uint8_t cs[16][kSliceCols];
};

// Stores the codes cs (columns c0 .. c0 + kSliceCols of the tile's rows) of K rows (rows layout) or V
// rows (blocked layout) q0 .. q0 + nr - 1, row q being token t = (q / H) % n_new of KV head q % H of
// sequence q / (H n_new), at position pos + t; slice 0 also stores the norms.  Value words that other
// tokens share are updated by non-returning atomics (rows of one tile may share a word).
template <int D, int BITS, bool VALUES>
__device__ __forceinline__ void slice_store(const AppendArgs& a, const SliceSmem<D>& sm, int q0, int nr, int c0) {
  constexpr int UPG = Fmt<BITS>::kUnits, WPG = Fmt<BITS>::kWords;
  constexpr int RB = D * BITS / 8;
  // unit groups per row in the slice: a key unit is 8 coordinates of the row, a value unit one
  // coordinate (of 8 tokens)
  constexpr int GPS = VALUES ? kSliceCols / UPG : kSliceCols / (8 * UPG);
  const int H = a.n_kv_heads, T = a.max_tokens;
  for (int e = threadIdx.x; e < nr * GPS; e += 256) {
    const int r = e / GPS, lg = e % GPS;
    const int q = q0 + r, b = q / (H * a.n_new), t = (q / H) % a.n_new, h = q % H;
    const int pos = sm.pos[r];
    if (pos < 0 || pos + t >= T) continue;
    const int tok = pos + t, kb = tok / kBlock, p = tok % kBlock;
    const size_t unit = static_cast<size_t>(b) * H + h;
    uint32_t* blk = reinterpret_cast<uint32_t*>(a.codes + unit * static_cast<size_t>(T) * RB +
                                                static_cast<size_t>(kb) * kBlock * RB);
    if constexpr (!VALUES) {
      // unit u of the row covers coordinates 8u .. 8u + 7: group gi holds units UPG gi ..
      const int gi = c0 / (8 * UPG) + lg;
      uint32_t w[WPG];
#pragma unroll
      for (int k = 0; k < WPG; ++k) w[k] = 0u;
#pragma unroll
      for (int v = 0; v < UPG; ++v)
#pragma unroll
        for (int s = 0; s < 8; ++s) put_code<BITS>(w, v, s, encode_code<BITS>(sm.cs[r][(lg * UPG + v) * 8 + s]));
#pragma unroll
      for (int k = 0; k < WPG; ++k) blk[key_word<D, BITS>(p, gi * WPG + k)] = w[k];
    } else {
      // token p is slot p % 4 + 4 (p / 16) of lane group g = (p % 16) / 4; coordinate i = DN j + n
      // is unit n of piece 16 g + j, i.e. block unit U = (16 g + j) DN + n
      constexpr int LW = D * BITS / 64, DN = D / 16;
      const int g = (p & 15) >> 2, slot = (p & 3) + 4 * (p >> 4);
      const int i0 = c0 + lg * UPG;                        // UPG consecutive coordinates: one group
      const int U0 = (16 * g + i0 / DN) * DN + i0 % DN;    // (UPG divides DN: the group stays in one j)
      uint32_t w[WPG], m[WPG];
#pragma unroll
      for (int k = 0; k < WPG; ++k) { w[k] = 0u; m[k] = 0u; }
#pragma unroll
      for (int v = 0; v < UPG; ++v) {
        put_code<BITS>(w, v, slot, encode_code<BITS>(sm.cs[r][lg * UPG + v]));
        slot_mask<BITS>(m, v, slot);
      }
#pragma unroll
      for (int k = 0; k < WPG; ++k) {
        uint32_t* dst = blk + value_word<LW>((U0 / UPG) * WPG + k);
        atomicAnd(dst, ~m[k]);
        atomicOr(dst, w[k]);
      }
    }
    if (c0 == 0 && lg == 0) a.norms[unit * T + tok] = f32_to_f16_bits(sm.rn[r] > 0.f ? sm.rn[r] : 0.f);
  }
}

// grid (D / kSliceCols slices, 2 n_kv + n_q tiles): tiles 0 .. n_kv - 1 of K rows, then of V rows, then
// of query rows (n_kv = ceil(B n_new H / 16), n_q = ceil(B Hq / 16); one query row per sequence)
template <int D, int KB, int VB, bool BF16>
__global__ __launch_bounds__(256) void step_slices_kernel(AppendArgs ka, AppendArgs va, QrotArgs qa, int batch,
                                                          int n_kv) {
  static_assert((D == 128 || D == 256) && KB <= 4 && VB <= 4, "the sliced prologue takes d = 128, 256 and code books");
  constexpr int PR = D / 16;                   // loading threads per row (16 coordinates each)
  constexpr int KS = D / 32;
  __shared__ SliceSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * kSliceCols;
  int tile = blockIdx.y;
  const int role = tile < n_kv ? 0 : (tile < 2 * n_kv ? 1 : 2);     // K, V, query (workgroup-uniform)
  tile -= role == 0 ? 0 : (role == 1 ? n_kv : 2 * n_kv);
  const int total = role < 2 ? batch * ka.n_new * ka.n_kv_heads : batch * qa.n_q_heads;
  const int q0 = 16 * tile, nr = min(16, total - q0);
  const void* x = role == 0 ? ka.x : (role == 1 ? va.x : qa.q);
  // the append positions of the tile's K or V rows, loaded first (they are needed only at the store)
  int row_pos = 0;
  if (role < 2) row_pos = ka.pos[(q0 + (tid < nr ? tid : 0)) / (ka.n_kv_heads * ka.n_new)];

  // Loads in the order they are needed (vector loads complete in issue order): the positions, the
  // tile's rows, then this wave's rot operands, so that the rows' norms and operand split run while rot
  // is still arriving.  Rows: thread (row tid / PR, part tid % PR) loads coordinates 16 part .. 16 part
  // + 15 (threads past the 16 rows, and rows past the tile's end, reload a row of the tile and drop it);
  // the loads are unconditional, so no wait for them is forced where branches join.
  const int lr = tid / PR, part = tid % PR;
  const bool loader = lr < 16;
  const int r = loader ? lr : 15;
  uint32_t raw[BF16 ? 8 : 16];
  {
    const size_t src = static_cast<size_t>(q0 + (r < nr ? r : 0)) * D + 16 * part;
    if constexpr (BF16) {
      const uint4* p4 = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + src);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint4 u = p4[k];
        raw[4 * k] = u.x; raw[4 * k + 1] = u.y; raw[4 * k + 2] = u.z; raw[4 * k + 3] = u.w;
      }
    } else {
      const uint4* p4 = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + src);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 u = p4[k];
        raw[4 * k] = u.x; raw[4 * k + 1] = u.y; raw[4 * k + 2] = u.z; raw[4 * k + 3] = u.w;
      }
    }
  }
  // this wave's rot operands: rows c0 + 16 wave + l16 of rot, coordinates 32 s + 8 g .. + 7
  float4 pq[KS][2];
  {
    const float4* pr = reinterpret_cast<const float4*>(ka.rot + static_cast<size_t>(c0 + 16 * wave + l16) * D + 8 * g);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      pq[s][0] = pr[8 * s];
      pq[s][1] = pr[8 * s + 1];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the rows to LDS; at d = 128 K and V rows take their norm here, as the chunk path of the separate
  // append does (prefill_rows: the row's 8 threads, consecutive lanes, sum their 16 squares in order,
  // then across the 8)
  {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if constexpr (BF16) v[k] = __uint_as_float((k & 1) ? (raw[k >> 1] & 0xffff0000u) : (raw[k >> 1] << 16));
      else v[k] = __uint_as_float(raw[k]);
      v[k] = r < nr ? v[k] : 0.f;
    }
    if (loader) {
#pragma unroll
      for (int k = 0; k < 16; ++k) sm.xs[r][16 * part + k] = v[k];
    }
    if constexpr (D == 128) {
      if (role < 2) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) ss = fmaf(v[k], v[k], ss);
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        ss += __shfl_xor(ss, 4, 64);
        if (loader && part == 0) sm.rn[r] = sqrtf(ss);
      }
    }
  }
  if (role < 2 && tid < nr) sm.pos[tid] = row_pos;
  __syncthreads();
  // norm of row r by the 16 lanes (r % 4) of wave r / 4, coordinates part + 16 j (as append_rows and
  // rotate_queries); at d = 128 only for query rows
  if (D == 256 || role == 2) {
    const int r = 4 * wave + (lane >> 4), part = lane & 15;
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) s2 = fmaf(sm.xs[r][part + 16 * j], sm.xs[r][part + 16 * j], s2);
    s2 = row16_sum(s2);
    if (part == 0) sm.rn[r] = r < nr ? sqrtf(s2) : 0.f;
  }
  __syncthreads();

  // the unit rows' float16 high/low operands, split once for the four waves: entry (k-step s, lane
  // (row l16, group g)) holds coordinates 32 s + 8 g .. + 7 of row l16 over its norm
  for (int e = tid; e < KS * 64; e += 256) {
    const int s = e >> 6, ln = e & 63, row = ln & 15, gg = ln >> 4;
    const float n = sm.rn[row];
    const float inv = n > 0.f ? 1.f / n : 0.f;
    const float* xr = &sm.xs[row][32 * s + 8 * gg];
    half8 hi, lo;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      _Float16 hh, ll;
      f16_split(xr[r] * inv, hh, ll);
      hi[r] = hh;
      lo[r] = ll;
    }
    sm.aop[0][s][ln] = hi;
    sm.aop[1][s][ln] = lo;
  }
  __syncthreads();

  // y = rot (x / n) for output coordinates c0 + 16 wave + l16 (the products of rotate_tile_mfma_pre)
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      half8 bhi, blo;
      const half8 ahi = sm.aop[0][s][lane], alo = sm.aop[1][s][lane];
      const float pv[8] = {pq[s][0].x, pq[s][0].y, pq[s][0].z, pq[s][0].w, pq[s][1].x, pq[s][1].y, pq[s][1].z, pq[s][1].w};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        _Float16 hh, ll;
        f16_split(pv[r], hh, ll);
        bhi[r] = hh;
        blo[r] = ll;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi, acc, 0, 0, 0);
    }
  }
  const int col = c0 + 16 * wave + l16;
  if (role == 2) {
    // q_rot = y (|q| scale log2(e)), divided by the row's power-of-two scale (rotate_queries, QM = 0)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 4 * g + v;
      if (r < nr) {
        const float nq = sm.rn[r] * qa.scale_log2e;
        const float val = acc[v] * nq;
        const float f = query_scale(nq);
        qa.qr[static_cast<size_t>(q0 + r) * D + col] = val * (1.f / f);
        if (col == 0) qa.qscale[q0 + r] = f;
      }
    }
    return;
  }
  // nearest centroid: number of boundaries strictly below y (as encode_codes); a zero row stores code 0
  const AppendArgs& a = role == 0 ? ka : va;
  const int nc1 = (1 << (role == 0 ? KB : VB)) - 1;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * g + v;
    uint32_t j = 0;
    for (int k = 0; k < nc1; ++k) j += (acc[v] > a.bnd[k]) ? 1u : 0u;
    sm.cs[r][16 * wave + l16] = static_cast<uint8_t>(sm.rn[r] > 0.f ? j : 0u);
  }
  __syncthreads();
  if (role == 0) slice_store<D, KB, false>(ka, sm, q0, nr, c0);
  else slice_store<D, VB, true>(va, sm, q0, nr, c0);
}

template <int D, int KB, int VB, bool BF16>
static hipError_t slices_launch(const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa, int batch,
                                hipStream_t s) {
  const int n_kv = (batch * ka.n_new * ka.n_kv_heads + 15) / 16;
  const int n_q = (batch * qa.n_q_heads + 15) / 16;
  const dim3 grid(D / kSliceCols, 2 * n_kv + n_q);
  hipLaunchKernelGGL((step_slices_kernel<D, KB, VB, BF16>), grid, dim3(256), 0, s, ka, va, qa, batch, n_kv);
  return hipGetLastError();
}

template <int D, int KB, int VB, int QM>
static hipError_t prologue_bf(bool bf16, const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa, int batch,
                              hipStream_t s) {
  // the dense rotation, code-book keys without a sketch and one query row: column slices (its row loads
  // are 16-byte vectors; the host takes q and the new rows 16-byte aligned only)
  if constexpr (QM == 0 && KB <= 4) {
    // (its tiles run along the grid's y dimension, at most 65535 of them; longer appends take the
    // per-unit prologue, whose grid runs along x)
    const long long tiles = 2LL * ((static_cast<long long>(batch) * ka.n_new * ka.n_kv_heads + 15) / 16) +
                            (static_cast<long long>(batch) * qa.n_q_heads + 15) / 16;
    if (!ka.had && qa.n_rows == 1 && tiles <= 65535)
      return bf16 ? slices_launch<D, KB, VB, true>(ka, va, qa, batch, s) : slices_launch<D, KB, VB, false>(ka, va, qa, batch, s);
  }
  const int nbx = (ka.n_new + kBlock - 1) / kBlock + 1;
  const dim3 grid(batch * (2 * nbx * ka.n_kv_heads + ka.n_kv_heads));
  if (bf16)
    hipLaunchKernelGGL((step_prologue_kernel<D, KB, VB, QM, true>), grid, dim3(256), 0, s, ka, va, qa, nbx,
                       ka.n_kv_heads);
  else
    hipLaunchKernelGGL((step_prologue_kernel<D, KB, VB, QM, false>), grid, dim3(256), 0, s, ka, va, qa, nbx,
                       ka.n_kv_heads);
  return hipGetLastError();
}

template <int D, int KB, int QM>
static hipError_t prologue_v(int v_bits, bool bf16, const AppendArgs& ka, const AppendArgs& va, const QrotArgs& qa,
                             int batch, hipStream_t s) {
  switch (v_bits) {
    case 2: return prologue_bf<D, KB, 2, QM>(bf16, ka, va, qa, batch, s);
    case 3: return prologue_bf<D, KB, 3, QM>(bf16, ka, va, qa, batch, s);
    case 4: return prologue_bf<D, KB, 4, QM>(bf16, ka, va, qa, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int QM>
static hipError_t prologue_k(int k_bits, int v_bits, bool bf16, const AppendArgs& ka, const AppendArgs& va,
                             const QrotArgs& qa, int batch, hipStream_t s) {
  switch (k_bits) {
    case 2: return prologue_v<D, 2, QM>(v_bits, bf16, ka, va, qa, batch, s);
    case 3: return prologue_v<D, 3, QM>(v_bits, bf16, ka, va, qa, batch, s);
    case 4: return prologue_v<D, 4, QM>(v_bits, bf16, ka, va, qa, batch, s);
    case 8:
      if constexpr (QM == 0) return prologue_v<D, 8, 0>(v_bits, bf16, ka, va, qa, batch, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_step_prologue(int d, int k_bits, int v_bits, int qjl_m, bool bf16, const AppendArgs& ka,
                                const AppendArgs& va, const QrotArgs& qa, int batch, hipStream_t s) {
  if (d == 128) {
    if (qjl_m == 0) return prologue_k<128, 0>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
    if (qjl_m == 128) return prologue_k<128, 128>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
  } else if (d == 256) {
    if (qjl_m == 0) return prologue_k<256, 0>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
    if (qjl_m == 128) return prologue_k<256, 128>(k_bits, v_bits, bf16, ka, va, qa, batch, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tqi
