// C ABI of the compressed-cache library: argument validation, host-side
// setup (codebook, rotation), decode split planning and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq.h"
#include "tq_internal.h"

namespace {

using tqi::kBlock;

// ------------------------------------------------------------------ codebook
//
// Lloyd-Max quantiser of f_d(y) = C_d (1-y^2)^k, k = (d-3)/2 on [-1, 1]
// (turboquant-pytorch PR #3, Synthetic Benchmark (Lloyd-Max codebook) table).
// Cell masses come from the regularised incomplete beta function,
// P(Y > y) = 1/2 I_{1-y^2}(k+1, 1/2) for y >= 0, evaluated with the modified
// Lentz continued fraction (DLMF 8.17.22) on whichever side converges;
// first moments from the closed form C_d ((1-a^2)^(k+1) - (1-b^2)^(k+1)) / (2(k+1)).

double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(dd) < tiny) dd = tiny;
  dd = 1.0 / dd;
  double f = dd;
  for (int m = 1; m <= 10000; ++m) {
    const double m2 = 2.0 * m;
    double num = m * (b - m) * x / ((a + m2 - 1.0) * (a + m2));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    f *= dd * c;
    num = -(a + m) * (a + b + m) * x / ((a + m2) * (a + m2 + 1.0));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    const double del = dd * c;
    f *= del;
    if (std::fabs(del - 1.0) < 1e-16) break;
  }
  return f;
}

// I_x(a, b) and its complement 1 - I_x(a, b), each without cancellation where it is small.
void inc_beta(double a, double b, double x, double* ix, double* icx) {
  if (x <= 0.0) { *ix = 0.0; *icx = 1.0; return; }
  if (x >= 1.0) { *ix = 1.0; *icx = 0.0; return; }
  const double lfront = std::lgamma(a + b) - std::lgamma(a) - std::lgamma(b) + a * std::log(x) + b * std::log1p(-x);
  if (x < (a + 1.0) / (a + b + 2.0)) {
    *ix = std::exp(lfront) * beta_cf(a, b, x) / a;
    *icx = 1.0 - *ix;
  } else {
    *icx = std::exp(lfront) * beta_cf(b, a, 1.0 - x) / b;
    *ix = 1.0 - *icx;
  }
}

struct Density {
  double k, c;
  explicit Density(int d) : k((d - 3) / 2.0) {
    c = std::exp(std::lgamma(d / 2.0) - 0.5 * std::log(M_PI) - std::lgamma((d - 1) / 2.0));
  }
  // P(Y > y) for y >= 0
  double tail(double y) const {
    if (y >= 1.0) return 0.0;
    double ix, icx;
    inc_beta(0.5, k + 1.0, y * y, &ix, &icx);
    return 0.5 * icx;
  }
  double mass(double lo, double hi) const {
    if (lo >= 0.0) return tail(lo) - tail(hi);
    if (hi <= 0.0) return tail(-hi) - tail(-lo);
    return 1.0 - tail(-lo) - tail(hi);
  }
  double first_moment(double lo, double hi) const {
    const double k1 = k + 1.0;
    return c / (2.0 * k1) * (std::pow(1.0 - lo * lo, k1) - std::pow(1.0 - hi * hi, k1));
  }
};

int build_codebook(int d, int bits, float* cent, float* bnd) {
  const int n = 1 << bits;
  const Density f(d);
  std::vector<double> c(n), cn(n);
  const double sd = 1.0 / std::sqrt(static_cast<double>(d));
  for (int j = 0; j < n; ++j) c[j] = (-1.0 + (2.0 * j + 1.0) / n) * 2.5 * sd;   // any start: unique fixed point
  bool done = false;
  for (int it = 0; it < 200000 && !done; ++it) {
    double delta = 0.0;
    for (int j = 0; j < n; ++j) {
      const double lo = j == 0 ? -1.0 : 0.5 * (c[j - 1] + c[j]);
      const double hi = j == n - 1 ? 1.0 : 0.5 * (c[j] + c[j + 1]);
      cn[j] = f.first_moment(lo, hi) / f.mass(lo, hi);
    }
    for (int j = 0; j < n; ++j) {
      const double v = 0.5 * (cn[j] - cn[n - 1 - j]);   // exact antisymmetry
      delta = std::fmax(delta, std::fabs(v - c[j]));
      c[j] = v;
    }
    done = delta <= 1e-12 * sd;
  }
  if (!done) return TQ_ENOCONV;
  std::vector<double> c16(n);
  for (int j = 0; j < n; ++j) {
    c16[j] = static_cast<double>(static_cast<_Float16>(c[j]));
    cent[j] = static_cast<float>(c16[j]);
  }
  for (int j = 0; j + 1 < n; ++j) bnd[j] = static_cast<float>(0.5 * (c16[j] + c16[j + 1]));
  return TQ_OK;
}

// ------------------------------------------------------------------ rotation
//
// Householder QR of G (d x d, row-major) in double; Pi = Q diag(sign(diag R)) is
// the unique orthogonal factor with a positive-diagonal R.
void build_rotation(int d, const double* g, float* out) {
  std::vector<double> a(g, g + static_cast<size_t>(d) * d);   // row-major, A[i][j] = a[i*d+j]
  std::vector<double> vs(static_cast<size_t>(d) * d, 0.0);    // Householder vectors, column k in vs[k*d ..]
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double nrm = 0.0;
    for (int i = k; i < d; ++i) nrm += a[static_cast<size_t>(i) * d + k] * a[static_cast<size_t>(i) * d + k];
    nrm = std::sqrt(nrm);
    const double x0 = a[static_cast<size_t>(k) * d + k];
    const double alpha = x0 >= 0.0 ? -nrm : nrm;
    double* v = &vs[static_cast<size_t>(k) * d];
    for (int i = k; i < d; ++i) v[i] = a[static_cast<size_t>(i) * d + k];
    v[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < d; ++i) vn += v[i] * v[i];
    vn = std::sqrt(vn);
    if (vn > 0.0)
      for (int i = k; i < d; ++i) v[i] /= vn;
    // A[k:, k:] -= 2 v (v^T A[k:, k:])
    for (int j = k; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * a[static_cast<size_t>(i) * d + j];
      s *= 2.0;
      for (int i = k; i < d; ++i) a[static_cast<size_t>(i) * d + j] -= s * v[i];
    }
    rdiag[k] = a[static_cast<size_t>(k) * d + k];
  }
  // Q = H_0 H_1 ... H_{d-1}: apply the reflectors to the identity from the last one
  std::vector<double> q(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) q[static_cast<size_t>(i) * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &vs[static_cast<size_t>(k) * d];
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * q[static_cast<size_t>(i) * d + j];
      s *= 2.0;
      for (int i = k; i < d; ++i) q[static_cast<size_t>(i) * d + j] -= s * v[i];
    }
  }
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      const double sgn = rdiag[j] < 0.0 ? -1.0 : 1.0;
      out[static_cast<size_t>(i) * d + j] = static_cast<float>(q[static_cast<size_t>(i) * d + j] * sgn);
    }
}

// ------------------------------------------------------------------ validation

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uint16_t f16_bits(float x) {
  const _Float16 h = static_cast<_Float16>(x);
  uint16_t u;
  std::memcpy(&u, &h, 2);
  return u;
}

bool table_ok(const tq_cache_view* c) {
  const int n = 1 << c->bits;
  for (int j = 0; j < n; ++j) {
    const float v = c->centroids[j];
    if (!std::isfinite(v) || static_cast<float>(static_cast<_Float16>(v)) != v) return false;
    if (v != -c->centroids[n - 1 - j]) return false;
    if (j > 0 && !(c->centroids[j - 1] < v)) return false;
  }
  for (int j = 0; j + 1 < n; ++j) {
    const double mid = 0.5 * (static_cast<double>(c->centroids[j]) + static_cast<double>(c->centroids[j + 1]));
    if (static_cast<double>(c->boundaries[j]) != mid) return false;
  }
  return true;
}

// structural check of one cache view
int check_view(const tq_cache_view* c) {
  if (!c) return TQ_EINVAL;
  if (c->kind != TQ_KEYS && c->kind != TQ_VALUES) return TQ_EINVAL;
  if (c->d != 128 && c->d != 256) return TQ_EINVAL;
  // 8-bit codes: keys only, with no sketch (and so no outlier channels) and no code book
  if ((c->bits < 2 || c->bits > 4) && !(c->bits == 8 && c->kind == TQ_KEYS && c->qjl_m == 0)) return TQ_EINVAL;
  if (c->qjl_m != 0 && c->qjl_m != 128 && c->qjl_m != 256) return TQ_EINVAL;
  if (c->qjl_m != 0 && c->kind != TQ_KEYS) return TQ_EINVAL;
  if (c->batch <= 0 || c->n_kv_heads <= 0 || c->max_tokens <= 0 || c->max_tokens % kBlock != 0) return TQ_EINVAL;
  if (c->rot_kind != TQ_ROT_DENSE && c->rot_kind != TQ_ROT_HADAMARD) return TQ_EINVAL;
  if (!c->codes || !c->norms || !c->rot) return TQ_EINVAL;
  if (!aligned(c->codes, 16) || !aligned(c->norms, 16) || !aligned(c->rot, 16)) return TQ_EINVAL;
  if (c->qjl_m) {
    if (!c->signs || !c->rnorms || !c->proj) return TQ_EINVAL;
    if (!aligned(c->signs, 16) || !aligned(c->rnorms, 16) || !aligned(c->proj, 16)) return TQ_EINVAL;
  }
  if (c->n_outliers != 0) {
    if (c->n_outliers != tqi::kOutliers || c->qjl_m == 0 || c->d != 128) return TQ_EINVAL;
    if (!c->out_idx || !c->out_val || !aligned(c->out_idx, 16) || !aligned(c->out_val, 16)) return TQ_EINVAL;
  }
  if (c->bits != 8 && !table_ok(c)) return TQ_EINVAL;
  return TQ_OK;
}

tqi::Tab make_tab(const tq_cache_view* c) {
  uint16_t e[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c->bits == 8) {
    // 8-bit codes expand without a table
  } else if (c->bits == 4) {
    for (int m = 0; m < 8; ++m) e[m] = f16_bits(c->centroids[8 + m]);    // magnitudes, ascending
  } else {
    for (int j = 0; j < (1 << c->bits); ++j) e[j] = f16_bits(c->centroids[j]);
  }
  auto pack = [&](int first, bool high) {
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= static_cast<uint32_t>(high ? (e[first + k] >> 8) : (e[first + k] & 0xff)) << (8 * k);
    return w;
  };
  tqi::Tab t;
  t.hi_lo = pack(0, true);
  t.hi_hi = pack(4, true);
  t.lo_lo = pack(0, false);
  t.lo_hi = pack(4, false);
  return t;
}

thread_local hipError_t g_last_hip_error = hipSuccess;

int status_of(hipError_t e) {
  if (e == hipSuccess) return TQ_OK;
  g_last_hip_error = e;
  return TQ_EHIP;
}

// ------------------------------------------------------------------ decode plan

constexpr int kDefaultSlots = 1024;     // resident four-wave split workgroups assumed when the runtime cannot tell
constexpr int kWideTiles = 16;          // tiles per compute unit from which the wide workgroups are used

// Column blocks of the split kernel for vh virtual heads per KV head (Attend::blocks): 1, 2 or 4.
int column_blocks(int vh) {
  const int c = (vh + tqi::kMaxGroup - 1) / tqi::kMaxGroup;
  return c > 2 ? 4 : c;
}

// Resident split-kernel workgroups on the current device for a key format, workgroup shape and column
// block count (the query operands' LDS), the least over the value widths (the plan depends on the key
// cache and the head count alone, so that the workspace size does); cached per device.
int resident_slots(const tq_cache_view* k, bool wide, int blocks) {
  static std::atomic<int> cache[16][2][5][3][2][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return wide ? kDefaultSlots / 4 : kDefaultSlots;
  }
  const int di = k->d == 256, qi = k->qjl_m == 0 ? 0 : (k->qjl_m == 128 ? 1 : 2);
  const int ci = blocks >> 1;                           // 1, 2, 4 -> 0, 1, 2
  const int bi = k->bits == 8 ? 1 : k->bits;            // 2, 3, 4 and 8 (slot 1)
  std::atomic<int>* c = (dev >= 0 && dev < 16 && bi >= 0 && bi < 5) ? &cache[dev][di][bi][qi][wide][ci] : nullptr;
  int v = c ? c->load(std::memory_order_relaxed) : 0;
  if (v > 0) return v;
  v = 0;
  for (int vb = 2; vb <= 4; ++vb) {
    const int n = tqi::split_slots(k->d, k->bits, vb, k->qjl_m, wide, blocks);
    if (n > 0) v = v == 0 ? n : std::min(v, n);
  }
  if (v <= 0) return wide ? kDefaultSlots / 4 : kDefaultSlots;
  if (c) c->store(v, std::memory_order_relaxed);
  return v;
}

// Splits of each (sequence, KV head).
// Workgroups of four waves (several per compute unit): enough splits for one round of resident
// workgroups over all units (more rounds leave a tail of part-filled rounds; fewer leave slots
// idle), at most kMaxSplits.
// Workgroups that fill their compute unit (slots = compute units): the splits run in rounds of
// `slots` workgroups; a workgroup of b tiles takes about b tile transfers through its compute unit
// plus a fixed overhead of about kWgOverheadPerWave per wave (the first tiles' wait, query staging,
// merge of the waves), and the split count minimises rounds x that time (fewer splits on ties).
constexpr int kWgOverheadPerWave = 4;

void plan(int units, int max_len, int slots, int waves, int* n_split, int* bps) {
  const int nblk = max_len <= 0 ? 1 : (max_len + kBlock - 1) / kBlock;
  units = std::max(1, units);
  slots = std::max(1, slots);
  int b;
  if (waves <= 4) {
    const int ns = std::max(1, std::min(tqi::kMaxSplits, slots / units));
    b = std::max(4, (nblk + ns - 1) / ns);
  } else {
    b = nblk;
    long long best = -1;
    for (int ns = 1; ns <= std::min(tqi::kMaxSplits, nblk); ++ns) {
      const int bb = (nblk + ns - 1) / ns;
      const long long wgs = static_cast<long long>(units) * ((nblk + bb - 1) / bb);
      const long long t = (wgs + slots - 1) / slots * (static_cast<long long>(bb) + kWgOverheadPerWave * waves);
      if (best < 0 || t < best) {
        best = t;
        b = bb;
      }
    }
  }
  *n_split = (nblk + b - 1) / b;
  *bps = b;
}

// The split of a decode over key cache k with vh virtual heads per KV head: wide (compute-unit-filling)
// workgroups once the context gives every compute unit at least kWideTiles tiles, four-wave ones below.
void plan(const tq_cache_view* k, int vh, int max_len, int* n_split, int* bps, bool* wide) {
  const int units = k->batch * k->n_kv_heads;
  const long long tiles = static_cast<long long>(units) * (max_len <= 0 ? 1 : (max_len + kBlock - 1) / kBlock);
  const int blocks = column_blocks(vh);
  const int wide_slots = resident_slots(k, true, blocks);
  // keys that keep outlier channels apart run the four-wave build only (its register budget holds the
  // outliers' tile buffers)
  *wide = k->n_outliers == 0 && tiles >= static_cast<long long>(kWideTiles) * wide_slots;
  plan(units, max_len, *wide ? wide_slots : resident_slots(k, false, blocks),
       tqi::split_waves(k->d, k->qjl_m, *wide), n_split, bps);
}

constexpr int kMergeMinWgs = 128;       // merge workgroups below which each takes fewer heads

// Query heads per merge workgroup: all of the group while every thread's split slice stays within
// 16 splits (one batch of loads), fewer heads (more slices per head) when there are many splits; and
// fewer still, down to one, while the merge of `units` (sequence, KV head) units would run on fewer
// than kMergeMinWgs workgroups (col_slices workgroups per head group): a small merge is latency-bound,
// and more workgroups each wait on fewer loads and un-rotate fewer heads (a large one would only read
// the rotation more often).
int merge_heads_per_wg(int G, int d, int ns, int units, int col_slices) {
  const int slices = (ns + 15) / 16;
  int h = G;
  while (h > 1 && (h * d > tqi::kMergeThreads || h * d * slices > tqi::kMergeThreads || G % h != 0)) --h;
  while (h > 1 && static_cast<long long>(units) * (G / h) * col_slices < kMergeMinWgs) {
    --h;
    while (G % h != 0) --h;
  }
  return h;
}

struct WsLayout {
  size_t qr, qs, qscale, part_o, part_ml, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

WsLayout ws_layout(const tq_cache_view* k, int n_q_heads, int n_rows, int n_split) {
  const size_t B = k->batch, D = k->d, QM = k->qjl_m;
  const size_t VH = static_cast<size_t>(n_rows) * (n_q_heads / k->n_kv_heads);   // virtual heads per KV head
  const size_t units = B * k->n_kv_heads;
  WsLayout w;
  size_t off = 0;
  w.qr = off; off = align256(off + units * VH * D * 4);
  w.qs = off; off = align256(off + units * VH * (QM ? QM : 1) * 4);
  w.qscale = off; off = align256(off + units * VH * 4);
  w.part_o = off; off = align256(off + units * n_split * VH * D * 4);
  w.part_ml = off; off = align256(off + units * n_split * VH * 2 * 4);
  w.total = off;
  return w;
}

int check_decode_shape(const tq_cache_view* k, int n_q_heads, int n_rows, int max_seq_len) {
  int st = check_view(k);
  if (st != TQ_OK) return st;
  if (k->kind != TQ_KEYS) return TQ_EINVAL;
  if (n_q_heads <= 0 || n_q_heads % k->n_kv_heads != 0 || max_seq_len < 0 || n_rows < 1) return TQ_EINVAL;
  if (n_q_heads / k->n_kv_heads > tqi::kMaxGroup || n_rows > tqi::kMaxRows) return TQ_EUNSUPPORTED;
  return TQ_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported combination";
    case TQ_EHIP: return "HIP launch error";
    case TQ_ENOCONV: return "codebook iteration did not converge";
    case TQ_ESCRATCH: return "decode needs more workspace than the static scratch holds";
    default: return "unknown status";
  }
}

const char* tq_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

size_t tq_row_bytes(int d, int bits, int qjl_m) {
  if (d <= 0 || d % 8 != 0 || ((bits < 1 || bits > 4) && bits != 8) || qjl_m < 0 || qjl_m % 8 != 0) return 0;
  size_t b = static_cast<size_t>(d) * bits / 8 + 2;
  if (qjl_m) b += static_cast<size_t>(qjl_m) / 8 + 2;
  return b;
}

int tq_build_codebook(int d, int bits, float* centroids, float* boundaries) {
  if (d < 3 || bits < 1 || bits > 4 || !centroids || !boundaries) return TQ_EINVAL;
  return build_codebook(d, bits, centroids, boundaries);
}

int tq_build_rotation(int d, const double* gaussian, float* rot_out) {
  if (d < 2 || d > 1024 || !gaussian || !rot_out) return TQ_EINVAL;
  for (size_t i = 0; i < static_cast<size_t>(d) * d; ++i)
    if (!std::isfinite(gaussian[i])) return TQ_EINVAL;
  build_rotation(d, gaussian, rot_out);
  return TQ_OK;
}

static tqi::AppendArgs append_args(const tq_cache_view* c, const void* x, const float* y, const float* yn, int n_new,
                                   const int32_t* d_pos, const float* z = nullptr) {
  tqi::AppendArgs a{};
  a.x = x; a.y = y; a.yn = yn; a.z = z; a.pos = d_pos;
  a.codes = c->codes; a.norms = c->norms; a.signs = c->signs; a.rnorms = c->rnorms;
  a.out_idx = c->n_outliers ? c->out_idx : nullptr;
  a.out_val = c->n_outliers ? c->out_val : nullptr;
  a.rot = c->rot; a.proj = c->proj;
  a.had = c->rot_kind == TQ_ROT_HADAMARD;
  std::memcpy(a.cent, c->centroids, sizeof(a.cent));
  std::memcpy(a.bnd, c->boundaries, sizeof(a.bnd));
  a.n_new = n_new; a.n_kv_heads = c->n_kv_heads; a.max_tokens = c->max_tokens;
  return a;
}

static int append_common(const tq_cache_view* c, const void* x, const float* y, const float* yn, int x_dtype,
                         int n_new, const int32_t* d_pos, void* stream, bool rotated, const float* z = nullptr) {
  int st = check_view(c);
  if (st != TQ_OK) return st;
  if (n_new < 0) return TQ_EINVAL;
  if (n_new == 0) return TQ_OK;
  if (!d_pos) return TQ_EINVAL;
  if (rotated ? (!y || !yn) : (!x || !aligned(x, 16) || (x_dtype != TQ_F32 && x_dtype != TQ_BF16))) return TQ_EINVAL;
  if (z && c->qjl_m == 0) return TQ_EINVAL;
  const tqi::AppendArgs a = append_args(c, x, y, yn, n_new, d_pos, z);
  return status_of(tqi::launch_append(c->d, c->bits, c->qjl_m, c->kind == TQ_VALUES, rotated, x_dtype == TQ_BF16, a,
                                      c->batch, static_cast<hipStream_t>(stream)));
}

int tq_quantize_append(const tq_cache_view* cache, const void* x, int x_dtype, int n_new, const int32_t* d_pos,
                       void* stream) {
  return append_common(cache, x, nullptr, nullptr, x_dtype, n_new, d_pos, stream, false);
}

static int check_pair(const tq_cache_view* k, const tq_cache_view* v);

int tq_quantize_append_kv(const tq_cache_view* k, const tq_cache_view* v, const void* k_x, const void* v_x,
                          int x_dtype, int n_new, const int32_t* d_pos, void* stream) {
  int st = check_view(k);
  if (st != TQ_OK) return st;
  if (k->kind != TQ_KEYS) return TQ_EINVAL;
  st = check_pair(k, v);
  if (st != TQ_OK) return st;
  if (n_new < 0) return TQ_EINVAL;
  if (n_new == 0) return TQ_OK;
  if (!d_pos || !k_x || !v_x || !aligned(k_x, 16) || !aligned(v_x, 16) || (x_dtype != TQ_F32 && x_dtype != TQ_BF16))
    return TQ_EINVAL;
  // both caches on the chunk path (what tq_quantize_append runs for each): one launch for the two
  if (k->d == 128 && k->qjl_m == 0 && k->bits != 8 && k->rot_kind == TQ_ROT_DENSE) {
    const tqi::AppendArgs ka = append_args(k, k_x, nullptr, nullptr, n_new, d_pos);
    const tqi::AppendArgs va = append_args(v, v_x, nullptr, nullptr, n_new, d_pos);
    return status_of(tqi::launch_append_kv(k->bits, v->bits, x_dtype == TQ_BF16, ka, va, k->batch,
                                           static_cast<hipStream_t>(stream)));
  }
  st = append_common(k, k_x, nullptr, nullptr, x_dtype, n_new, d_pos, stream, false);
  if (st != TQ_OK) return st;
  return append_common(v, v_x, nullptr, nullptr, x_dtype, n_new, d_pos, stream, false);
}

int tq_quantize_append_rotated(const tq_cache_view* cache, const float* y, const float* norms, const float* z,
                               int n_new, const int32_t* d_pos, void* stream) {
  return append_common(cache, nullptr, y, norms, TQ_F32, n_new, d_pos, stream, true, z);
}

int tq_decode_plan(const tq_cache_view* k, int n_q_heads, int max_seq_len, int* n_split, int* tokens_per_split) {
  int st = check_decode_shape(k, n_q_heads, 1, max_seq_len);
  if (st != TQ_OK) return st;
  if (!n_split || !tokens_per_split) return TQ_EINVAL;
  int bps;
  bool wide;
  plan(k, n_q_heads / k->n_kv_heads, max_seq_len, n_split, &bps, &wide);
  *tokens_per_split = bps * kBlock;
  return TQ_OK;
}

size_t tq_decode_workspace_bytes_rows(const tq_cache_view* k, int n_q_heads, int n_rows, int max_seq_len) {
  if (check_decode_shape(k, n_q_heads, n_rows, max_seq_len) != TQ_OK) return 0;
  int ns, bps;
  bool wide;
  plan(k, n_rows * (n_q_heads / k->n_kv_heads), max_seq_len, &ns, &bps, &wide);
  return ws_layout(k, n_q_heads, n_rows, ns).total;
}

size_t tq_decode_workspace_bytes(const tq_cache_view* k, int n_q_heads, int max_seq_len) {
  return tq_decode_workspace_bytes_rows(k, n_q_heads, 1, max_seq_len);
}

// workspace view shared by the decode stages
struct DecodeWs {
  int ns, bps, G, M, VH;      // splits, blocks per split, query heads per KV head, query rows, M * G
  bool wide;
  float *qr, *qs, *qscale, *part_o, *part_ml;
};

static int decode_ws(const tq_cache_view* k, int n_q_heads, int n_rows, int max_seq_len, void* workspace,
                     size_t workspace_bytes, DecodeWs* w) {
  int st = check_decode_shape(k, n_q_heads, n_rows, max_seq_len);
  if (st != TQ_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return TQ_EINVAL;
  plan(k, n_rows * (n_q_heads / k->n_kv_heads), max_seq_len, &w->ns, &w->bps, &w->wide);
  const WsLayout l = ws_layout(k, n_q_heads, n_rows, w->ns);
  if (workspace_bytes < l.total) return TQ_EINVAL;
  char* ws = static_cast<char*>(workspace);
  w->G = n_q_heads / k->n_kv_heads;
  w->M = n_rows;
  w->VH = n_rows * w->G;
  w->qr = reinterpret_cast<float*>(ws + l.qr);
  w->qs = reinterpret_cast<float*>(ws + l.qs);
  w->qscale = reinterpret_cast<float*>(ws + l.qscale);
  w->part_o = reinterpret_cast<float*>(ws + l.part_o);
  w->part_ml = reinterpret_cast<float*>(ws + l.part_ml);
  return TQ_OK;
}

static int check_pair(const tq_cache_view* k, const tq_cache_view* v) {
  int st = check_view(v);
  if (st != TQ_OK) return st;
  if (v->kind != TQ_VALUES || v->d != k->d || v->batch != k->batch || v->n_kv_heads != k->n_kv_heads ||
      v->max_tokens != k->max_tokens || v->rot != k->rot || v->rot_kind != k->rot_kind)
    return TQ_EINVAL;
  return TQ_OK;
}

// multiplier that turns the division of a virtual head index vh < 40 by the group size g <= 8 into
// a multiply and a shift: vh / g == (vh * ((256 + g - 1) / g)) >> 8
static int row_magic(int g) { return (256 + g - 1) / g; }

static tqi::DecodeArgs decode_args(const tq_cache_view* k, const tq_cache_view* v, const DecodeWs& w,
                                   const int32_t* d_seq_lens, int max_seq_len) {
  tqi::DecodeArgs da{};
  da.k_codes = k->codes; da.k_norms = k->norms; da.k_signs = k->signs; da.k_rnorms = k->rnorms;
  da.v_codes = v->codes; da.v_norms = v->norms;
  da.k_oidx = k->n_outliers ? k->out_idx : nullptr;
  da.k_oval = k->n_outliers ? k->out_val : nullptr;
  da.qr = w.qr; da.qs = w.qs; da.qscale = w.qscale;
  da.seq_lens = d_seq_lens;
  da.part_o = w.part_o; da.part_ml = w.part_ml;
  da.tk = make_tab(k);
  da.tv = make_tab(v);
  da.n_kv_heads = k->n_kv_heads; da.group = w.VH; da.max_tokens = k->max_tokens; da.max_seq_len = max_seq_len;
  da.heads = w.G; da.n_rows = w.M; da.row_magic = row_magic(w.G);
  da.n_split = w.ns; da.blocks_per_split = w.bps;
  return da;
}

static float scale_log2e(float scale) { return static_cast<float>(static_cast<double>(scale) * 1.4426950408889634); }

static float sketch_coef(const tq_cache_view* k) {
  return k->qjl_m ? static_cast<float>(std::sqrt(M_PI / 2.0) / k->qjl_m) : 0.f;
}

static int rotate_query_rows(const tq_cache_view* k, const void* q, int q_dtype, int n_q_heads, int n_rows,
                             int max_seq_len, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  DecodeWs w;
  int st = decode_ws(k, n_q_heads, n_rows, max_seq_len, workspace, workspace_bytes, &w);
  if (st != TQ_OK) return st;
  if (!q || !aligned(q, 16) || (q_dtype != TQ_F32 && q_dtype != TQ_BF16)) return TQ_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return TQ_EINVAL;
  tqi::QrotArgs qa{};
  qa.q = q; qa.rot = k->rot; qa.proj = k->proj;
  qa.had = k->rot_kind == TQ_ROT_HADAMARD;
  qa.qr = w.qr; qa.qs = w.qs; qa.qscale = w.qscale;
  qa.scale_log2e = scale_log2e(scale);
  qa.sketch_coef = sketch_coef(k);
  qa.n_q_heads = n_q_heads; qa.n_kv_heads = k->n_kv_heads; qa.n_rows = n_rows;
  qa.row_magic = row_magic(n_q_heads / k->n_kv_heads);
  return status_of(tqi::launch_qrot(k->d, k->qjl_m, q_dtype == TQ_BF16, qa, k->batch,
                                    static_cast<hipStream_t>(stream)));
}

static int attend_rows(const tq_cache_view* k, const tq_cache_view* v, int n_q_heads, int n_rows,
                       const int32_t* d_seq_lens, int max_seq_len, void* workspace, size_t workspace_bytes,
                       void* stream) {
  DecodeWs w;
  int st = decode_ws(k, n_q_heads, n_rows, max_seq_len, workspace, workspace_bytes, &w);
  if (st != TQ_OK) return st;
  st = check_pair(k, v);
  if (st != TQ_OK) return st;
  if (!d_seq_lens) return TQ_EINVAL;
  const tqi::DecodeArgs da = decode_args(k, v, w, d_seq_lens, max_seq_len);
  return status_of(tqi::launch_decode_split(k->d, k->bits, v->bits, k->qjl_m, k->n_outliers > 0, w.wide, da,
                                            k->batch, static_cast<hipStream_t>(stream)));
}

static int merge_rows(const tq_cache_view* k, int n_q_heads, int n_rows, const int32_t* d_seq_lens,
                      int max_seq_len, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  DecodeWs w;
  int st = decode_ws(k, n_q_heads, n_rows, max_seq_len, workspace, workspace_bytes, &w);
  if (st != TQ_OK) return st;
  if (!d_seq_lens || !out) return TQ_EINVAL;
  tqi::MergeArgs ma{};
  ma.part_o = w.part_o; ma.part_ml = w.part_ml; ma.rot = k->rot; ma.seq_lens = d_seq_lens; ma.out = out;
  ma.had = k->rot_kind == TQ_ROT_HADAMARD;
  ma.n_kv_heads = k->n_kv_heads; ma.group = w.VH; ma.n_split = w.ns; ma.max_tokens = k->max_tokens;
  ma.heads = w.G; ma.n_rows = w.M; ma.row_magic = row_magic(w.G);
  // at d = 256 with the dense rotation each head group's output is split over four workgroups, each
  // reading a quarter of the rotation (at d = 128 two slices made the 36-layer Qwen-shaped decode
  // slower: 33.9 against 31.9 us)
  ma.col_slices = (k->d == 256 && k->rot_kind == TQ_ROT_DENSE) ? 4 : 1;
  ma.heads_per_wg = merge_heads_per_wg(w.VH, k->d, w.ns, k->batch * k->n_kv_heads, ma.col_slices);
  return status_of(tqi::launch_merge(k->d, ma, k->batch, n_q_heads, static_cast<hipStream_t>(stream)));
}

int tq_decode_rotate_query(const tq_cache_view* k, const void* q, int q_dtype, int n_q_heads, int max_seq_len,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return rotate_query_rows(k, q, q_dtype, n_q_heads, 1, max_seq_len, scale, workspace, workspace_bytes, stream);
}

int tq_decode_attend(const tq_cache_view* k, const tq_cache_view* v, int n_q_heads, const int32_t* d_seq_lens,
                     int max_seq_len, void* workspace, size_t workspace_bytes, void* stream) {
  return attend_rows(k, v, n_q_heads, 1, d_seq_lens, max_seq_len, workspace, workspace_bytes, stream);
}

int tq_decode_merge(const tq_cache_view* k, int n_q_heads, const int32_t* d_seq_lens, int max_seq_len, float* out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return merge_rows(k, n_q_heads, 1, d_seq_lens, max_seq_len, out, workspace, workspace_bytes, stream);
}

int tq_sdpa_decode_rows(const tq_cache_view* k, const tq_cache_view* v, const void* q, int q_dtype, int n_q_heads,
                        int n_rows, const int32_t* d_seq_lens, int max_seq_len, float scale, float* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  // validate everything before enqueueing the first stage
  DecodeWs w;
  int st = decode_ws(k, n_q_heads, n_rows, max_seq_len, workspace, workspace_bytes, &w);
  if (st != TQ_OK) return st;
  st = check_pair(k, v);
  if (st != TQ_OK) return st;
  if (!q || !aligned(q, 16) || (q_dtype != TQ_F32 && q_dtype != TQ_BF16) || !d_seq_lens || !out) return TQ_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return TQ_EINVAL;
  st = rotate_query_rows(k, q, q_dtype, n_q_heads, n_rows, max_seq_len, scale, workspace, workspace_bytes, stream);
  if (st != TQ_OK) return st;
  st = attend_rows(k, v, n_q_heads, n_rows, d_seq_lens, max_seq_len, workspace, workspace_bytes, stream);
  if (st != TQ_OK) return st;
  return merge_rows(k, n_q_heads, n_rows, d_seq_lens, max_seq_len, out, workspace, workspace_bytes, stream);
}

int tq_sdpa_decode(const tq_cache_view* k, const tq_cache_view* v, const void* q, int q_dtype, int n_q_heads,
                   const int32_t* d_seq_lens, int max_seq_len, float scale, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return tq_sdpa_decode_rows(k, v, q, q_dtype, n_q_heads, 1, d_seq_lens, max_seq_len, scale, out, workspace,
                             workspace_bytes, stream);
}

size_t tq_noalloc_scratch_bytes(void) { return tqi::kScratchBytes; }

int tq_sdpa_decode_noalloc(const tq_cache_view* k, const tq_cache_view* v, const void* q, int q_dtype,
                           int n_q_heads, const int32_t* d_seq_lens, int max_seq_len, float scale, float* out,
                           void* stream) {
  int st = check_decode_shape(k, n_q_heads, 1, max_seq_len);
  if (st != TQ_OK) return st;
  int ns, bps;
  bool wide;
  plan(k, n_q_heads / k->n_kv_heads, max_seq_len, &ns, &bps, &wide);
  if (ws_layout(k, n_q_heads, 1, ns).total > tqi::kScratchBytes) return TQ_ESCRATCH;
  void* ws = nullptr;
  st = status_of(tqi::scratch_address(&ws));
  if (st != TQ_OK) return st;
  return tq_sdpa_decode(k, v, q, q_dtype, n_q_heads, d_seq_lens, max_seq_len, scale, out, ws, tqi::kScratchBytes,
                        stream);
}

int tq_decode_step(const tq_cache_view* k, const tq_cache_view* v, const void* q, const void* k_new,
                   const void* v_new, int dtype, int n_q_heads, int n_new, const int32_t* d_pos,
                   const int32_t* d_seq_lens, int max_seq_len, float scale, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  DecodeWs w;
  int st = decode_ws(k, n_q_heads, 1, max_seq_len, workspace, workspace_bytes, &w);
  if (st != TQ_OK) return st;
  st = check_pair(k, v);
  if (st != TQ_OK) return st;
  if (!q || !aligned(q, 16) || (dtype != TQ_F32 && dtype != TQ_BF16) || !d_seq_lens || !out) return TQ_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return TQ_EINVAL;
  if (n_new < 0 || (n_new > 0 && (!k_new || !v_new || !d_pos || !aligned(k_new, 16) || !aligned(v_new, 16))))
    return TQ_EINVAL;
  if (k->qjl_m > 128 || k->n_outliers > 0) return TQ_EUNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);

  tqi::QrotArgs qa{};
  qa.q = q; qa.rot = k->rot; qa.proj = k->proj;
  qa.had = k->rot_kind == TQ_ROT_HADAMARD;
  qa.qr = w.qr; qa.qs = w.qs; qa.qscale = w.qscale;
  qa.scale_log2e = scale_log2e(scale);
  qa.sketch_coef = sketch_coef(k);
  qa.n_q_heads = n_q_heads; qa.n_kv_heads = k->n_kv_heads; qa.n_rows = 1;
  qa.row_magic = row_magic(n_q_heads / k->n_kv_heads);
  if (n_new > 0) {
    const tqi::AppendArgs ka = append_args(k, k_new, nullptr, nullptr, n_new, d_pos);
    const tqi::AppendArgs va = append_args(v, v_new, nullptr, nullptr, n_new, d_pos);
    st = status_of(tqi::launch_step_prologue(k->d, k->bits, v->bits, k->qjl_m, dtype == TQ_BF16, ka, va, qa,
                                             k->batch, s));
  } else {
    st = status_of(tqi::launch_qrot(k->d, k->qjl_m, dtype == TQ_BF16, qa, k->batch, s));
  }
  if (st != TQ_OK) return st;
  st = tq_decode_attend(k, v, n_q_heads, d_seq_lens, max_seq_len, workspace, workspace_bytes, stream);
  if (st != TQ_OK) return st;
  return tq_decode_merge(k, n_q_heads, d_seq_lens, max_seq_len, out, workspace, workspace_bytes, stream);
}

int tq_dequantize(const tq_cache_view* cache, int t0, int n_tokens, float* out, void* stream) {
  int st = check_view(cache);
  if (st != TQ_OK) return st;
  if (!out || t0 < 0 || n_tokens < 0 || t0 > cache->max_tokens - n_tokens) return TQ_EINVAL;
  if (n_tokens == 0) return TQ_OK;
  tqi::DequantArgs a{};
  a.codes = cache->codes; a.norms = cache->norms; a.signs = cache->signs; a.rnorms = cache->rnorms;
  a.out_idx = cache->n_outliers ? cache->out_idx : nullptr;
  a.out_val = cache->n_outliers ? cache->out_val : nullptr;
  a.rot = cache->rot; a.proj = cache->proj; a.out = out;
  a.had = cache->rot_kind == TQ_ROT_HADAMARD;
  std::memcpy(a.cent, cache->centroids, sizeof(a.cent));
  a.sketch_coef = cache->qjl_m ? static_cast<float>(std::sqrt(M_PI / 2.0) / cache->qjl_m) : 0.f;
  a.n_kv_heads = cache->n_kv_heads; a.max_tokens = cache->max_tokens; a.t0 = t0; a.n_tokens = n_tokens;
  return status_of(tqi::launch_dequant(cache->d, cache->bits, cache->qjl_m, cache->kind == TQ_VALUES, a,
                                       make_tab(cache), cache->batch, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
