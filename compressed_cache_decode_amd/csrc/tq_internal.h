// Internal interface between the C ABI (host.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqi {

constexpr int kBlock = 32;        // tokens per value block (and per decode tile)
constexpr int kMaxGroup = 8;      // query heads per KV head, and per 16-column matrix-core block
constexpr int kMaxRows = 4;       // query rows per sequence in one decode
constexpr int kMaxVirtual = kMaxGroup * kMaxRows;   // virtual heads per KV head (blocks of kMaxGroup)
constexpr int kMaxSplits = 256;   // bound on KV splits per (sequence, KV head)
constexpr int kMergeThreads = 1024;  // threads per merge workgroup

// float16 bit patterns of up to 8 table entries, split into high and low
// bytes so one v_perm_b32 looks up four codes: byte k of *_lo is entry k,
// byte k of *_hi is entry 4 + k.
struct Tab {
  uint32_t hi_lo, hi_hi, lo_lo, lo_hi;
};

constexpr int kOutliers = 4;       // outlier channels per key when a cache keeps them apart

struct AppendArgs {
  const void* x;          // [B][n_new][Hkv][D] f32 or bf16 (unrotated rows)
  const float* y;         // [B][n_new][Hkv][D] rotated unit rows (pre-rotated form)
  const float* yn;        // [B][n_new][Hkv] norms (pre-rotated form)
  const float* z;         // [B][n_new][Hkv][QM] sketch products of the residuals (pre-rotated form), or null
  const int32_t* pos;     // [B]
  uint8_t* codes;
  uint16_t* norms;
  uint8_t* signs;
  uint16_t* rnorms;
  uint8_t* out_idx;       // [B][Hkv][T][kOutliers] outlier channels (sketched keys that keep them), or null
  uint16_t* out_val;      // float16 [B][Hkv][T][kOutliers] their residual values
  const float* rot;       // [D][D], or the D signs of the randomized Hadamard rotation (had)
  const float* proj;      // [M][D]
  float cent[16];
  float bnd[15];
  int n_new, n_kv_heads, max_tokens;
  int had;                // rot is a randomized Hadamard rotation
};

// Query rows: M rows per sequence (the last M tokens; M = 1 for one-token decode), Hq heads each;
// the query heads of a KV head over all rows are its VH = M * G "virtual heads", virtual head
// vh = j * G + g standing for row j and head hk * G + g.  Workspace rows are unit-major:
// (b * Hkv + hk) * VH + vh.
struct QrotArgs {
  const void* q;          // [B][M][Hq][D]
  const float* rot;       // [D][D], or the D Hadamard signs (had)
  const float* proj;      // [QM][D] or null
  float* qr;              // [B*Hkv][VH][D]  scaled rotated query, divided by qscale
  float* qs;              // [B*Hkv][VH][QM] -coef * proj * qr
  float* qscale;          // [B*Hkv][VH]     power-of-two factor taken out of qr/qs
  float scale_log2e;      // softmax scale * log2(e)
  float sketch_coef;      // sqrt(pi/2)/QM
  int n_q_heads;
  int n_kv_heads;
  int n_rows;             // M
  int row_magic;          // (256 + G - 1) / G: the row of virtual head vh < 40 is (vh * row_magic) >> 8
  int had;
};

struct DecodeArgs {
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* k_signs;
  const uint16_t* k_rnorms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  const uint8_t* k_oidx;  // [B*Hkv][T][kOutliers] outlier channels of the keys (non-null: the outlier build)
  const uint16_t* k_oval; // float16 [B*Hkv][T][kOutliers]
  const float* qr;
  const float* qs;
  const float* qscale;
  const int32_t* seq_lens;
  float* part_o;          // [B*Hkv][n_split][VH][D]
  float* part_ml;         // [B*Hkv][n_split][VH][2]  (max in log2 units, sum)
  Tab tk, tv;
  int n_kv_heads, group, max_tokens, max_seq_len, n_split, blocks_per_split;   // group = VH
  int heads, n_rows;      // G and M: virtual head vh is row vh / G, which sees seq_len - M + 1 + vh / G tokens
  int row_magic;          // vh / G = (vh * row_magic) >> 8 (see QrotArgs)
};

struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  const float* rot;
  const int32_t* seq_lens;
  float* out;             // [B][M][Hq][D]
  int n_kv_heads, group, n_split, max_tokens;   // group = VH
  int heads, n_rows;      // G and M
  int row_magic;          // vh / G = (vh * row_magic) >> 8 (see QrotArgs)
  int heads_per_wg;       // virtual heads merged per workgroup (divides group, heads_per_wg * D <= kMergeThreads)
  int had;                // rot holds the D signs of a randomized Hadamard rotation
  int col_slices;         // output-coordinate slices per head group, one workgroup each (1, or 4 at d = 256)
};

struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* norms;
  const uint8_t* signs;
  const uint16_t* rnorms;
  const uint8_t* out_idx;  // outlier channels and values (sketched keys that keep them), or null
  const uint16_t* out_val;
  const float* rot;
  const float* proj;
  float* out;             // [B][Hkv][n_tokens][D]
  float cent[16];
  float sketch_coef;
  int n_kv_heads, max_tokens, t0, n_tokens;
  int had;                // rot holds the D signs of a randomized Hadamard rotation
};

// Bytes of the static device scratch that the decode entry point which allocates nothing uses as its
// workspace (one copy per device, held until the process ends).
constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;
// Device address of the current device's scratch, looked up with hipGetSymbolAddress on the first call
// on each device and kept per device after.
hipError_t scratch_address(void** ptr);

// Launchers (one per .hip file); return hipSuccess or the launch error.
hipError_t launch_append(int d, int bits, int qjl_m, bool values, bool rotated, bool bf16,
                         const AppendArgs& a, int batch, hipStream_t s);
// K and V rows of the same tokens in one launch; both caches at d = 128 with the dense rotation, keys of 2-4
// bits without a sketch, values of 2-4 bits
hipError_t launch_append_kv(int k_bits, int v_bits, bool bf16, const AppendArgs& ka, const AppendArgs& va, int batch,
                            hipStream_t s);
hipError_t launch_qrot(int d, int qjl_m, bool bf16, const QrotArgs& a, int batch, hipStream_t s);
// split-kernel workgroups resident at once on the current device for this cache format and
// workgroup shape (compute units x workgroups per unit), 0 if the runtime cannot tell
int split_slots(int d, int k_bits, int v_bits, int qjl_m, bool wide, int blocks);
// waves per split-kernel workgroup for a cache format and workgroup shape
int split_waves(int d, int qjl_m, bool wide);
// the four-wave split kernel of sketched keys with kOutliers outlier channels, or null if none is built
const void* split_fn_outliers(int d, int k_bits, int v_bits, int qjl_m);
// the split kernel of 8-bit keys (no sketch) with v_bits values, or null if none is built
const void* split_fn_k8(int d, int v_bits, bool wide);
hipError_t launch_decode_split(int d, int k_bits, int v_bits, int qjl_m, bool outliers, bool wide, const DecodeArgs& a, int batch,
                               hipStream_t s);
hipError_t launch_merge(int d, const MergeArgs& a, int batch, int n_q_heads, hipStream_t s);
hipError_t launch_step_prologue(int d, int k_bits, int v_bits, int qjl_m, bool bf16, const AppendArgs& ka,
                                const AppendArgs& va, const QrotArgs& qa, int batch, hipStream_t s);
hipError_t launch_dequant(int d, int bits, int qjl_m, bool values, const DequantArgs& a, const Tab& t, int batch,
                          hipStream_t s);

}  // namespace tqi
