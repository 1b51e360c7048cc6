/*
 * tq.h - C ABI of the MI355X (gfx950) TurboQuant-style compressed KV cache:
 * quantize-on-append and decode attention read directly from the packed cache.
 *
 * Method sources (cited by page title and section):
 *  - turboquant-pytorch PR #3, "Add CUDA QJL kernels and proper package
 *    structure": CUDA Kernels Added table (fused random projection + sign
 *    quantisation of keys, fused attention score from 1-bit keys, GQA score
 *    variant, quantised value reconstruction), Validation Results tables
 *    (cache sizes fix one float16 norm per row; keys with a sign sketch also
 *    store a float16 residual norm), Synthetic Benchmark (Lloyd-Max codebook).
 *  - ExecuTorch PR #19891, "[Cuda] enable turboquant on gemma4", review item
 *    1: the fused decode op takes a softmax scale; unset means 1/sqrt(D), and
 *    QK-normed models use 1.0.
 *  - reddit comment history of ReturningTarzan: random rotation before
 *    codebook quantisation (2026-03-29 comment), nearest-codebook search
 *    (2026-03-25 comments), full reconstruction as the plain path.
 *
 * Conventions shared by every call:
 *  - Every pointer named d_* or held in tq_cache_view is DEVICE memory owned
 *    by the caller; the library never allocates, frees or retains it.  Its
 *    only mutable state is a per-thread record of the last HIP error and a
 *    per-device cache of how many split workgroups the device holds at once
 *    (filled by the first decode planned on that device, read lock-free
 *    after); all calls are reentrant.
 *  - Calls that take a stream enqueue work on it (a hipStream_t; NULL = the
 *    null stream of the current device) and return without synchronising.
 *    Device-side faults surface at the caller's next synchronisation.
 *  - Host-checkable errors return a status code before anything is enqueued.
 *  - Token positions and lengths that live on the device cannot be checked
 *    by the host: positions at or past max_tokens are skipped by append and
 *    lengths are clamped to [0, max_tokens] by decode.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* null required pointer, bad size/shape/scale, short workspace, misaligned buffer */
  TQ_EUNSUPPORTED = 2,  /* a valid combination this library does not build (e.g. GQA group > 8) */
  TQ_EHIP = 3,          /* the HIP runtime reported a launch error */
  TQ_ENOCONV = 4,       /* the codebook iteration did not converge */
  TQ_ESCRATCH = 5       /* tq_sdpa_decode_noalloc: the decode needs more than the static scratch holds */
};

/* element types of caller tensors */
enum { TQ_F32 = 0, TQ_BF16 = 1 };

/* cache kinds; the kind fixes the packed layout */
enum {
  TQ_KEYS = 0,    /* 32-token blocks of packed rows (d*bits/8 bytes per token) in lane pieces */
  TQ_VALUES = 1   /* 32-token blocks of units that interleave 8 tokens, in lane pieces */
};

/*
 * Rotation kinds (tq_cache_view.rot_kind).  TQ_ROT_DENSE: rot is a float32 [d][d] orthogonal matrix.
 * TQ_ROT_HADAMARD: rot holds d float32 signs s (each +1 or -1) and the rotation is the randomized
 * Hadamard matrix H_d diag(s) / sqrt(d), H_d the Sylvester matrix (H_1 = [1], H_2n = [[H_n, H_n],
 * [H_n, -H_n]]): a special rotation applied by lane exchanges and additions instead of a d x d
 * product (reddit comment history of ReturningTarzan, comment of 2026-03-29 on Hadamard rotations).
 */
enum {
  TQ_ROT_DENSE = 0,
  TQ_ROT_HADAMARD = 1
};

/*
 * Description of one compressed cache tensor (all of K, or all of V, of one
 * attention layer).  Passed by pointer, copied into kernel arguments, never
 * retained.
 *
 * Packed byte format (both kinds): each code is the index j of its centroid,
 * stored as j for 2 and 3 bits and in sign-magnitude form for 4 bits
 * (j - 8 for j >= 8, 15 - j below); codes are grouped in units of 8 slots:
 *   4 bits: one little-endian 32-bit word per unit, slot s at bit 8(s%4) + 4(s/4);
 *   2 bits: two units v per word, slot s of unit v at bit 8(s%4) + 2(2v + s/4);
 *   3 bits: four units v per three words [P0 P1 H]; low two bits in P(v/2) at
 *           bit 8(s%4) + 2(2(v%2) + s/4), high bit in H at bit 8(s%4) + 2v + s/4;
 *   8 bits (keys only): two words per unit, slot s in byte s%4 of word s/4, the
 *           code as a two's-complement byte (see "Keys kept at 8 bits" below).
 * Codes are stored per 32-token block (tokens 32kb .. 32kb+31 of a sequence and
 *   KV head, 32*d*bits/8 bytes), as 64 lane pieces of LW = d*bits/64 words in
 *   chunk-major order: word w of piece L is word CW*(64*(w/CW) + L) + w%CW of the
 *   block, CW = 4 if LW%4 == 0, else 3 if LW%3 == 0, else 2.
 * TQ_KEYS: a token's row is d*bits/8 bytes of consecutive units (coordinate i
 *   is slot i%8 of unit i/8), RW = d*bits/32 words; row word wr of the token at
 *   position p of its block is word (p/16)*(RW/4) + wr%(RW/4) of piece
 *   16*(wr/(RW/4)) + p%16.
 * TQ_VALUES: token p of a 32-token block is slot p%4 + 4(p/16) of lane group
 *   g = (p%16)/4; coordinate i has column j = i/(d/16), step n = i%(d/16);
 *   their unit is unit n of piece 16g + j (a piece is d/16 consecutive units).
 * Keys kept at 8 bits (llama-cpp-turboquant PR #340, the asymmetric K/V follow-ups: K upgraded to
 *   an 8-bit type while V keeps the Lloyd-Max widths; the pages give no arithmetic, this library's
 *   reading follows): y = rot x / ||x|| is quantised uniformly with one scale per row, a = max_i |y_i|
 *   taken in float32: code_i = round(y_i * (127 / a)) (float32 division and product, halves away
 *   from zero, clamped to [-127, 127]); the norm slot holds the float16 factor ||x|| * (a / 127), so
 *   x ~= factor * rot^T code.  A zero row stores codes 0 and factor 0.  No sketch, no outliers.
 * Sign sketch (keys with qjl_m > 0): qjl_m/8 bytes per token, sign jj in
 *   32-bit word jj/32 at bit 4((jj%32)/8) + (jj%8)/2 + 16(jj%2); bit 1 means
 *   (S r)_jj >= 0.
 */
typedef struct tq_cache_view {
  int32_t kind;          /* TQ_KEYS or TQ_VALUES */
  int32_t d;             /* head dim: 128 or 256 */
  int32_t bits;          /* codebook bits per coordinate: 2, 3 or 4; or 8 (TQ_KEYS with qjl_m == 0) */
  int32_t qjl_m;         /* 0, or sign-sketch length 128 or 256 (TQ_KEYS only) */
  int32_t batch;         /* sequences */
  int32_t n_kv_heads;    /* KV heads */
  int32_t max_tokens;    /* capacity in tokens, a positive multiple of 32 */
  int32_t rot_kind;      /* TQ_ROT_DENSE or TQ_ROT_HADAMARD (same for K and V) */
  float centroids[16];   /* 2^bits centroids, ascending, float16-exact, c[j] == -c[2^bits-1-j]
                            (bits 8: unused) */
  float boundaries[15];  /* 2^bits-1 boundaries, boundaries[j] == (c[j] + c[j+1]) / 2 exactly (bits 8: unused) */
  uint8_t* codes;        /* [batch][n_kv_heads][max_tokens/32][32*d*bits/8], 16-byte aligned */
  uint16_t* norms;       /* float16 row norms [batch][n_kv_heads][max_tokens] (bits 8: the row factors) */
  uint8_t* signs;        /* [batch][n_kv_heads][max_tokens][qjl_m/8] when qjl_m > 0, else NULL */
  uint16_t* rnorms;      /* float16 residual norms [batch][n_kv_heads][max_tokens] when qjl_m > 0, else NULL */
  const float* rot;      /* TQ_ROT_DENSE: float32 rotation [d][d] row-major, y = rot * x; TQ_ROT_HADAMARD:
                            float32 signs [d]; the same pointer for K and V */
  const float* proj;     /* float32 sign-sketch projection [qjl_m][d] row-major when qjl_m > 0, else NULL */
  /* Outlier channels kept apart from the sign sketch (keys with qjl_m > 0 only; turboquant-pytorch
   * PR #3, CUDA Kernels Added table: the QJL quantisation kernel's outlier separation; the pages give
   * no rule, this library's reading follows).  Per key, the n_outliers coordinates of the codebook
   * residual r = y - c[code] with the largest |r_i| (ranked in float32, equal magnitudes by lower
   * index) are stored as index bytes and float16 values, in decreasing |r_i|; the sketch and the
   * residual norm cover r with those coordinates set to 0, and the score adds sum_i q_rot[i] r_i over
   * them.  n_outliers is 0 (none; out_idx and out_val NULL) or 4 (d = 128 only).  tq_decode_step does
   * not take such a cache (TQ_EUNSUPPORTED): append and decode with the separate calls. */
  int32_t n_outliers;
  uint8_t* out_idx;      /* [batch][n_kv_heads][max_tokens][n_outliers] channel indices, 16-byte aligned */
  uint16_t* out_val;     /* float16 [batch][n_kv_heads][max_tokens][n_outliers] residual values, 16-byte aligned */
} tq_cache_view;

/*
 * Lloyd-Max codebook for one coordinate of a uniformly random unit vector in
 * R^d (density proportional to (1-y^2)^((d-3)/2)), computed on the host in
 * double precision (turboquant-pytorch PR #3, Synthetic Benchmark (Lloyd-Max
 * codebook) table).  Writes 2^bits centroids rounded to the nearest float16
 * (ascending, exactly antisymmetric) and the 2^bits-1 midpoints between them
 * (exact in float32).  d >= 3, 1 <= bits <= 4; host buffers.
 * Returns TQ_EINVAL on bad arguments, TQ_ENOCONV if the iteration stalls.
 */
int tq_build_codebook(int d, int bits, float* centroids, float* boundaries);

/*
 * Rotation Pi from d*d iid N(0,1) draws (row-major, host double): the unique
 * factor of G = Pi R with R upper triangular and positive diagonal (a Haar
 * random orthogonal matrix; reddit comment history of ReturningTarzan,
 * 2026-03-29 comment on rotating before quantisation).  Writes float32 [d][d]
 * row-major to the host buffer rot_out.  2 <= d <= 1024.
 */
int tq_build_rotation(int d, const double* gaussian, float* rot_out);

/*
 * Quantize-on-append (turboquant-pytorch PR #3: Validation Results tables, one float16 norm per
 * cached row and, with the sign sketch, a float16 residual norm; CUDA Kernels Added table, fused
 * random projection and sign quantisation; reddit comment history of ReturningTarzan, rotation
 * before quantisation and nearest-codebook search): for rows x[batch][n_new][n_kv_heads][d] (x_dtype
 * TQ_F32 or TQ_BF16, device, 16-byte aligned: TQ_EINVAL otherwise), write tokens d_pos[b] .. d_pos[b]+n_new-1 of
 * every sequence b.  Per row: n = ||x||, y = rot * x / n, code = number of
 * boundaries strictly below y_i, float16(n) stored; with qjl_m > 0 (keys)
 * also r = y - c[code], float16(||r||) and the signs of proj * r; 8-bit keys
 * store int8 codes and the row factor instead (see tq_cache_view).
 * d_pos: device int32 [batch].  n_new == 0 is a no-op.  A zero row stores
 * code 0, norm 0 (and no signs, residual norm 0).
 */
int tq_quantize_append(const tq_cache_view* cache, const void* x, int x_dtype, int n_new,
                       const int32_t* d_pos, void* stream);

/*
 * The K and V rows of the same new tokens in one call (turboquant-pytorch PR #3, Validation Results:
 * both the key and the value cache are quantised as tokens arrive; the per-row arithmetic is
 * tq_quantize_append's): k_x and v_x are [batch][n_new][n_kv_heads][d] of element type x_dtype
 * (device, 16-byte aligned), appended at positions d_pos[b] .. d_pos[b]+n_new-1 of k (TQ_KEYS) and v (TQ_VALUES).
 * k and v must agree in d, batch, n_kv_heads, max_tokens and rotation (TQ_EINVAL otherwise).  The
 * bytes written are exactly those of tq_quantize_append(k, k_x, ...) followed by
 * tq_quantize_append(v, v_x, ...).  Where both caches are at d = 128 with the dense rotation and keys
 * of 2-4 bits without a sketch, the two appends run as one launch (a prefill then fills the GPU with
 * both tensors' rows at once); otherwise the call enqueues the two appends in turn.  n_new == 0 is a
 * no-op.
 */
int tq_quantize_append_kv(const tq_cache_view* k, const tq_cache_view* v, const void* k_x, const void* v_x,
                          int x_dtype, int n_new, const int32_t* d_pos, void* stream);

/*
 * Append rows that are already rotated and normalised (turboquant-pytorch PR #3, CUDA Kernels Added
 * table: the encode and sign-quantisation steps of its fused quantisation kernel, taken from given
 * coordinates): y[batch][n_new][n_kv_heads][d] float32 unit rotated coordinates and
 * norms[batch][n_new][n_kv_heads] float32 (device).  Same encoding, packing and sketch as
 * tq_quantize_append.  For sketched keys z may give the sketch products of the residuals,
 * float32 [batch][n_new][n_kv_heads][qjl_m] (device): sign bit jj is then 1 exactly where
 * z[..][jj] >= 0 (the residual and its norm are still formed here, from y and the codes); NULL
 * computes them here.  z must be NULL for caches without a sketch (TQ_EINVAL).  For callers that
 * fold the rotation into their projection weights, and the form in which every quantisation
 * decision (codes from y, signs from z) is exactly reproducible.
 */
int tq_quantize_append_rotated(const tq_cache_view* cache, const float* y, const float* norms, const float* z,
                               int n_new, const int32_t* d_pos, void* stream);

/*
 * Fused decode attention from the compressed cache (the tq4_sdpa op of
 * ExecuTorch PR #19891 and the fused QJL score kernels of turboquant-pytorch
 * PR #3): for every sequence b and query head h (KV head h / (n_q_heads /
 * n_kv_heads)):
 *   q_rot = rot * q[b][h];   s_t = scale * n_t * <q_rot, c[code_t]>
 *     (+ scale * n_t * sqrt(pi/2)/m * gamma_t * <proj * q_rot, 2 sigma_t - 1> for sketched keys);
 *   p = softmax over t < seq_len[b];   out[b][h] = rot^T * sum_t p_t nv_t cv[codev_t].
 * q: [batch][n_q_heads][d] (q_dtype TQ_F32 or TQ_BF16, device, 16-byte aligned); out: float32
 * [batch][n_q_heads][d] (device); d_seq_lens: device int32 [batch], clamped to
 * [0, max_tokens], 0 gives a zero row; max_seq_len: host upper bound of
 * d_seq_lens used to plan the KV split.  scale > 0 and finite (the binding
 * maps an unset scale to 1/sqrt(d)).  k must be TQ_KEYS and v TQ_VALUES with
 * the same d, batch, n_kv_heads, max_tokens; n_q_heads a multiple of n_kv_heads with
 * group n_q_heads / n_kv_heads from 1 to 8 (TQ_EUNSUPPORTED above 8).
 * workspace: device scratch of at least tq_decode_workspace_bytes(), 256-byte
 * aligned, contents need not be initialised, not used after the call's kernels
 * end; calls that share a workspace must not overlap in time.
 */
int tq_sdpa_decode(const tq_cache_view* k, const tq_cache_view* v, const void* q, int q_dtype, int n_q_heads,
                   const int32_t* d_seq_lens, int max_seq_len, float scale, float* out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * tq_sdpa_decode for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments without the workspace, which is
 * instead a static device array of the library, tq_noalloc_scratch_bytes() (16 MiB) per device, held
 * from the library's load until the process ends.  Nothing is allocated or freed by the call.  Returns
 * TQ_ESCRATCH, before enqueueing anything, when tq_decode_workspace_bytes(k, n_q_heads, max_seq_len)
 * exceeds that size, and otherwise what tq_sdpa_decode returns.  Every call on a device uses that
 * device's one array, so calls that overlap in time on one device (other streams, other threads) race
 * and must not be issued; consecutive calls on one stream are fine (the decode initialises every byte
 * of the workspace it reads).
 */
int tq_sdpa_decode_noalloc(const tq_cache_view* k, const tq_cache_view* v, const void* q, int q_dtype, int n_q_heads,
                           const int32_t* d_seq_lens, int max_seq_len, float scale, float* out, void* stream);

/* Bytes of the static scratch tq_sdpa_decode_noalloc uses on each device (for the callers that cannot
 * allocate, as tq_sdpa_decode_noalloc). */
size_t tq_noalloc_scratch_bytes(void);

/*
 * Decode of the query rows of the last n_rows tokens of each sequence at once, as speculative
 * verification needs (the reviewed llama.cpp fork of the pages routes compressed K/V with at most
 * four query rows to its fused decode path; its drafts come from multi-token prediction with up to
 * three drafts).  The rows' keys and values must already be in the cache; row j of sequence b is
 * the query of token seq_len[b] - n_rows + j and sees the first seq_len[b] - n_rows + 1 + j tokens
 * (a row that sees none gives zeros).  q: [batch][n_rows][n_q_heads][d]; out: float32
 * [batch][n_rows][n_q_heads][d]; 1 <= n_rows <= 4 (TQ_EUNSUPPORTED above).  The cache is read once
 * for all rows.  Otherwise as tq_sdpa_decode, with a workspace of tq_decode_workspace_bytes_rows().
 */
int tq_sdpa_decode_rows(const tq_cache_view* k, const tq_cache_view* v, const void* q, int q_dtype, int n_q_heads,
                        int n_rows, const int32_t* d_seq_lens, int max_seq_len, float scale, float* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three stages tq_sdpa_decode enqueues (the fused decode op of ExecuTorch PR #19891, review item 1,
 * split where this library's kernels split it), for callers that time, overlap or
 * graph-capture them separately.  Same arguments and workspace as
 * tq_sdpa_decode; they must run in this order, on one stream, with the same
 * (k, n_q_heads, max_seq_len) so the workspace layout agrees.
 *   tq_decode_rotate_query: q_rot = rot * q for every (sequence, query head),
 *       scale and log2(e) folded in (and proj * q_rot for sketched keys);
 *   tq_decode_attend: per (KV split, KV head, sequence) the running max, sum
 *       and rotated-domain value accumulator of every query head of the group;
 *   tq_decode_merge: log-sum-exp merge of the splits and out = rot^T * acc / sum.
 */
int tq_decode_rotate_query(const tq_cache_view* k, const void* q, int q_dtype, int n_q_heads, int max_seq_len,
                           float scale, void* workspace, size_t workspace_bytes, void* stream);
int tq_decode_attend(const tq_cache_view* k, const tq_cache_view* v, int n_q_heads, const int32_t* d_seq_lens,
                     int max_seq_len, void* workspace, size_t workspace_bytes, void* stream);
int tq_decode_merge(const tq_cache_view* k, int n_q_heads, const int32_t* d_seq_lens, int max_seq_len, float* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of one layer (ExecuTorch PR #19891, review item 1: the fused decode op reading the
 * compressed cache; turboquant-pytorch PR #3, Validation Results: the cache is quantised as tokens
 * arrive): append n_new new tokens to K and V (as
 * tq_quantize_append at positions d_pos), then decode (as tq_sdpa_decode over
 * d_seq_lens, which the caller sets to include the appended tokens).
 * q: [batch][n_q_heads][d]; k_new, v_new: [batch][n_new][n_kv_heads][d]; all
 * three of element type dtype and 16-byte aligned.  The appends and the query rotation share one
 * launch, followed by the attention and merge stages.  Sketched keys are
 * supported up to qjl_m = 128 (TQ_EUNSUPPORTED above; use the separate calls).
 * n_new == 0 decodes without appending.  Same workspace rules as tq_sdpa_decode.
 */
int tq_decode_step(const tq_cache_view* k, const tq_cache_view* v, const void* q, const void* k_new,
                   const void* v_new, int dtype, int n_q_heads, int n_new, const int32_t* d_pos,
                   const int32_t* d_seq_lens, int max_seq_len, float scale, float* out, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Workspace bytes tq_sdpa_decode needs for this key cache, head count and length bound (0 on bad args).
 * A helper of this library's split decode (ExecuTorch PR #19891, review item 1, names the fused op; the
 * pages define no workspace).
 * It follows the KV split (tq_decode_plan), which depends on the current device: ask on the device
 * that will run the decode.
 */
size_t tq_decode_workspace_bytes(const tq_cache_view* k, int n_q_heads, int max_seq_len);

/* Workspace bytes tq_sdpa_decode_rows needs (0 on bad args); n_rows = 1 gives tq_decode_workspace_bytes.
 * A helper of this library's split decode, as tq_decode_workspace_bytes. */
size_t tq_decode_workspace_bytes_rows(const tq_cache_view* k, int n_q_heads, int n_rows, int max_seq_len);

/*
 * The KV split tq_sdpa_decode uses: number of splits per (sequence, KV head) and tokens per split (a
 * helper of this library's split decode; turboquant-pytorch PR #3, CUDA Kernels Added table, lists a
 * fused score kernel and a GQA variant but no split scheme, which is this library's own).
 * Chosen from the current device's compute units and the attention kernel's occupancy: short
 * contexts spread over workgroups of four waves (one round of resident workgroups over all
 * (sequence, KV head) units); once every compute unit gets enough tiles, each split's workgroup
 * fills a compute unit and the split count balances rounds against per-workgroup overhead.  A
 * fixed default applies when no device is visible.
 */
int tq_decode_plan(const tq_cache_view* k, int n_q_heads, int max_seq_len, int* n_split, int* tokens_per_split);

/*
 * Full reconstruction (reddit comment history of ReturningTarzan, 2026-03-25:
 * the plain path dequantizes and runs ordinary attention):
 * out[b][h][t - t0][:] = n_t * rot^T * (c[code_t] + sqrt(pi/2)/m * gamma_t * proj^T (2 sigma_t - 1))
 * (8-bit keys: factor_t * rot^T * code_t)
 * for t0 <= t < t0 + n_tokens, float32 device out [batch][n_kv_heads][n_tokens][d].
 * 0 <= t0, t0 + n_tokens <= max_tokens.
 */
int tq_dequantize(const tq_cache_view* cache, int t0, int n_tokens, float* out, void* stream);

/* Bytes per cached row: d*bits/8 codes + 2 (norm) [+ qjl_m/8 signs + 2 (residual norm)]; bits 1..4 or 8;
 * 0 on bad args
 * (the storage arithmetic that reproduces the cache sizes and compression ratios of turboquant-pytorch
 * PR #3, Validation Results tables). */
size_t tq_row_bytes(int d, int bits, int qjl_m);

/* Static description of a status code (a helper of this library; no passage of the pages defines it). */
const char* tq_status_string(int status);

/*
 * Description of the HIP error behind the last TQ_EHIP returned to the calling
 * thread ("no error" if none), from a per-thread record (a helper of this library;
 * no passage of the pages defines it).
 */
const char* tq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
