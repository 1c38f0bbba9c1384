/*
 * tq.h — C ABI of the MI355X (gfx950) library for online KV-vector
 * quantization and decode attention computed from the packed codes.
 *
 * Method (web pages, cited by title and section):
 *  [WIT]  "什么是TurboQuant？谷歌突破性AI压缩技术实现6倍KV缓存缩减和8倍推理加速"
 *         (a2a-mcp.org blog, "What is TurboQuant?"):
 *         - "TurboQuant 工作原理" > "第一阶段" item 1: one data-independent random
 *           orthogonal rotation (QR of a Gaussian matrix); rotated coordinates
 *           follow Beta((d-1)/2,(d-1)/2) on [-1, 1].
 *         - "第一阶段" item 2: normalise the vector; a Lloyd-Max quantizer that
 *           is MSE-optimal for that law gives a few bits per coordinate.
 *         - "第二阶段：QJL 残差校正": a 1-bit quantized Johnson-Lindenstrauss
 *           sketch of the residual corrects inner-product bias.
 *         - "如何实现 TurboQuant" item 1: the codebook is precomputed per head
 *           dimension and bit width; vectors are quantized on every cache
 *           update; the query is rotated once and attention dot products are
 *           taken straight from the stored indices.
 *  [VLLM] "A First Comprehensive Study of TurboQuant: Accuracy and
 *         Performance" (papercache.org), section A3: variants k8v4, 4bit_nc,
 *         k3v4_nc, 3bit_nc (nc = norm correction).
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller, unless a
 *    parameter says "host".  The library owns only tq_codebook objects.
 *  - Calls that take a `stream` (a hipStream_t passed as void*; NULL = the
 *    default stream) only enqueue work on it and return before it runs; the
 *    other calls are synchronous.
 *  - Every call returns a tq_status.  On failure nothing has been enqueued
 *    and tq_last_error() returns a message (thread-local, valid until the
 *    next failing call on the same thread).  No C++ exception crosses the ABI.
 *  - Non-finite inputs are undefined behaviour (not checked on the hot path).
 *  - Only tq_codebook_build allocates device memory.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID = 1,     /* bad argument (null, out of range, inconsistent) */
  TQ_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for    */
  TQ_ERR_HIP = 3,         /* a HIP runtime call failed                        */
  TQ_ERR_ALLOC = 4,       /* device or host allocation failed                 */
  TQ_ERR_NUMERIC = 5      /* codebook solver did not converge                 */
} tq_status;

/* Element types.  Calls take a dtype as int32_t holding one of these values
 * (any other value is rejected with TQ_ERR_INVALID). */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* Code layouts (the pages only say "bit-packed"; both are LSB-first).
 *  TQ_LAYOUT_ROW: vector v of sequence s is row r = s*seq_stride + v.
 *    idx  row r at idx + r*idx_row_bytes: coordinate i at bits [i*b, i*b+b)
 *         of a little-endian bit stream (bit p in byte p>>3, position p&7),
 *         zero bits after coordinate d-1.  Minimum idx_row_bytes is
 *         4*b*ceil(d/32).
 *    sign row r at sign + r*sign_row_bytes: sketch row j at bit j, zero bits
 *         after j = m-1.  Minimum sign_row_bytes is 4*ceil(m/32).
 *  TQ_LAYOUT_TILE32 (value codes for decode): sequence s is cut into blocks
 *    of 32 vectors of BB = 64*ceil(d/16)*b bytes; block k of sequence s
 *    starts at idx + (s*(seq_stride/32) + k)*BB.  Inside a block, index i of
 *    vector t (0..31) sits at bits [p, p+b) of the block's little-endian bit
 *    stream with p = ((r*ceil(d/16) + i/16)*8 + e)*b, r = 16*((t%16)/4) + i%16,
 *    e = t%4 + 4*(t/16): 64 records, each holding 8 vectors x ceil(d/16)
 *    groups of 16-strided coordinates.  Padding bits are zero.  seq_stride
 *    must be a multiple of 32; idx_row_bytes is ignored.  Sign codes are not
 *    supported in this layout.
 *  scale[r] / rnorm[r] (fp32) are indexed by r = s*seq_stride + v in both. */
typedef enum { TQ_LAYOUT_ROW = 0, TQ_LAYOUT_TILE32 = 1 } tq_layout;

typedef struct tq_codebook tq_codebook; /* opaque; immutable after build */

/* Everything a codebook is a pure function of.
 *  d               vector length, 3..256
 *  bits            Lloyd-Max bits per coordinate, 1..8 (L = 2^bits levels)
 *  qjl_m           QJL sketch rows, 0 (off) or 1..256
 *  norm_correction 0: scale = |x|; 1: scale = |x| / |c[idx]| (nc variants)
 *  rot_seed        seed of the Gaussian matrix whose QR gives the rotation
 *  qjl_seed        seed of the Gaussian sketch matrix S (m x d)           */
typedef struct {
  int32_t d, bits, qjl_m, norm_correction;
  uint64_t rot_seed, qjl_seed;
} tq_params;

/* Caller-owned code planes of one tensor (keys or values).
 *  idx    packed indices (layout above)                       device
 *  sign   packed QJL sign bits, NULL iff the codebook's qjl_m == 0
 *  scale  fp32 per vector: |x| (or |x|/|c[idx]| with nc)
 *  rnorm  fp32 per vector: |x| * |r| (QJL residual norm), NULL iff qjl_m == 0
 *  idx_row_bytes, sign_row_bytes  row pitch (ROW layout), multiple of 4
 *  seq_stride  capacity in vectors per sequence
 *  layout      a tq_layout                                                */
typedef struct {
  void* idx;
  void* sign;
  float* scale;
  float* rnorm;
  int64_t idx_row_bytes;
  int64_t sign_row_bytes;
  int64_t seq_stride;
  int32_t layout;
  int32_t reserved;
} tq_codes;

/* Builds a codebook on the host and uploads it to the current HIP device
 * ([WIT] 第一阶段 items 1-2; 如何实现 item 1):
 *  - Lloyd-Max centroids c[0..L-1] and boundaries t_k = (c[k-1]+c[k])/2 for
 *    the density f_d(y) = (1-y^2)^((d-3)/2) / B(1/2,(d-1)/2) on [-1, 1];
 *  - rotation Pi = Q of G = QR with diag(R) > 0, G (d x d, row-major) drawn
 *    by splitmix64(rot_seed) + Box-Muller (cosine branch);
 *  - S (m x d, row-major) drawn the same way from qjl_seed.
 * Synchronous.  On success *out owns device memory until
 * tq_codebook_destroy.  Errors: TQ_ERR_INVALID (params), TQ_ERR_NUMERIC,
 * TQ_ERR_ALLOC / TQ_ERR_HIP (upload). */
tq_status tq_codebook_build(const tq_params* params, tq_codebook** out);

/* Frees a codebook (NULL is accepted).  The caller must make sure no
 * enqueued call still uses it.  Synchronous. */
tq_status tq_codebook_destroy(tq_codebook* cb);

/* Copies the codebook's float64 values to HOST buffers (any may be NULL):
 * centroids[L], boundaries[L-1], rot[d*d] (row-major Pi), qjl[m*d]. */
tq_status tq_codebook_export(const tq_codebook* cb, double* centroids, double* boundaries,
                             double* rot, double* qjl);

/* Host only (no device is touched): computes the float64 values a codebook
 * with these params holds, into HOST buffers (any may be NULL):
 * centroids[L], boundaries[L-1], rot[d*d] (row-major Pi), qjl[m*d].
 * Same construction and errors as tq_codebook_build. */
tq_status tq_codebook_values(const tq_params* params, double* centroids, double* boundaries,
                             double* rot, double* qjl);

/* Iteration limits of the Lloyd-Max solve behind tq_codebook_build and
 * tq_codebook_values on the calling thread (host only): at most lloyd_iters
 * Lloyd steps (midpoint then centroid condition), then at most newton_iters
 * Newton steps on the midpoint residual; a solve whose residual is not below
 * 1e-12 then fails with TQ_ERR_NUMERIC.  A value <= 0 restores that limit's
 * default (400000 and 80, enough for every d in 3..256 and bits in 1..8).
 * Meant for exercising the error path; never fails. */
tq_status tq_codebook_solver_limits(int32_t lloyd_iters, int32_t newton_iters);

/* ---- PolarQuant codebooks ([WIT] "TurboQuant 工作原理" > "第一阶段：随机旋转 +
 * PolarQuant 压缩" item 2: the rotated, normalised vector is carried to polar
 * form by pairing dimensions recursively; the angles' law is known in
 * advance and each angle gets a Lloyd-Max code for it).
 * With y = Pi x / |x| (d a power of two): level 1 pairs coordinates,
 * angle atan2(y[2i+1], y[2i]) in [-pi, pi] (uniform law: b1-bit uniform
 * quantizer, centroids at cell centres); level l >= 2 pairs the radii of
 * level l-1, angle atan2(r[2i+1], r[2i]) in [0, pi/2], whose sin^2 follows
 * Beta(k/2, k/2) with k = 2^(l-1) (br-bit Lloyd-Max quantizer).  The last
 * radius is |y| = 1; scale = |x|.  The reconstruction y_hat (rebuilt
 * top-down from radius 1, |y_hat| = 1) replaces c[idx]; with QJL the
 * residual is r = y - y_hat.  Codes: ROW layout only, one little-endian bit
 * stream per vector, level-major (the d/2 level-1 fields of b1 bits, then
 * the d/4 level-2 fields of br bits, ..., the single top field), row pitch
 * at least 4 ceil(T/32) bytes with T = (d/2) b1 + (d/2 - 1) br.
 *  d           power of two, 4..128 on the GPU (2..256 host values)
 *  bits_first  b1, 1..8;  bits_rest  br, 1..8;  qjl_m 0 or 1..128
 * A polar codebook works with tq_quantize_kv (and _paged), tq_dequantize,
 * tq_code_row_bytes, tq_codebook_export (per-level values concatenated:
 * centroids level 1 then 2 ..., boundaries likewise) and, as the key
 * codebook of tq_attn_decode (and _paged, _noalloc) with d = 128, b1 = 4,
 * br = 2 and a scalar value codebook; tq_ip_topk rejects it
 * (TQ_ERR_UNSUPPORTED). */
typedef struct {
  int32_t d, bits_first, bits_rest, qjl_m;
  uint64_t rot_seed, qjl_seed;
} tq_polar_params;

/* Builds a polar codebook on the host (angle codebooks in float64, the
 * rotation and sketch as tq_codebook_build) and uploads it to the current
 * device.  Synchronous.  Errors: TQ_ERR_INVALID, TQ_ERR_NUMERIC,
 * TQ_ERR_ALLOC / TQ_ERR_HIP. */
tq_status tq_polar_codebook_build(const tq_polar_params* params, tq_codebook** out);

/* Host only: the float64 values a polar codebook holds, into HOST buffers
 * (any may be NULL): centroids and boundaries of every level concatenated
 * (level 1 first; 2^b1 + (log2 d - 1) 2^br centroids, one fewer boundary per
 * level), rot[d*d], qjl[m*d]. */
tq_status tq_polar_codebook_values(const tq_polar_params* params, double* centroids, double* boundaries,
                                   double* rot, double* qjl);

/* Minimum ROW-layout pitches for this codebook: 4*bits*ceil(d/32) (polar:
 * 4*ceil(T/32)) and 4*ceil(m/32) (0 when qjl_m == 0). */
tq_status tq_code_row_bytes(const tq_codebook* cb, int64_t* idx_row_bytes,
                            int64_t* sign_row_bytes);

/* Online quantization of a batch of key and/or value vectors
 * ([WIT] 第一阶段, 第二阶段; 如何实现 item 1: quantize at each cache update):
 * for each vector x: n = |x|, y = Pi x / n (y = 0 if n = 0),
 * idx_i = #{k : y_i >= t_k}, scale = n (nc: n/|c[idx]|); with QJL,
 * r = y - (scale/n) c[idx], sign_j = [(S r)_j >= 0], rnorm = n |r|.
 *  k, v        inputs [n_seq][n_tok][d] contiguous, dtype dt; v may be NULL
 *              (then vcb and v_out are ignored); k may be NULL likewise.
 *              n_seq == 0 or n_tok == 0 is a no-op that returns TQ_OK.
 *  tok_offset  vector t of the input goes to position tok_offset + t of its
 *              sequence; tok_offset + n_tok <= seq_stride.  Codes of other
 *              positions are left untouched (tile32 blocks are updated by
 *              read-modify-write; calls on one stream are ordered).
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED (layout/d combination),
 * TQ_ERR_HIP (launch). */
tq_status tq_quantize_kv(const tq_codebook* kcb, const tq_codebook* vcb, const void* k,
                         const void* v, int32_t dt, int64_t n_seq, int64_t n_tok,
                         int64_t tok_offset, const tq_codes* k_out, const tq_codes* v_out,
                         void* stream);

/* Workspace bytes tq_attn_decode needs for this shape (host only); d in
 * 3..256 (TQ_ERR_INVALID otherwise), valid for any codebooks of that d. */
tq_status tq_attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_ctx,
                                   int32_t d, size_t* bytes);

/* Decode attention straight from packed codes ([WIT] 如何实现 item 1; 专业提示):
 * per query head hq of batch b (KV head h = hq / (Hq/Hkv), sequence
 * s = b*Hkv + h), with q~ = Pi_K q:
 *   logit_j = sm_scale * ( scaleK_j <q~, cK[idxK_j]>
 *                          + sqrt(pi/2)/m rnormK_j <S_K q~, 2 sign_j - 1> )
 *   p = softmax over j < len_b (no mask otherwise)
 *   out = Pi_V^T sum_j p_j scaleV_j cV[idxV_j]
 *  q         [B][Hq][d], dtype qdt
 *  k         key codes, TQ_LAYOUT_ROW; v value codes, TQ_LAYOUT_TILE32;
 *            both with seq_stride a multiple of 32 and >= n_ctx
 *  seq_lens  device int32 [B] with 0 <= len_b <= n_ctx, or NULL (all n_ctx);
 *            len_b = 0 gives out = 0 and logits -inf
 *  out       fp32 [B][Hq][d]
 *  logits    fp32 [B][Hq][n_ctx] or NULL; -inf for j >= len_b
 *  workspace device scratch of >= tq_attn_decode_workspace bytes
 * Kernels: d = 128 with key and value codes of 2, 3, 4 or 8 bits and
 * qjl_m <= 128 run on bf16 hi/lo MFMA (about 2^-16 relative per product);
 * every other scalar shape (d <= 256, 1..8 bits, qjl_m <= 256) on fp32 FMAs.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED (polar codebooks other than
 * (4, 2) keys at d = 128 with qjl_m <= 128 and scalar values of 2, 3, 4 or
 * 8 bits), TQ_ERR_HIP. */
tq_status tq_attn_decode(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                         int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv, const tq_codes* k,
                         const tq_codes* v, const int32_t* seq_lens, int64_t n_ctx,
                         float sm_scale, float* out, float* logits, void* workspace,
                         size_t ws_bytes, void* stream);

/* One decode step: append the step's new keys and values to the caches,
 * then attend ([WIT] 如何实现 item 1: quantize at each cache update, rotate
 * the query once, attention from the indices).  Same results as
 * tq_quantize_kv(kcb, vcb, k_new, v_new, kv_dtype, B*Hkv, n_new, tok_offset,
 * k, v, stream) followed by tq_attn_decode(...) with the remaining
 * arguments; the query prologue of the d = 128 kernels then runs in the
 * append launch instead of a launch of its own.
 *  k_new, v_new  device [B*Hkv][n_new][d] (sequence s = b*Hkv + h), dtype
 *                kv_dtype, both required; written to positions
 *                [tok_offset, tok_offset + n_new) with tok_offset + n_new <= n_ctx
 *  other arguments as tq_attn_decode (workspace: tq_attn_decode_workspace)
 * Every argument of both parts is checked before anything is launched.
 * Errors: those of tq_quantize_kv and tq_attn_decode. */
tq_status tq_attn_decode_append(const tq_codebook* kcb, const tq_codebook* vcb, const void* k_new,
                                const void* v_new, int32_t kv_dtype, int64_t n_new, int64_t tok_offset,
                                const void* q, int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv,
                                const tq_codes* k, const tq_codes* v, const int32_t* seq_lens, int64_t n_ctx,
                                float sm_scale, float* out, float* logits, void* workspace, size_t ws_bytes,
                                void* stream);

/* tq_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same computation, arguments, results and errors as tq_attn_decode, but
 * with no workspace argument: the scratch it needs (the rotated query
 * operands and the split partials, the same bytes tq_attn_decode_workspace
 * reports) lives in a fixed 8 MiB device array inside the library, one per
 * device, kept until the process ends.  The call allocates nothing and
 * records no profiling events.
 *  - Shapes whose scratch exceeds 8 MiB fail with TQ_ERR_UNSUPPORTED before
 *    anything is enqueued (the 128K layer, B=8, Hq=64, Hkv=8, needs 1.9 MB).
 *  - Every call on a device uses that device's one array, which keeps the
 *    last call's contents (no part of it needs to start zeroed).  Calls
 *    ordered on one stream are safe; calls that may overlap in time on one
 *    device (several streams or threads) race and give wrong results.
 *  - The array's address is looked up on the first call on each device. */
tq_status tq_attn_decode_noalloc(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                                 int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv, const tq_codes* k,
                                 const tq_codes* v, const int32_t* seq_lens, int64_t n_ctx,
                                 float sm_scale, float* out, float* logits, void* stream);

/* ---- Paged pools.  A serving engine keeps its cache in fixed-size pages
 * (the pages present TurboQuant as a KV-cache dtype of such an engine,
 * [VLLM] A3 方法细节, quantized at every cache update, [WIT] 如何实现
 * item 1).  A pool is a tq_codes whose sequence h (0 <= h < Hkv) is the
 * plane of KV head h; its seq_stride is n_pages * page_tokens and page p of
 * head h holds plane positions [p * page_tokens, (p + 1) * page_tokens).
 *  block_table  device int32 [B][max_pages]: logical page i (positions
 *               [i * page_tokens, (i + 1) * page_tokens)) of batch b is
 *               pool page block_table[b * max_pages + i], the same page id
 *               for every KV head.  Entries outside [0, n_pages) are clamped
 *               (the result is then wrong, but no access leaves the pool).
 *  page_tokens  a power of two in 32..65536; pools' seq_stride a multiple.
 * The pool buffers must hold Hkv planes (Hkv * seq_stride positions). */

/* tq_quantize_kv into paged pools: inputs k, v [B*Hkv][n_tok][d] (sequence
 * b*Hkv + h), vector t of sequence (b, h) goes to logical position
 * tok_offset + t of batch b, KV head h, i.e. through block_table into plane
 * h of k_pool / v_pool.  max_pages * page_tokens >= tok_offset + n_tok.
 * Otherwise as tq_quantize_kv (same kernels, same codes). */
tq_status tq_quantize_kv_paged(const tq_codebook* kcb, const tq_codebook* vcb, const void* k,
                               const void* v, int32_t dt, int64_t B, int64_t Hkv, int64_t n_tok,
                               int64_t tok_offset, const int32_t* block_table, int64_t max_pages,
                               int32_t page_tokens, const tq_codes* k_pool, const tq_codes* v_pool,
                               void* stream);

/* Workspace bytes tq_attn_decode_paged needs for this shape (host only). */
tq_status tq_attn_decode_paged_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_ctx, int32_t d,
                                         int32_t page_tokens, size_t* bytes);

/* tq_attn_decode over paged pools: the keys and values of batch b, KV head h
 * at logical positions j < len_b are read through block_table from plane h
 * of k_pool (TQ_LAYOUT_ROW) and v_pool (TQ_LAYOUT_TILE32).
 * max_pages * page_tokens >= n_ctx; workspace >= tq_attn_decode_paged_workspace.
 * Same results as tq_attn_decode on the same codes laid out contiguously, up
 * to the order of the split-K partial sums (each wave covers whole pages). */
tq_status tq_attn_decode_paged(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                               int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv, const tq_codes* k_pool,
                               const tq_codes* v_pool, const int32_t* block_table, int64_t max_pages,
                               int32_t page_tokens, const int32_t* seq_lens, int64_t n_ctx, float sm_scale,
                               float* out, float* logits, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes tq_ip_topk needs (host only); valid for any qjl_m of a
 * codebook with this d. */
tq_status tq_ip_topk_workspace(int64_t nq, int64_t n_db, int32_t k, int32_t d, size_t* bytes);

/* Inner-product top-k over coded vectors ([WIT] 基准测试与实际性能表现: the
 * top-k recall evaluation of vector search at d = 200; the estimate of
 * 第二阶段: QJL 残差校正).  The score of database vector j for
 * query q (fp32 [d]) is
 *   s_j = scale_j <Pi q, c[idx_j]> + sqrt(pi/2)/m rnorm_j <S Pi q, 2 sign_j - 1>
 * (the QJL term only when qjl_m > 0), the unbiased estimate of <q, x_j>.
 *  queries   device fp32 [nq][d], row-major
 *  db        database codes, TQ_LAYOUT_ROW, vectors 0..n_db-1 of sequence 0
 *            (idx_row_bytes <= 256, sign_row_bytes <= 32)
 *  k         1..32, k <= n_db (k == 0 or nq == 0: no-op)
 *  out_idx   device int64 [nq][k]: indices by descending score, ties to the
 *            lower index
 *  out_score device fp32 [nq][k]: their scores
 *  workspace device scratch of >= tq_ip_topk_workspace bytes, 256-byte aligned
 * The result is the exact top-k of s_j evaluated in float64 from the codes
 * (Pi q and S Pi q formed in float64), and out_score is that float64 score
 * rounded to fp32.  An MFMA pass keeps kc candidates per query (kc = 16 for
 * k <= 10, else min(2k, 64); fp16 operands, each query scaled by a power of
 * two, for kc <= 32, bf16 hi/lo beyond); the candidates are rescored in
 * float64, and a query is settled when the kc-th approximate score plus a
 * bound on the approximate score's error (over every row of the database)
 * stays below the k-th exact score.  Other queries (near-ties at the k-th
 * place, repeated rows) are answered by an exact float64 scan of the
 * database.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED (k > 32, oversized rows),
 * TQ_ERR_HIP. */
tq_status tq_ip_topk(const tq_codebook* cb, const float* queries, int64_t nq,
                     const tq_codes* db, int64_t n_db, int32_t k, int64_t* out_idx,
                     float* out_score, void* workspace, size_t ws_bytes, void* stream);

/* Diagnostic: the number of queries of the last tq_ip_topk call made with
 * this workspace (and the same cb, nq, n_db, k) that the exact scan
 * answered.  Reads 4 bytes of the workspace on `stream` and waits for it.
 * Errors: TQ_ERR_INVALID, TQ_ERR_HIP. */
tq_status tq_ip_topk_scan_count(const tq_codebook* cb, const void* workspace, int64_t nq, int64_t n_db,
                                int32_t k, void* stream, int64_t* count);

/* Diagnostic switch of tq_ip_topk (process-wide, default 0): 1 sends every
 * query to the exact float64 scan, skipping the candidates' test, so the
 * scan can be checked and timed on any input; 0 restores the default.
 * Errors: TQ_ERR_INVALID (other values). */
tq_status tq_ip_topk_exact_scan(int32_t always);

/* Vectors back from their codes: the decompress half of the compress /
 * decompress pair of [AGENT] 三、工程实现 item 1, computing the estimate of
 * [WIT] 工作原理 > 第一阶段 items 1-2 and 第二阶段：QJL 残差校正 in the original
 * domain:
 *   x_hat = Pi^T ( scale c[idx] + sqrt(pi/2)/m rnorm S^T (2 sign - 1) )
 * (the sketch term only when qjl_m > 0), so <q, x_hat> is the estimate that
 * tq_attn_decode and tq_ip_topk form from the codes.
 *  codes       positions [tok_offset, tok_offset + n_tok) of sequences
 *              0..n_seq-1, ROW or TILE32 layout as tq_quantize_kv writes them
 *              (tok_offset + n_tok <= seq_stride)
 *  out         device [n_seq][n_tok][d] of out_dt (TQ_F32, TQ_BF16 or TQ_F16;
 *              the 16-bit types round to nearest even), 16-byte aligned
 *  n_seq == 0 or n_tok == 0 is a no-op that returns TQ_OK.
 * With d == 128 and qjl_m <= 128 the contractions run on bf16 MFMA with
 * two-part (hi + lo) splits of Pi, of the centroids and of the sketch
 * operand (about 2^-16 relative to |x_hat|); other shapes use fp32 FMAs.
 * Errors: TQ_ERR_INVALID, TQ_ERR_HIP. */
tq_status tq_dequantize(const tq_codebook* cb, const tq_codes* codes, int64_t n_seq,
                        int64_t n_tok, int64_t tok_offset, void* out, int32_t out_dt,
                        void* stream);

/* Kernel timing (instrumentation; not part of the method).
 * tq_profile_enable(1) clears the calling thread's records and starts
 * recording: every later tq_quantize_kv / tq_attn_decode / tq_ip_topk /
 * tq_dequantize on this thread
 * records a hipEvent pair on its stream around each launch of its main
 * kernel (the quantize kernel, once per tensor; the decode split kernel;
 * the top-k score kernel; the dequantize kernel).
 * tq_profile_enable(0) stops recording and keeps the records.
 * tq_profile_read waits for the recorded events and returns the summed
 * elapsed milliseconds and the number of launches of one kernel
 * (TQ_KERNEL_QUANTIZE, TQ_KERNEL_DECODE_SPLIT, TQ_KERNEL_TOPK or
 * TQ_KERNEL_DEQUANTIZE).  Events are created by the
 * library (no device memory is allocated). */
typedef enum {
  TQ_KERNEL_QUANTIZE = 0,
  TQ_KERNEL_DECODE_SPLIT = 1,
  TQ_KERNEL_TOPK = 2,
  TQ_KERNEL_DEQUANTIZE = 3
} tq_kernel;
tq_status tq_profile_enable(int32_t on);
tq_status tq_profile_read(int32_t kernel, double* total_ms, int64_t* launches);

/* The same records one launch at a time: ms[i] (HOST buffer of capacity
 * entries) receives the elapsed milliseconds of launch i, for the first
 * min(capacity, launches) launches; *launches (may be NULL) the count. */
tq_status tq_profile_durations(int32_t kernel, double* ms, int64_t capacity, int64_t* launches);

/* Measurement helper (not part of the method): enqueues a kernel that only
 * reads `bytes` bytes of buf (device, 16-byte aligned, bytes a multiple of
 * 16) with 16-byte loads and writes sink[0] (device uint32) only when the XOR
 * of everything read equals a fixed value.  Its rate is the device's
 * streaming-read ceiling, the bound every memory-bound kernel here is read
 * against.  Errors: TQ_ERR_INVALID, TQ_ERR_HIP. */
tq_status tq_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* Measurement helper (not part of the method): enqueues a kernel that only
 * writes: every 32-bit word of the first `bytes` bytes of buf (device,
 * 16-byte aligned, bytes a multiple of 16) becomes `value`, with 16-byte
 * stores.  Its rate is the device's streaming-write ceiling, the bound of the
 * store-dominated kernels (dequantize).  Errors: TQ_ERR_INVALID, TQ_ERR_HIP. */
tq_status tq_stream_write(void* buf, int64_t bytes, uint32_t value, void* stream);

/* Message of the last failing call on this thread ("" if none).  With the
 * environment variable TQ_LOG set (to anything but "0") when the library is
 * first used, every hot-path call (codebook builds, quantize, decode, top-k,
 * dequantize) prints its arguments, and every failure its status and this
 * message, as one "[tq] ..." line on stderr. */
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
