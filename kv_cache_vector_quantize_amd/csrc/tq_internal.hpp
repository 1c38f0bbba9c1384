// Internal declarations shared by the C-ABI front end and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "tq.h"

namespace tq {

// float64 results of the host-side construction
struct HostCodebook {
  std::vector<double> centroids;   // [L]
  std::vector<double> boundaries;  // [L-1]
  std::vector<double> rot;         // [d*d] row-major Pi
  std::vector<double> qjl;         // [m*d] row-major S (empty when m == 0)
};

bool build_codebook_host(const tq_params& p, HostCodebook& out, std::string& err);

// PolarQuant codebook: centroids / boundaries of every angle level
// concatenated (level 1 first); cent_off[l] / bnd_off[l] (l = 1..levels+1)
// index level l's first entry.
bool build_polar_codebook_host(const tq_polar_params& p, HostCodebook& out, std::vector<int>& cent_off,
                               std::vector<int>& bnd_off, std::string& err);
// thread-local iteration limits of the Lloyd-Max solve (<= 0: default)
void set_solver_limits(int lloyd_iters, int newton_iters);

// Device-resident tables of one codebook.
struct DeviceCodebook {
  float* cent = nullptr;    // [L] fp32
  float* bnd = nullptr;     // [L-1] fp32
  float* rot = nullptr;     // [dp*dp] fp32 row-major Pi, zero-padded to dp
  float* qjl = nullptr;     // [mp*dp] fp32 row-major S, zero-padded (or null)
  float* rotT = nullptr;    // [dp*dp] fp32, rotT[k][i] = Pi[i][k]
  float* qjlT = nullptr;    // [dp*mp] fp32, qjlT[i][j] = S[j][i] (or null)
  // [dp*mp] fp32, sprotT[k][j] = sqrt(pi/2)/m * (S Pi)[j][k] (or null): the
  // sketch of a rotated query in one product, t = sqrt(pi/2)/m S (Pi q)
  float* sprotT = nullptr;
  // dequantize (dequantize.hip):
  //  sprot: [mp*dp] fp32 row-major sqrt(pi/2)/m (S Pi) (or null)
  //  dqop:  Pi^T as bf16 A operands of v_mfma_f32_32x32x16_bf16 in the layout
  //         of rop, columns permuted so that k-step s, lane half h, element j
  //         is column 64h + 8s + j (d = 128 only)
  //  dqs:   sqrt(pi/2)/m (S Pi)^T with column j scaled by 2^(127 - 2^(j % 8)),
  //         same layout and permutation, zero columns past m (d = 128, m <= 128)
  //  dqcs:  [128] fp32 column sums sum_j sqrt(pi/2)/m (S Pi)[j][k]
  float* sprot = nullptr;
  uint32_t* dqop = nullptr;
  uint32_t* dqs = nullptr;
  float* dqcs = nullptr;
  // decode operand tables (bf16 hi/lo split of the centroids):
  //  bits <= 4: entry e = a | (b << bits) holds two dwords
  //             {hi(c[a]) | hi(c[b]) << 16, lo(c[a]) | lo(c[b]) << 16}
  //  bits  > 4: entry a holds one dword {hi(c[a]) | lo(c[a]) << 16}
  uint32_t* pair_tab = nullptr;
  int pair_tab_dwords = 0;
  //  quad_tab (bits == 2): entry e = a | b << bits | c << 2 bits | d << 3 bits
  //  holds four dwords {hi(c[a]) | hi(c[b]) << 16, lo(c[a]) | lo(c[b]) << 16,
  //  hi(c[c]) | hi(c[d]) << 16, lo(c[c]) | lo(c[d]) << 16}: one 16-byte read
  //  gives the decode key operand of four coordinates
  uint32_t* quad_tab = nullptr;
  // exact top-k refinement (float64): rotT64 [d][d] = Pi^T, qjlT64 [d][m]
  // = S^T (or null), cent64 [L] centroids
  double* rotT64 = nullptr;
  double* qjlT64 = nullptr;
  double* cent64 = nullptr;
  // top-k fp16 operand table: the layout of pair_tab with fp16 hi/lo parts
  // of 2^6 c (lo parts below the fp16 normal range are 0)
  uint32_t* pair_tab16 = nullptr;
  // d = 128 quantize (see quantize128.hip), absent for other d:
  //  rop: Pi as bf16 operands of v_mfma_f32_32x32x16_bf16 in three parts
  //  (hi, lo, lo2), uint4 [wave 4][k-step 8][part 3][lane 64]; lane l of wave
  //  w, step s holds Pi[32w + l%32][16s + 8(l/32) + 0..7]
  //  qtab: index cells of y in [-1, 1]: cell c = floor((y + 1) * qG) covers
  //  [c/qG - 1, (c+1)/qG - 1) and holds {#boundaries below it, (t + 1) qG for
  //  the boundary t inside it (fp32 bits) or FLT_MAX}; cells are narrower than
  //  the closest pair of boundaries, so at most one lies inside
  uint32_t* rop = nullptr;
  uint32_t* qtab = nullptr;
  //  sop: S (rows past m zero) as hi / lo / lo2 operands in the layout of rop
  //  (d = 128, 0 < m <= 128); keys with a sketch use hi and lo
  uint32_t* sop = nullptr;
  int qcells = 0;
  float qG = 0.f;
  // PolarQuant codebooks: ptrig [2 * centroids] (cos, sin) of every angle
  // centroid, pbnd [boundaries] fp32, both level-major as cent_off / bnd_off
  float* ptrig = nullptr;
  float* pbnd = nullptr;
};

// PolarQuant layout of a codebook (polar == false for scalar codebooks)
constexpr int kPolarMaxLevels = 8;
struct PolarInfo {
  bool polar = false;
  int b1 = 0, br = 0, levels = 0;
  int cent_off[kPolarMaxLevels + 2] = {};
  int bnd_off[kPolarMaxLevels + 2] = {};
  int field_bits = 0;        // (d/2) b1 + (d/2 - 1) br
};

constexpr int kQ128Cells = 2048;   // largest index-cell table the d = 128 kernel stages

// padded sizes used by the kernels
inline int pad32(int x) { return (x + 31) / 32 * 32; }

}  // namespace tq

struct tq_codebook {
  tq_params p;
  int L = 0, dp = 0, mp = 0;
  double emax_c16 = 0.0;   // max_l |c_l - 2^-6 (hi + lo)_l| of pair_tab16
  int device = 0;
  tq::HostCodebook host;
  tq::DeviceCodebook dev;
  tq::PolarInfo pq;
};

namespace tq {

void set_error(const std::string& msg);

// Instrumentation: hipEvent pairs around main-kernel launches (per thread).
struct ProfileScope {
  ProfileScope(int kernel, hipStream_t stream);
  ~ProfileScope();
  int kernel;
  hipStream_t stream;
  void* stop = nullptr;
};

// ---- kernels (launchers return hipSuccess or the launch error)

// Paged code pools.  Sequence s = b * hkv + h of a job lives in pool plane h:
// its 32-position block blk is block page * ppb + blk % ppb of that plane,
// page = table[b * max_pages + blk / ppb] clamped to [0, n_pages), with
// ppb = 2^ppb_shift blocks per page.  table == nullptr: no paging (sequence
// s is plane s and block blk is block blk).
struct PageMap {
  const int32_t* table = nullptr;
  int64_t max_pages = 0;
  int64_t n_pages = 0;
  int64_t hkv = 1;
  int ppb_shift = 0;
};

__device__ inline void page_block(const PageMap& pm, int64_t seq, int64_t blk, int64_t& oseq, int64_t& oblk) {
  if (pm.table == nullptr) {
    oseq = seq;
    oblk = blk;
    return;
  }
  const int64_t b = seq / pm.hkv;
  oseq = seq - b * pm.hkv;
  int64_t lp = blk >> pm.ppb_shift;
  lp = lp < pm.max_pages ? lp : pm.max_pages - 1;
  // the block's page is the same for the whole workgroup: read it through
  // the scalar cache (constant address space), so that it takes no part in
  // the vector-memory waits of the tile loads in flight
  typedef const __attribute__((address_space(4))) int32_t* ctab_t;
  int64_t pg = ((ctab_t)(uintptr_t)pm.table)[b * pm.max_pages + lp];
  pg = pg < 0 ? 0 : (pg >= pm.n_pages ? pm.n_pages - 1 : pg);
  oblk = (pg << pm.ppb_shift) + (blk & ((1LL << pm.ppb_shift) - 1));
}

struct QuantJob {
  const void* x;          // [n_seq][n_tok][d]
  tq_dtype dt;
  int64_t n_seq, n_tok, tok_offset;
  tq_codes out;
  PageMap pm{};
};

hipError_t launch_quantize(const tq_codebook* cb, const QuantJob& job, hipStream_t stream);

// d = 128 bulk quantize (split-bf16 MFMA rotation, table index; sketches of
// up to 128 rows in the row layout); used by launch_quantize when
// quantize128_supported
bool quantize128_supported(const tq_codebook* cb, const QuantJob& job);
hipError_t launch_quantize128(const tq_codebook* cb, const QuantJob& job, hipStream_t stream);

// Few vectors per sequence (appends): one workgroup per vector; K and V jobs in
// one launch.  njobs in 1..2, jobs share n_seq, n_tok and dtype.
// Query prologue of the d = 128 decode kernels (decode_prologue.hpp): one
// workgroup per (part, row) of a plan, part 0..3 covering 32 coordinates.
struct PArgs {
  const void* q;
  int qdt;
  int Hq, Hkv, g, qgroups;
  int m, mp;
  float qscale;           // sm_scale * log2(e)
  const float* rotKT;     // [128][128], rotKT[k][i] = Pi_K[i][k]
  const float* sprotKT;   // [128][mp], sprotKT[k][j] = sqrt(pi/2)/m (S_K Pi_K)[j][k] (or null)
  uint32_t* qop;          // [rows][query-operand dwords]
};

// pro != nullptr: the launch also runs the decode query prologue of pro_rows
// rows (4 workgroups per row) beside the appends, saving its own launch.
hipError_t launch_quantize_small(const tq_codebook* const* cbs, const QuantJob* jobs, int njobs,
                                 hipStream_t stream, const PArgs* pro = nullptr, int64_t pro_rows = 0);
constexpr int64_t kSmallMaxTok = 8;   // appends of up to this many tokens per sequence

// Dequantize positions [tok_offset, tok_offset + n_tok) of n_seq sequences
// into out [n_seq][n_tok][d] of dtype dt.
struct DequantJob {
  tq_codes codes;
  int64_t n_seq, n_tok, tok_offset;
  void* out;
  tq_dtype dt;
};
bool dequantize128_supported(const tq_codebook* cb);
hipError_t launch_dequantize(const tq_codebook* cb, const DequantJob& job, hipStream_t stream);

struct DecodePlan {
  int64_t B, Hq, Hkv, n_ctx;
  int d;
  int page_tokens;  // 0, or the page size of a paged pool (chunks are whole pages, <= 64 per wave)
  int g;            // Hq / Hkv
  int qgroups;      // ceil(g / 8)
  int64_t rows;     // B * Hkv * qgroups (one row = one KV head and <= 8 query heads)
  int chunk;        // tokens per wave (multiple of 32)
  int n_parts;      // waves per row = ceil(n_ctx / chunk)
  int n_wg;         // workgroups per row = ceil(n_parts / waves per workgroup)
  size_t off_qop, off_part_o, off_part_ml, bytes;
};

DecodePlan plan_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_ctx, int d, int page_tokens = 0);

// pm.table != nullptr: k and v are page pools (plane h = KV head h), read
// through pm (plan.page_tokens = 32 << pm.ppb_shift)
hipError_t launch_decode(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                         tq_dtype qdt, const DecodePlan& plan, const tq_codes& k,
                         const tq_codes& v, const int32_t* seq_lens, float sm_scale,
                         float* out, float* logits, void* ws, hipStream_t stream,
                         const PageMap& pm = PageMap{}, bool prologue_done = false);
// The query-prologue arguments of a d = 128 plan (false when the any-shape
// kernels serve the codebooks, whose prologue is their own).
bool make_decode_prologue(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, tq_dtype qdt,
                          const DecodePlan& plan, float sm_scale, void* ws, PArgs* out);

// d = 128 MFMA kernels (decode.hip)
bool decode_supported(const tq_codebook* kcb, const tq_codebook* vcb);
// fp32 kernels for every other scalar shape (decode_gen.hip): d <= 256, bits
// 1..8, sketches <= 256 rows; launch_decode hands them such codebooks
bool decode_generic_supported(const tq_codebook* kcb, const tq_codebook* vcb);
int64_t decode_generic_row_bytes(int d);   // prologue output per row
hipError_t launch_decode_generic(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, tq_dtype qdt,
                                 const DecodePlan& plan, const tq_codes& k, const tq_codes& v,
                                 const int32_t* seq_lens, float sm_scale, float* out, float* logits, void* ws,
                                 hipStream_t stream, const PageMap& pm);

// Inner-product top-k (limits of the LDS-resident per-lane lists and operands)
constexpr int kIpTopkMax = 32;   // k
constexpr int kIpCandMax = 64;   // candidates of the approximate pass (k > 10: 2k)
constexpr int kIpNuMax = 16;     // MSE MFMAs per query block: dp / 16 (d <= 256)
constexpr int kIpNsMax = 8;      // sign MFMAs: ceil(m / 32) (m <= 256)
constexpr int64_t kIpMaxRowBytes = 256, kIpMaxSignRowBytes = 32;

constexpr int kIpFbChunks = 64;   // workgroups per query of the exact fallback scan

struct TopkPlan {
  int64_t nq, n_db, nqb, n_tiles, tiles_per_chunk;
  int k, nu, ns, n_chunks;
  int kc;               // candidates per query of the approximate pass (>= k)
  bool shared;          // k <= 16: workgroups of 128 queries share unpacked tiles
  int64_t sample_stride, sample_tiles;   // sample pass over every sample_stride-th tile (0: none)
  int sample_chunks;
  int64_t sample_ld;                     // floats per query of the sample scores
  size_t off_sample, off_floor;          // [nqp][sample_ld] sample scores, [nq] floors
  size_t off_qop, off_cinit, off_cand_s, off_cand_i;
  // exact refinement: float64 rotated query and sketch [nqp][d], [nqp][m],
  // per-query norms, database bounds, the approximate top-kc, flags and the
  // fallback lists [nq][kIpFbChunks][k]
  size_t off_qt64, off_tt64, off_qinfo, off_bounds, off_acand_s, off_acand_i, off_flags, off_fb_s, off_fb_i;
  size_t off_fblist;    // [nq] the queries the exact scan answers (count in bounds[3])
  size_t off_bpart;     // per-workgroup database maxima of the bounds kernel
  size_t bytes;
};

TopkPlan plan_topk(int64_t nq, int64_t n_db, int k, int d, int m);

// force_scan: every query takes the exact scan
hipError_t launch_topk(const tq_codebook* cb, const float* queries, const TopkPlan& plan,
                       const tq_codes& db, int64_t* out_idx, float* out_score, void* ws,
                       hipStream_t stream, bool force_scan);

// Allocation-free decode: the fixed per-device scratch array (bytes) and its
// device address on the current device (looked up on the first call there).
constexpr size_t kNoallocScratchBytes = 8u << 20;
hipError_t noalloc_scratch(void** out);

// PolarQuant kernels (polar.hip): bulk and append quantize into the row
// layout (d a power of two <= 128, qjl_m <= 128) and dequantize.
bool polar_quantize_supported(const tq_codebook* cb);
hipError_t launch_polar_quantize(const tq_codebook* cb, const QuantJob& job, hipStream_t stream);
hipError_t launch_polar_dequantize(const tq_codebook* cb, const DequantJob& job, hipStream_t stream);

// Streaming read of bytes (a multiple of 16) of buf; writes sink[0] only
// in the rare case that the XOR of the data equals a fixed value.
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_stream_write(void* buf, int64_t bytes, uint32_t value, hipStream_t stream);

}  // namespace tq
