// Inner-product top-k over coded database vectors (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog): the inner-product estimate of
// the two-stage scheme ("第二阶段：QJL 残差校正": the 1-bit sketch of the
// residual corrects the bias of the MSE stage) and its use for nearest
// neighbour search ("基准测试与实际性能表现": top-k recall of vector search at
// d = 200).  The score of database vector
// j for query q is
//     s_j = scale_j <Pi q, c[idx_j]> + sqrt(pi/2)/m * rnorm_j <S Pi q, 2 sigma_j - 1>
// (no softmax scale), and the result is the k largest s_j per query, ties to
// the lower index.
//
// k_ip_prologue  one workgroup per query: q~ = Pi q, t = sqrt(pi/2)/m S q~,
//                written as bf16 hi/lo MFMA B operands for blocks of 8 queries.
// k_ip_score2    (k <= 16) grid (database chunk, group of 128 queries); eight
//                waves (two per SIMD) hold two 8-query blocks each as MFMA B
//                operands in registers.  Each 16-row database tile is unpacked once per
//                workgroup into A operands in LDS (centroid operand from the
//                pair table, sign operand from sign bytes) and feeds all 16
//                blocks through v_mfma_f32_16x16x32_bf16 (hi/lo query
//                columns).  Tiles go in pairs between barriers: while the
//                MFMAs of a tile run, the tile two ahead is unpacked, and
//                raw code rows are fetched four to five tiles ahead.
//                Each query keeps one unsorted top-k list in LDS with its
//                worst entry (score, slot): the four lanes that hold the
//                query's rows insert in row order, a better candidate
//                overwrites the worst slot and one 128-bit read pass finds
//                the new worst; every lane filters against a cached copy of
//                the worst score.  The workgroup then sorts each list into k
//                candidates per (query, chunk).  For large databases a first
//                pass over every 64th tile gives each query the k-th best
//                score of that sample, a lower bound of its final k-th score
//                that the full pass starts from, so few candidates reach the
//                lists.
// k_ip_score     (k > 16) the same product with one 8-query block per
//                workgroup and each wave unpacking its own tiles.
// k_ip_merge     one wave per query selects the final k from the candidates.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIpWaves = 4;
constexpr int kSignShiftIp = 64;    // the sketch-query operand carries 2^-64
constexpr int32_t kNoIndex = 0x7FFFFFFF;

__device__ inline uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  u32x4v v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

// lane j gets x[j] + x[j + 8] within each row of 16 lanes (hi + lo columns)
__device__ inline float dpp_ror8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// (score, index) order: larger score first, then lower index
__device__ inline bool better(float s, int32_t i, float ps, int32_t pi) {
  return s > ps || (s == ps && i < pi);
}

// ------------------------------------------------------------ prologue

struct IPArgs {
  const float* q;       // [nq][d]
  int64_t nq;
  int d, m, dp, mp, nu, ns;
  const double* rotT64; // [d][d], rotT64[k][i] = Pi[i][k]
  const double* qjlT64; // [d][m], qjlT64[i][j] = S[j][i]
  uint32_t* qop;        // [nqb][nu + ns][64 lanes][4 dwords]
  float* cinit;         // [nqb * 8]
  double* qt64;         // [nq][256] q~ = Pi q (float64)
  double* tt64;         // [nq][256] t = sqrt(pi/2)/m S q~ (float64)
  double* qinfo;        // [nq][2] |q~|_2, |t|_1
  uint32_t* bounds;     // [2] database max |scale|, max |rnorm| (zeroed here)
};

// Operand layouts (lane = column j + 16 g4 of the B operand; columns 0-7 are
// the hi parts of the block's 8 queries, 8-15 their lo parts):
//  MSE MFMA u: element el of lane group g4 is coordinate
//    16 u + 4 g4 + 2 (el / 4) + el % 2, matching the key operand dwords
//    {hi pair, lo pair} of coordinate pairs (a, b) and (c, d);
//  sign MFMA v: element el is sketch row 32 v + 8 g4 + el, scaled by
//    2^(128 - 2^el - 64): the sign operand leaves bit el of the lane's sign
//    byte at bf16 bit 7 + el, the normal value 2^(2^el - 127).
// q~ and t are formed in float64 (kept for the exact refinement) and rounded
// to float before the bf16 hi/lo split.
__global__ void __launch_bounds__(256) k_ip_prologue(IPArgs a) {
  __shared__ double qs[256], qt[256], tt[256];
  __shared__ double red[2][4];
  const int64_t qi = blockIdx.x;        // over the padded query count
  const int tid = threadIdx.x;
  const bool valid = qi < a.nq;
  if (qi == 0 && tid < 2) a.bounds[tid] = 0u;
  qs[tid] = (valid && tid < a.d) ? (double)a.q[qi * a.d + tid] : 0.0;
  __syncthreads();
  double z = 0.0;
  if (tid < a.d) {
    for (int k = 0; k < a.d; ++k) z = fma(a.rotT64[(int64_t)k * a.d + tid], qs[k], z);
  }
  qt[tid] = z;
  __syncthreads();
  double t = 0.0;
  if (tid < a.m) {
    for (int i = 0; i < a.d; ++i) t = fma(a.qjlT64[(int64_t)i * a.m + tid], qt[i], t);
    t *= 1.2533141373155002512 / (double)a.m;      // sqrt(pi/2) / m
  }
  tt[tid] = t;
  if (valid) {
    a.qt64[qi * 256 + tid] = z;
    a.tt64[qi * 256 + tid] = t;
  }
  {
    double n2 = z * z, n1 = fabs(t);
    for (int o = 32; o >= 1; o >>= 1) {
      n2 += __shfl_xor(n2, o);
      n1 += __shfl_xor(n1, o);
    }
    if ((tid & 63) == 0) { red[0][tid >> 6] = n2; red[1][tid >> 6] = n1; }
  }
  __syncthreads();
  if (valid && tid == 0) {
    a.qinfo[qi * 2 + 0] = sqrt(red[0][0] + red[0][1] + red[0][2] + red[0][3]);
    a.qinfo[qi * 2 + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
  const int64_t qb = qi >> 3;
  const int c = (int)(qi & 7);
  uint32_t* rec = a.qop + qb * (int64_t)(a.nu + a.ns) * 256;
  for (int e = tid; e < a.nu * 32; e += 256) {
    const int dw = e & 3, g4 = (e >> 2) & 3, hl = (e >> 4) & 1, u = e >> 5;
    uint32_t hv[2];
    for (int h2 = 0; h2 < 2; ++h2) {
      const int el = 2 * dw + h2;
      const float v = (float)qt[16 * u + 4 * g4 + 2 * (el >> 2) + (el & 1)];
      const uint32_t hi = bf16_rne_bits(v);
      hv[h2] = hl ? bf16_rne_bits(v - __uint_as_float(hi << 16)) : hi;
    }
    rec[(u * 64 + hl * 8 + c + 16 * g4) * 4 + dw] = hv[0] | (hv[1] << 16);
  }
  for (int e = tid; e < a.ns * 32; e += 256) {
    const int dw = e & 3, g4 = (e >> 2) & 3, hl = (e >> 4) & 1, v = e >> 5;
    uint32_t hv[2];
    for (int h2 = 0; h2 < 2; ++h2) {
      const int el = 2 * dw + h2;
      const float x = ldexpf((float)tt[32 * v + 8 * g4 + el], 128 - (1 << el) - kSignShiftIp);
      const uint32_t hi = bf16_rne_bits(x);
      hv[h2] = hl ? bf16_rne_bits(x - __uint_as_float(hi << 16)) : hi;
    }
    rec[((a.nu + v) * 64 + hl * 8 + c + 16 * g4) * 4 + dw] = hv[0] | (hv[1] << 16);
  }
  // QJL accumulator offset: -sum_j (hi + lo)(t_j), in the scale of the products
  if (tid < 64) {
    float s = 0.f;
    for (int j = tid; j < 256; j += 64) {
      const float v = (float)tt[j];
      const float fh = __uint_as_float(bf16_rne_bits(v) << 16);
      s += fh + __uint_as_float(bf16_rne_bits(v - fh) << 16);
    }
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (tid == 0) a.cinit[qi] = -ldexpf(s, -kSignShiftIp);
  }
}

// Database bounds of the refinement's error bound: max |scale| and max
// |rnorm| (as float bits; non-negative floats order as their bits).
__global__ void __launch_bounds__(256) k_ip_bounds(const float* scale, const float* rnorm, int64_t n,
                                                   uint32_t* bounds) {
  float ms = 0.f, mr = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    ms = fmaxf(ms, fabsf(scale[i]));
    if (rnorm) mr = fmaxf(mr, fabsf(rnorm[i]));
  }
  for (int o = 32; o >= 1; o >>= 1) {
    ms = fmaxf(ms, __shfl_xor(ms, o));
    mr = fmaxf(mr, __shfl_xor(mr, o));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(bounds, __float_as_uint(ms));
    atomicMax(bounds + 1, __float_as_uint(mr));
  }
}

// ------------------------------------------------------------ scores + lists

struct ISArgs {
  const uint32_t* qop;
  const float* cinit;
  const uint32_t* idx;     // row layout, idx_pitch bytes per vector
  const uint32_t* sign;    // sign_pitch bytes per vector (or null)
  const float* scale;
  const float* rnorm;
  const uint32_t* tab;     // decode operand table of the codebook
  int64_t n_db, n_tiles, tiles_per_chunk;
  int rw, sw;              // 32-bit words per idx / sign row
  int nu, ns, k, n_chunks;
  float* cand_s;           // [nq_pad][n_chunks][k]
  int32_t* cand_i;
};

// LM: capacity of the per-lane lists (>= k)
template <int B, bool QJL, int LM>
__global__ void __launch_bounds__(64 * kIpWaves) k_ip_score(ISArgs a) {
  constexpr int TABW = (B <= 4) ? (2 << (2 * B)) : (1 << B);
  __shared__ __align__(16) uint4 s_q[(kIpNuMax + kIpNsMax) * 64];
  __shared__ __align__(16) uint32_t s_tab[TABW];
  __shared__ uint32_t s_st[kIpWaves][16 * 64];      // the wave's 16 idx rows
  __shared__ uint32_t s_ss[kIpWaves][16 * 8];       // and their sign rows
  __shared__ float s_ls[LM][kIpWaves * 32];  // per-lane lists, slot-major
  __shared__ int32_t s_li[LM][kIpWaves * 32];
  __shared__ float s_cinit[8];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int64_t qb = blockIdx.y;
  const int chunk = blockIdx.x;
  const int nus = a.nu + a.ns;
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.qop) + qb * (int64_t)nus * 64;
    for (int i = tid; i < nus * 64; i += 64 * kIpWaves) s_q[i] = src[i];
    for (int i = tid; i < TABW; i += 64 * kIpWaves) s_tab[i] = a.tab[i];
    if (tid < 8) s_cinit[tid] = a.cinit[qb * 8 + tid];
    for (int i = tid; i < a.k * kIpWaves * 32; i += 64 * kIpWaves) {
      s_ls[i / (kIpWaves * 32)][i % (kIpWaves * 32)] = -INFINITY;
      s_li[i / (kIpWaves * 32)][i % (kIpWaves * 32)] = kNoIndex;
    }
  }
  __syncthreads();

  const int ln = wave * 32 + g4 * 8 + (c16 & 7);   // list column (lanes c16 < 8)
  const float cin = (QJL && c16 < 8) ? s_cinit[c16] : 0.f;
  float thr = -INFINITY;
  const int64_t t_begin = (int64_t)chunk * a.tiles_per_chunk;
  int64_t t_end = t_begin + a.tiles_per_chunk;
  if (t_end > a.n_tiles) t_end = a.n_tiles;
  uint32_t* st = s_st[wave];
  uint32_t* ss = s_ss[wave];
  const char* tab = reinterpret_cast<const char*>(s_tab);

  for (int64_t tile = t_begin + wave; tile < t_end; tile += kIpWaves) {
    const int64_t row0 = tile * 16;
    // stage the 16 rows (rows past the end repeat the last one; masked below)
    for (int e = lane; e < 16 * a.rw; e += 64) {
      const int r = e / a.rw, w = e - r * a.rw;
      int64_t rr = row0 + r;
      if (rr > a.n_db - 1) rr = a.n_db - 1;
      st[e] = a.idx[rr * a.rw + w];
    }
    if constexpr (QJL) {
      for (int e = lane; e < 16 * a.sw; e += 64) {
        const int r = e / a.sw, w = e - r * a.sw;
        int64_t rr = row0 + r;
        if (rr > a.n_db - 1) rr = a.n_db - 1;
        ss[e] = a.sign[rr * a.sw + w];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // <q~, c[idx]> over MFMAs of 16 coordinates (hi/lo)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int u = 0; u < a.nu; ++u) {
      const int o = (16 * u + 4 * g4) * B;
      const int i0 = o >> 5, sh = o & 31;
      const int i1 = (i0 + 1 < a.rw) ? i0 + 1 : i0;
      const uint32_t f = __builtin_amdgcn_alignbit(st[c16 * a.rw + i1], st[c16 * a.rw + i0], sh);
      uint32_t d0, d1, d2, d3;
      if constexpr (B <= 4) {
        constexpr uint32_t PM = (1u << (2 * B)) - 1u;
        const uint2 e0 = *reinterpret_cast<const uint2*>(tab + ((f & PM) << 3));
        const uint2 e1 = *reinterpret_cast<const uint2*>(tab + (((f >> (2 * B)) & PM) << 3));
        d0 = e0.x; d1 = e0.y; d2 = e1.x; d3 = e1.y;
      } else {
        constexpr uint32_t CM = (1u << B) - 1u;
        const uint32_t* t32 = reinterpret_cast<const uint32_t*>(tab);
        const uint32_t ca = t32[f & CM], cb = t32[(f >> B) & CM];
        const uint32_t cc = t32[(f >> (2 * B)) & CM], cd = t32[(f >> (3 * B)) & CM];
        d0 = __builtin_amdgcn_perm(cb, ca, 0x05040100u);
        d1 = __builtin_amdgcn_perm(cb, ca, 0x07060302u);
        d2 = __builtin_amdgcn_perm(cd, cc, 0x05040100u);
        d3 = __builtin_amdgcn_perm(cd, cc, 0x07060302u);
      }
      acc = mfma(as_bf16x8(d0, d1, d2, d3), __builtin_bit_cast(bf16x8, s_q[u * 64 + lane]), acc);
    }
    // <t, sigma> over MFMAs of 32 sketch rows
    f32x4 accq = {cin, cin, cin, cin};
    if constexpr (QJL) {
      for (int v = 0; v < a.ns; ++v) {
        const uint32_t sb = (ss[c16 * a.sw + v] >> (8 * g4)) & 0xFFu;
        const uint32_t x7 = (sb | (sb << 16)) << 7;
        accq = mfma(as_bf16x8(x7 & 0x01000080u, x7 & 0x04000200u, x7 & 0x10000800u, x7 & 0x40002000u),
                    __builtin_bit_cast(bf16x8, s_q[(a.nu + v) * 64 + lane]), accq);
      }
    }
    // scores of rows row0 + 4 g4 + r for query c16 (lanes c16 < 8)
    float sc[4], rn[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int64_t rr = row0 + 4 * g4 + r;
      if (rr > a.n_db - 1) rr = a.n_db - 1;
      sc[r] = a.scale[rr];
      rn[r] = QJL ? a.rnorm[rr] : 0.f;
    }
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = sc[r] * (acc[r] + dpp_ror8(acc[r]));
      if constexpr (QJL) v = fmaf(rn[r] * 0x1p64f, accq[r] + dpp_ror8(accq[r]), v);
      s[r] = (row0 + 4 * g4 + r < a.n_db) ? v : -INFINITY;
    }
    if (c16 < 8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (s[r] > thr) {
          const int32_t id = (int32_t)(row0 + 4 * g4 + r);
          int j = a.k - 1;
          while (j > 0) {
            const float p = s_ls[j - 1][ln];
            if (!(s[r] > p)) break;
            s_ls[j][ln] = p;
            s_li[j][ln] = s_li[j - 1][ln];
            --j;
          }
          s_ls[j][ln] = s[r];
          s_li[j][ln] = id;
          thr = s_ls[a.k - 1][ln];
        }
      }
    }
  }
  __syncthreads();

  // merge the 16 lists of each query (4 waves x 4 lane groups) into k candidates
  if (tid < 8) {
    const int c = tid;
    int head[kIpWaves * 4];
#pragma unroll
    for (int h = 0; h < kIpWaves * 4; ++h) head[h] = 0;
    const int64_t base = ((qb * 8 + c) * a.n_chunks + chunk) * (int64_t)a.k;
    for (int o = 0; o < a.k; ++o) {
      int best = -1;
      float bs = -INFINITY;
      int32_t bi = kNoIndex;
#pragma unroll
      for (int h = 0; h < kIpWaves * 4; ++h) {
        if (head[h] >= a.k) continue;
        const int col = (h >> 2) * 32 + (h & 3) * 8 + c;
        const float hs = s_ls[head[h]][col];
        const int32_t hi = s_li[head[h]][col];
        if (best < 0 || better(hs, hi, bs, bi)) { best = h; bs = hs; bi = hi; }
      }
      head[best]++;
      a.cand_s[base + o] = bs;
      a.cand_i[base + o] = bi;
    }
  }
}

// ------------------------------------------------------------ scores, shared tiles

constexpr int kIp2Waves = 8;        // waves per workgroup, two per SIMD
constexpr int kIp2Blocks = 2;       // 8-query blocks per wave (their operands fit in VGPRs)
constexpr int kIp2Queries = 8 * kIp2Waves * kIp2Blocks;   // 128 queries per workgroup
constexpr int kIp2TopK = 16;        // largest k of this kernel
constexpr int kIp2Lists = kIp2Queries;                        // one list per query
constexpr int kIp2Raw = 16 * (kIpMaxRowBytes / 4) + 16 * (kIpMaxSignRowBytes / 4) + 32;  // words of a raw tile
constexpr int kIp2IdxPer = 16 * (kIpMaxRowBytes / 4) / (64 * kIp2Waves);                   // idx words per thread
static_assert(16 * (kIpMaxSignRowBytes / 4) + 32 <= 64 * kIp2Waves, "one sign / scalar word per thread");
static_assert(kIp2IdxPer >= 1, "at least one idx word per thread");

struct IS2Args {
  const uint32_t* qop;
  const float* cinit;
  const uint32_t* idx;     // row layout, rw words per vector
  const uint32_t* sign;    // sw words per vector (or null)
  const float* scale;
  const float* rnorm;
  const uint32_t* tab;     // decode operand table of the codebook
  int64_t n_db, n_tiles, tiles_per_chunk;
  int64_t tstride;         // tile i of a chunk is database tile (t_begin + i) * tstride
  int64_t nq;
  const float* floor_s;    // [nq][k] sample top-k scores (entry k-1 is the floor), or null
  int rw, sw, bits, nu, ns, k, n_chunks;
  float* cand_s;           // [nq_pad][n_chunks][k]
  int32_t* cand_i;
};

template <int NU, int NS>
__global__ void __launch_bounds__(64 * kIp2Waves) k_ip_score2(IS2Args a) {
  constexpr int NUS = NU + NS;
  // tiles go in pairs between barriers: slots 2c, 2c + 1 of buffer c
  __shared__ __align__(16) uint4 s_a[4][NUS][64];          // A operands of a tile
  __shared__ float s_sr[4][2][16];                         // its scale and 2^64 rnorm
  __shared__ __align__(16) uint32_t s_raw[4][kIp2Raw];     // raw code rows of a tile
  __shared__ __align__(16) uint32_t s_tab[512];
  __shared__ __align__(16) float s_ls[kIp2Lists][kIp2TopK];    // per-query lists (unsorted)
  __shared__ __align__(16) int32_t s_li[kIp2Lists][kIp2TopK];
  __shared__ float s_ws[kIp2Lists];                           // worst score of each list
  __shared__ int s_wj[kIp2Lists];                             // and its slot
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int chunk = blockIdx.x;
  const int64_t qb0 = (int64_t)blockIdx.y * (kIp2Waves * kIp2Blocks) + wave * kIp2Blocks;
  const int B = a.bits, nu = NU, nus = NUS;
  const int tabw = B <= 4 ? (2 << (2 * B)) : (1 << B);
  for (int i = tid; i < tabw; i += 64 * kIp2Waves) s_tab[i] = a.tab[i];
  // slots below k start empty (-inf, no index); slots from k on hold +inf so
  // that they are never the worst entry
  for (int i = tid; i < kIp2Lists * kIp2TopK; i += 64 * kIp2Waves) {
    const bool live = (i % kIp2TopK) < a.k;
    s_ls[i / kIp2TopK][i % kIp2TopK] = live ? -INFINITY : INFINITY;
    s_li[i / kIp2TopK][i % kIp2TopK] = live ? kNoIndex : -1;
  }
  for (int i = tid; i < kIp2Lists; i += 64 * kIp2Waves) {
    s_ws[i] = -INFINITY;
    s_wj[i] = 0;
  }
  // this wave's query operands (registers) and QJL accumulator offsets
  bf16x8 bq[kIp2Blocks][NUS];
  float cin[kIp2Blocks];
#pragma unroll
  for (int qb = 0; qb < kIp2Blocks; ++qb) {
    const uint4* src = reinterpret_cast<const uint4*>(a.qop) + (qb0 + qb) * (int64_t)nus * 64;
#pragma unroll
    for (int u = 0; u < NUS; ++u) bq[qb][u] = __builtin_bit_cast(bf16x8, src[u * 64 + lane]);
    cin[qb] = (NS > 0 && c16 < 8) ? a.cinit[(qb0 + qb) * 8 + c16] : 0.f;
  }

  // fixed share of the raw tile words of this thread: up to kIp2IdxPer words
  // of the 16 idx rows, and one word that is a sign word, a scale or an rnorm
  const int n_idx = 16 * a.rw, n_sgn = 16 * a.sw;
  int ioff[kIp2IdxPer], irow[kIp2IdxPer];
#pragma unroll
  for (int j = 0; j < kIp2IdxPer; ++j) {
    const int e = tid + 64 * kIp2Waves * j;
    irow[j] = e < n_idx ? e / a.rw : -1;
    ioff[j] = e < n_idx ? e - irow[j] * a.rw : 0;
  }
  const uint32_t* mbase;
  int mrow, mstr, mw;
  if (tid < n_sgn) { mbase = a.sign; mrow = tid / a.sw; mw = tid - mrow * a.sw; mstr = a.sw; }
  else if (tid < n_sgn + 16) { mbase = reinterpret_cast<const uint32_t*>(a.scale); mrow = tid - n_sgn; mw = 0; mstr = 1; }
  else if (tid < n_sgn + 32) { mbase = reinterpret_cast<const uint32_t*>(a.rnorm); mrow = tid - n_sgn - 16; mw = 0; mstr = 1; }
  else { mbase = nullptr; mrow = 0; mw = 0; mstr = 0; }
  const int last = (int)(a.n_db - 1);
  struct Pre {
    uint32_t i[kIp2IdxPer];
    uint32_t m;
  };
  Pre ra, rb;
  auto raw_load = [&](Pre& P, int64_t tile) {
    uint32_t (&pre_i)[kIp2IdxPer] = P.i;
    uint32_t& pre_m = P.m;
    pre_m = 0u;
    // the tile's base is formed in 64 bits (a database may exceed 2^31
    // words); a lane's offset from it spans at most 16 rows
    const int64_t r0 = tile * 16;
    const uint32_t* tbase = a.idx + r0 * a.rw;
#pragma unroll
    for (int j = 0; j < kIp2IdxPer; ++j) {
      pre_i[j] = 0u;
      if (irow[j] >= 0) {
        const int rr = (int)(min(r0 + irow[j], (int64_t)last) - r0);   // rows past the end repeat the last one
        pre_i[j] = tbase[rr * a.rw + ioff[j]];
      }
    }
    if (mbase) pre_m = (mbase + r0 * mstr)[(int)(min(r0 + mrow, (int64_t)last) - r0) * mstr + mw];
  };
  // raw tile layout: idx rows [0, n_idx), sign rows [n_idx, n_idx + n_sgn),
  // scale [.., +16), rnorm [.., +16)
  auto raw_store = [&](const Pre& P, int buf) {
#pragma unroll
    for (int j = 0; j < kIp2IdxPer; ++j)
      if (irow[j] >= 0) s_raw[buf][tid + 64 * kIp2Waves * j] = P.i[j];
    if (mbase) s_raw[buf][n_idx + tid] = P.m;
  };
  // unpack raw buffer rb into operand buffer ob: task (u, lane) = tid + 512 j
  auto build = [&](int rb, int ob) {
    const uint32_t* raw = s_raw[rb];
    const char* tab = reinterpret_cast<const char*>(s_tab);
#pragma unroll
    for (int jj = 0; jj < (NUS * 64 + 64 * kIp2Waves - 1) / (64 * kIp2Waves); ++jj) {
      const int t = tid + 64 * kIp2Waves * jj;
      if (t >= NUS * 64) break;
      const int u = t >> 6, l = t & 63, r = l & 15, g = l >> 4;
      uint32_t d0, d1, d2, d3;
      if (u < nu) {
        const int o = (16 * u + 4 * g) * B;
        const int i0 = o >> 5, sh = o & 31;
        const int i1 = (i0 + 1 < a.rw) ? i0 + 1 : i0;
        const uint32_t f = __builtin_amdgcn_alignbit(raw[r * a.rw + i1], raw[r * a.rw + i0], sh);
        if (B <= 4) {
          const uint32_t pm = (1u << (2 * B)) - 1u;
          const uint2 e0 = *reinterpret_cast<const uint2*>(tab + ((f & pm) << 3));
          const uint2 e1 = *reinterpret_cast<const uint2*>(tab + (((f >> (2 * B)) & pm) << 3));
          d0 = e0.x; d1 = e0.y; d2 = e1.x; d3 = e1.y;
        } else {
          const uint32_t cm = (1u << B) - 1u;
          const uint32_t* t32 = reinterpret_cast<const uint32_t*>(tab);
          const uint32_t ca = t32[f & cm], cb = t32[(f >> B) & cm];
          const uint32_t cc = t32[(f >> (2 * B)) & cm], cd = t32[(f >> (3 * B)) & cm];
          d0 = __builtin_amdgcn_perm(cb, ca, 0x05040100u);
          d1 = __builtin_amdgcn_perm(cb, ca, 0x07060302u);
          d2 = __builtin_amdgcn_perm(cd, cc, 0x05040100u);
          d3 = __builtin_amdgcn_perm(cd, cc, 0x07060302u);
        }
      } else {
        const uint32_t sb = (raw[n_idx + r * a.sw + (u - nu)] >> (8 * g)) & 0xFFu;
        const uint32_t x7 = (sb | (sb << 16)) << 7;
        d0 = x7 & 0x01000080u; d1 = x7 & 0x04000200u; d2 = x7 & 0x10000800u; d3 = x7 & 0x40002000u;
      }
      s_a[ob][u][l] = make_uint4(d0, d1, d2, d3);
    }
    if (tid < 32) {
      const float v = __uint_as_float(raw[n_idx + n_sgn + tid]);
      s_sr[ob][tid >> 4][tid & 15] = (tid < 16) ? v : v * 0x1p64f;
    }
  };

  // thq: cached worst score of the list of this lane's query in a block.  A
  // query's candidates are inserted in increasing row order (tile by tile,
  // lane group g4 = 0..3 within a tile, then its 4 rows), so a candidate that
  // only ties the worst entry loses to it and the strict tests are exact.
  // tqf: the sample floor of the query (candidates below it cannot be in the
  // final top k; equal ones may, so that test is not strict)
  float thq[kIp2Blocks], tqf[kIp2Blocks];
#pragma unroll
  for (int qb = 0; qb < kIp2Blocks; ++qb) {
    thq[qb] = -INFINITY;
    const int64_t q = (qb0 + qb) * 8 + c16;
    tqf[qb] = (a.floor_s && c16 < 8 && q < a.nq) ? a.floor_s[q * a.k + a.k - 1] : -INFINITY;
  }
  const int64_t t_begin = (int64_t)chunk * a.tiles_per_chunk;
  int64_t t_end = t_begin + a.tiles_per_chunk;
  if (t_end > a.n_tiles) t_end = a.n_tiles;
  const int64_t nt = t_end > t_begin ? t_end - t_begin : 0;

  auto dbt = [&](int64_t i) { return (t_begin + i) * a.tstride; };   // database tile of step i
  // prologue: raw tiles 0, 1 -> slots 0, 1 -> operands; raw tiles 2, 3 ->
  // slots 2, 3; raw tiles 4, 5 in registers
  raw_load(ra, dbt(0));
  raw_load(rb, dbt(1));
  raw_store(ra, 0);
  raw_store(rb, 1);
  raw_load(ra, dbt(2));
  raw_load(rb, dbt(3));
  raw_store(ra, 2);
  raw_store(rb, 3);
  raw_load(ra, dbt(4));
  raw_load(rb, dbt(5));
  __syncthreads();
  build(0, 0);
  build(1, 1);
  __syncthreads();

  // one tile: its MFMAs from operand slot ab, then the unpack of raw slot
  // ub into operand slot ub (a tile two ahead), then its scores and lists
  auto tile_step = [&](const int ab, const int ub, const int64_t row0, const bool live)
                       __attribute__((always_inline)) {
    f32x4 acc[kIp2Blocks], accq[kIp2Blocks];
#pragma unroll
    for (int qb = 0; qb < kIp2Blocks; ++qb) {
      acc[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      accq[qb] = (f32x4){cin[qb], cin[qb], cin[qb], cin[qb]};
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, s_a[ab][u][lane]);
#pragma unroll
      for (int qb = 0; qb < kIp2Blocks; ++qb) acc[qb] = mfma(av, bq[qb][u], acc[qb]);
    }
#pragma unroll
    for (int v = 0; v < NS; ++v) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, s_a[ab][NU + v][lane]);
#pragma unroll
      for (int qb = 0; qb < kIp2Blocks; ++qb) accq[qb] = mfma(av, bq[qb][NU + v], accq[qb]);
    }
    // unpack a tile two ahead while the MFMAs run (past the last tile it
    // rebuilds a slot nobody reads)
    build(ub, ub);
    if (!live) return;
    float sc[4], rn[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = s_sr[ab][0][4 * g4 + r];
      rn[r] = s_sr[ab][1][4 * g4 + r];
    }
#pragma unroll
    for (int qb = 0; qb < kIp2Blocks; ++qb) {
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[r] * (acc[qb][r] + dpp_ror8(acc[qb][r]));
        if constexpr (NS > 0) v = fmaf(rn[r], accq[qb][r] + dpp_ror8(accq[qb][r]), v);
        sv[r] = (row0 + 4 * g4 + r < a.n_db) ? v : -INFINITY;
      }
      uint32_t pm = 0u;                 // rows of this lane that beat the cached worst
#pragma unroll
      for (int r = 0; r < 4; ++r) pm |= (c16 < 8 && sv[r] > thq[qb] && sv[r] >= tqf[qb]) ? (1u << r) : 0u;
      if (__ballot(pm != 0u) != 0ull) {
        const int li = (wave * kIp2Blocks + qb) * 8 + c16;     // list of this lane's query
        for (int g = 0; g < 4; ++g) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool me = g4 == g && ((pm >> r) & 1u);
            if (__ballot(me) != 0ull && me) {
              if (sv[r] > s_ws[li]) {
                const int wj = s_wj[li];
                s_ls[li][wj] = sv[r];
                s_li[li][wj] = (int32_t)(row0 + 4 * g4 + r);
                // new worst: lowest score, then highest index
                float ws = INFINITY;
                int32_t wi = -1;
                int nj = 0;
#pragma unroll
                for (int c4 = 0; c4 < kIp2TopK / 4; ++c4) {
                  const float4 sc4 = reinterpret_cast<const float4*>(s_ls[li])[c4];
                  const int4 id4 = reinterpret_cast<const int4*>(s_li[li])[c4];
                  const float sa[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
                  const int32_t ia[4] = {id4.x, id4.y, id4.z, id4.w};
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const bool worse = sa[e] < ws || (sa[e] == ws && ia[e] > wi);
                    ws = worse ? sa[e] : ws;
                    wi = worse ? ia[e] : wi;
                    nj = worse ? 4 * c4 + e : nj;
                  }
                }
                s_ws[li] = ws;
                s_wj[li] = nj;
              }
            }
          }
        }
        if (c16 < 8) thq[qb] = s_ws[li];
      }
    }
  };

  const int64_t np = (nt + 1) / 2;
  for (int64_t p = 0; p < np; ++p) {
    const int c = (int)(p & 1), n = c ^ 1;
    // tiles 2p, 2p + 1 sit in operand slots 2c, 2c + 1; raw tiles 2p + 2,
    // 2p + 3 in raw slots 2n, 2n + 1; raw tiles 2p + 4, 2p + 5 in ra, rb
    tile_step(2 * c, 2 * n, dbt(2 * p) * 16, true);
    tile_step(2 * c + 1, 2 * n + 1, dbt(2 * p + 1) * 16, 2 * p + 1 < nt);
    // raw slots 2c, 2c + 1 were unpacked before the last barrier
    raw_store(ra, 2 * c);
    raw_store(rb, 2 * c + 1);
    raw_load(ra, dbt(2 * p + 6));
    raw_load(rb, dbt(2 * p + 7));
    __syncthreads();
  }

  // sort each query's list into its k candidates, (score desc, index asc)
  if (tid < kIp2Queries) {
    const int li = tid;      // list of query tid of the workgroup
    const int64_t q = (int64_t)blockIdx.y * kIp2Queries + tid;
    const int64_t base = (q * a.n_chunks + chunk) * (int64_t)a.k;
    float ps = INFINITY;
    int32_t pi = -1;
    for (int o = 0; o < a.k; ++o) {
      float bs = -INFINITY;
      int32_t bi = kNoIndex;
      for (int j = 0; j < a.k; ++j) {
        const float hs = s_ls[li][j];
        const int32_t hi = s_li[li][j];
        if (better(ps, pi, hs, hi) && better(hs, hi, bs, bi)) { bs = hs; bi = hi; }
      }
      a.cand_s[base + o] = bs;
      a.cand_i[base + o] = bi;
      ps = bs;
      pi = bi;
    }
  }
}

template <int NU, int NS>
void launch_score2_ns(const IS2Args& a, int ns, dim3 grid, hipStream_t st) {
  if constexpr (NS > kIpNsMax) {
    (void)a; (void)ns; (void)grid; (void)st;
  } else {
    if (ns == NS) hipLaunchKernelGGL((k_ip_score2<NU, NS>), grid, dim3(64 * kIp2Waves), 0, st, a);
    else launch_score2_ns<NU, NS + 1>(a, ns, grid, st);
  }
}

// NU = dp / 16 is even (dp is a multiple of 32)
template <int NU>
void launch_score2(const IS2Args& a, dim3 grid, hipStream_t st) {
  if constexpr (NU > kIpNuMax) {
    (void)a; (void)grid; (void)st;
  } else {
    if (a.nu == NU) launch_score2_ns<NU, 0>(a, a.ns, grid, st);
    else launch_score2<NU + 2>(a, grid, st);
  }
}

// ------------------------------------------------------------ final merge

struct IMArgs {
  const float* cand_s;
  const int32_t* cand_i;
  int64_t nq;
  int n_chunks, k;
  int64_t* out_idx;     // final indices (-1: none), or null
  float* out_score;
  int32_t* out_i32;     // candidate indices (kNoIndex: none), when out_idx is null
};

// One wave per query: k rounds, each picking the best candidate that comes
// after the previous pick in (score desc, index asc) order; indices are
// distinct, so the order is strict.
__global__ void __launch_bounds__(64) k_ip_merge(IMArgs a) {
  const int64_t q = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = a.n_chunks * a.k;
  const float* cs = a.cand_s + q * n;
  const int32_t* ci = a.cand_i + q * n;
  float ps = INFINITY;
  int32_t pi = -1;
  for (int o = 0; o < a.k; ++o) {
    float bs = -INFINITY;
    int32_t bi = kNoIndex;
    bool have = false;
    for (int e = lane; e < n; e += 64) {
      const float s = cs[e];
      const int32_t i = ci[e];
      if (!better(ps, pi, s, i)) continue;          // not after the previous pick
      if (!have || better(s, i, bs, bi)) { bs = s; bi = i; have = true; }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const float os = __shfl_xor(bs, off);
      const int32_t oi = __shfl_xor(bi, off);
      if (better(os, oi, bs, bi)) { bs = os; bi = oi; }
    }
    if (lane == 0) {
      a.out_score[q * a.k + o] = bs;
      if (a.out_idx) a.out_idx[q * a.k + o] = (bi == kNoIndex) ? -1 : (int64_t)bi;
      else a.out_i32[q * a.k + o] = bi;
    }
    ps = bs;
    pi = bi;
  }
}

template <int B>
void launch_score_b(const ISArgs& a, bool qjl, dim3 grid, hipStream_t st) {
  if (a.k <= 32) {
    if (qjl) hipLaunchKernelGGL((k_ip_score<B, true, 32>), grid, dim3(64 * kIpWaves), 0, st, a);
    else hipLaunchKernelGGL((k_ip_score<B, false, 32>), grid, dim3(64 * kIpWaves), 0, st, a);
  } else {
    if (qjl) hipLaunchKernelGGL((k_ip_score<B, true, kIpCandMax>), grid, dim3(64 * kIpWaves), 0, st, a);
    else hipLaunchKernelGGL((k_ip_score<B, false, kIpCandMax>), grid, dim3(64 * kIpWaves), 0, st, a);
  }
}

// ------------------------------------------------------------ exact refinement
//
// The approximate pass keeps the kc best rows by the bf16 hi/lo MFMA score
// A_j.  Each candidate is rescored in float64 from its codes (E_j, the
// score's definition evaluated with q~ and t in float64), and the k best by
// E are the answer when no other row can beat the k-th of them: a row left
// out has A_j <= A_kc (the kc-th approximate score) and E_j <= A_j + delta,
// so A_kc + delta < E_k settles it.  delta bounds |A_j - E_j| for every row
// of the database from the operand rounding (q~, t and the centroids go
// through float and a bf16 hi + lo pair, relative error <= 2^-16 + 2^-24
// each), the float accumulation of n products (gamma_n = n u / (1 - n u),
// u = 2^-24) and the final combination, over the bounds
//     |scale_j <q~, c[idx_j]>| <= max|scale| sqrt(d) max|c| |q~|_2
//     |rnorm_j <t, 2 sigma_j - 1>| <= max|rnorm| |t|_1,
// and is doubled to cover an MFMA that rounds toward zero.  A query that
// fails the test (near-ties at the k-th score, or a database of repeated
// rows) is answered by an exact float64 scan of the whole database.

struct IRArgs {
  const float* acand_s;     // [nq][kc] approximate top-kc (sorted)
  const int32_t* acand_i;
  const double* qt64;       // [nq][256]
  const double* tt64;
  const double* qinfo;      // [nq][2]
  const uint32_t* bounds;   // max |scale|, max |rnorm| (float bits)
  const double* cent64;     // [2^bits]
  const uint32_t* idx;      // row layout, rw words per vector
  const uint32_t* sign;     // sw words per vector (or null)
  const float* scale;
  const float* rnorm;
  int64_t nq, n_db;
  int d, m, bits, rw, sw, nu, ns, k, kc;
  int force_scan;           // 1: no query is settled by the candidates
  int64_t* out_idx;
  float* out_score;
  int32_t* flags;           // [nq]: 1 settled by the candidates, 0 needs the scan
  double* fb_s;             // [nq][kIpFbChunks][k] scan lists
  int32_t* fb_i;
};

// float64 score of database row `row` from its codes; sq = q~, st = t
// (sqrt(pi/2)/m folded in), cent = centroids, all in LDS
__device__ double exact_score(const IRArgs& a, int64_t row, const double* sq, const double* st,
                              const double* cent) {
  const uint32_t* ir = a.idx + row * (int64_t)a.rw;
  const uint32_t mask = (1u << a.bits) - 1u;
  double mse = 0.0;
  for (int i = 0; i < a.d; ++i) {
    const int bit = i * a.bits, w = bit >> 5, sh = bit & 31;
    uint32_t v = ir[w] >> sh;
    if (sh + a.bits > 32) v |= ir[w + 1] << (32 - sh);
    mse = fma(sq[i], cent[v & mask], mse);
  }
  double qj = 0.0;
  if (a.m > 0) {
    const uint32_t* sr = a.sign + row * (int64_t)a.sw;
    for (int j = 0; j < a.m; ++j) qj += ((sr[j >> 5] >> (j & 31)) & 1u) ? st[j] : -st[j];
  }
  double s = (double)a.scale[row] * mse;
  if (a.m > 0) s = fma((double)a.rnorm[row], qj, s);
  return s;
}

__device__ inline bool better64(double s, int32_t i, double ps, int32_t pi) {
  return s > ps || (s == ps && i < pi);
}

__device__ void load_exact_operands(const IRArgs& a, int64_t q, double* sq, double* st, double* cent) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    sq[i] = a.qt64[q * 256 + i];
    st[i] = a.tt64[q * 256 + i];
    if (i < (1 << a.bits)) cent[i] = a.cent64[i];
  }
}

// One wave per query: float64 scores of the kc candidates, their top k, and
// the test that settles the query.
__global__ void __launch_bounds__(64) k_ip_refine(IRArgs a) {
  __shared__ double sq[256], st[256], cent[256];
  __shared__ double es[64];
  __shared__ int32_t ei[64];
  __shared__ double ek;
  const int64_t q = blockIdx.x;
  const int lane = threadIdx.x;
  load_exact_operands(a, q, sq, st, cent);
  __syncthreads();
  double e = -INFINITY;
  int32_t id = kNoIndex;
  if (lane < a.kc) {
    id = a.acand_i[q * a.kc + lane];
    if (id != kNoIndex) e = exact_score(a, id, sq, st, cent);
  }
  es[lane] = e;
  ei[lane] = id;
  if (lane == 0) ek = -INFINITY;
  __syncthreads();
  if (lane < a.kc) {
    // rank by (score desc, index asc); empty slots last, in slot order
    int rank = 0;
    for (int j = 0; j < a.kc; ++j)
      rank += (better64(es[j], ei[j], e, id) || (es[j] == e && ei[j] == id && j < lane)) ? 1 : 0;
    if (rank < a.k) {
      a.out_idx[q * a.k + rank] = (id == kNoIndex) ? -1 : (int64_t)id;
      a.out_score[q * a.k + rank] = (id == kNoIndex) ? -INFINITY : (float)e;
    }
    if (rank == a.k - 1) ek = e;
  }
  double cm = 0.0;
  for (int i = lane; i < (1 << a.bits); i += 64) cm = fmax(cm, fabs(cent[i]));
  for (int o = 32; o >= 1; o >>= 1) cm = fmax(cm, __shfl_xor(cm, o));
  __syncthreads();
  if (lane == 0) {
    bool ok = (int64_t)a.kc >= a.n_db;                    // every row was rescored
    if (!ok && !a.force_scan) {
      const double u = 0x1p-24;
      auto gam = [u](double n) { return n * u / (1.0 - n * u); };
      const double rel = 0x1p-16 + 0x1p-24;
      const double bm = (double)__uint_as_float(a.bounds[0]) * sqrt((double)a.d) * cm * a.qinfo[q * 2];
      const double bq = (double)__uint_as_float(a.bounds[1]) * a.qinfo[q * 2 + 1];
      const double nm = 32.0 * a.nu + 16.0, nsk = 32.0 * a.ns + 16.0;
      const double delta = 2.0 * ((2.0 * rel + rel * rel + gam(nm)) * (1.0 + 2.0 * rel) * bm +
                                  (rel + gam(320.0) + 3.0 * gam(nsk)) * bq + 4.0 * u * (bm + bq));
      const float akc = a.acand_s[q * a.kc + a.kc - 1];
      ok = (double)akc + delta < ek;
    }
    a.flags[q] = ok ? 1 : 0;
  }
}

// Exact scan for the queries the candidates did not settle: grid
// (query slots, kIpFbChunks); each workgroup keeps the k best rows of its
// share of the database by float64 score, for queries blockIdx.x,
// blockIdx.x + gridDim.x, ...
__global__ void __launch_bounds__(256) k_ip_fallback(IRArgs a) {
  __shared__ double sq[256], st[256], cent[256];
  __shared__ double ls[kIpTopkMax];
  __shared__ int32_t li[kIpTopkMax];
  __shared__ double bs[256];
  __shared__ int32_t bi[256];
  __shared__ uint64_t bal[4];
  const int tid = threadIdx.x;
  const int64_t per = (a.n_db + kIpFbChunks - 1) / kIpFbChunks;
  const int64_t r0 = (int64_t)blockIdx.y * per;
  const int64_t r1 = (r0 + per < a.n_db) ? r0 + per : a.n_db;
  for (int64_t q = blockIdx.x; q < a.nq; q += gridDim.x) {
    if (a.flags[q] != 0) continue;                      // uniform over the workgroup
    __syncthreads();                                    // LDS of the previous query is free
    load_exact_operands(a, q, sq, st, cent);
    if (tid < kIpTopkMax) { ls[tid] = -INFINITY; li[tid] = kNoIndex; }
    __syncthreads();
    for (int64_t base = r0; base < r1; base += 256) {
      const int64_t row = base + tid;
      double s = -INFINITY;
      int32_t id = kNoIndex;
      if (row < r1) { s = exact_score(a, row, sq, st, cent); id = (int32_t)row; }
      bs[tid] = s;
      bi[tid] = id;
      const bool pass = id != kNoIndex && better64(s, id, ls[a.k - 1], li[a.k - 1]);
      const uint64_t b = __ballot(pass);
      if ((tid & 63) == 0) bal[tid >> 6] = b;
      __syncthreads();
      if (tid == 0) {
        // insert the rows that beat the k-th entry, in row order
        for (int w = 0; w < 4; ++w) {
          uint64_t msk = bal[w];
          while (msk) {
            const int t = w * 64 + __builtin_ctzll(msk);
            msk &= msk - 1;
            const double v = bs[t];
            const int32_t vi = bi[t];
            if (!better64(v, vi, ls[a.k - 1], li[a.k - 1])) continue;
            int j = a.k - 1;
            while (j > 0 && better64(v, vi, ls[j - 1], li[j - 1])) {
              ls[j] = ls[j - 1];
              li[j] = li[j - 1];
              --j;
            }
            ls[j] = v;
            li[j] = vi;
          }
        }
      }
      __syncthreads();
    }
    if (tid < a.k) {
      const int64_t o = (q * kIpFbChunks + blockIdx.y) * (int64_t)a.k + tid;
      a.fb_s[o] = ls[tid];
      a.fb_i[o] = li[tid];
    }
  }
}

// One wave per unsettled query: the k best of its kIpFbChunks scan lists.
__global__ void __launch_bounds__(64) k_ip_fbmerge(IRArgs a) {
  const int64_t q = blockIdx.x;
  if (a.flags[q] != 0) return;
  const int lane = threadIdx.x;
  const int n = kIpFbChunks * a.k;
  const double* cs = a.fb_s + q * n;
  const int32_t* ci = a.fb_i + q * n;
  double ps = INFINITY;
  int32_t pi = -1;
  for (int o = 0; o < a.k; ++o) {
    double bsv = -INFINITY;
    int32_t biv = kNoIndex;
    bool have = false;
    for (int e = lane; e < n; e += 64) {
      const double s = cs[e];
      const int32_t i = ci[e];
      if (i == kNoIndex || !better64(ps, pi, s, i)) continue;
      if (!have || better64(s, i, bsv, biv)) { bsv = s; biv = i; have = true; }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const double os = __shfl_xor(bsv, off);
      const int32_t oi = __shfl_xor(biv, off);
      if (better64(os, oi, bsv, biv)) { bsv = os; biv = oi; }
    }
    if (lane == 0) {
      a.out_score[q * a.k + o] = (biv == kNoIndex) ? -INFINITY : (float)bsv;
      a.out_idx[q * a.k + o] = (biv == kNoIndex) ? -1 : (int64_t)biv;
    }
    ps = bsv;
    pi = biv;
  }
}

}  // namespace

// candidates of the approximate pass: k <= 10 keeps the shared-tile kernel
// (16 candidates); larger k take twice k, at most kIpCandMax
static int topk_candidates(int k) { return k <= 10 ? 16 : (2 * k < kIpCandMax ? 2 * k : kIpCandMax); }

TopkPlan plan_topk(int64_t nq, int64_t n_db, int k, int d, int m) {
  TopkPlan p{};
  p.nq = nq; p.n_db = n_db; p.k = k;
  p.kc = topk_candidates(k);
  p.nu = (pad32(d) + 15) / 16;
  p.ns = m > 0 ? (m + 31) / 32 : 0;
  p.shared = p.kc <= kIp2TopK;
  // query blocks of 8, padded to whole workgroups of 128 queries for the shared-tile kernel
  p.nqb = p.shared ? (nq + kIp2Queries - 1) / kIp2Queries * (kIp2Queries / 8) : (nq + 7) / 8;
  p.n_tiles = (n_db + 15) / 16;
  const int64_t groups = p.shared ? p.nqb / (kIp2Queries / 8) : p.nqb;
  // workgroups: shared tiles take 122 KB of LDS, one workgroup per CU, so
  // 256 is one round over the CUs (3% faster than two rounds at 10^6 rows)
  const int64_t target = p.shared ? 256 : 2048;
  int64_t chunks = groups > 0 ? (target + groups - 1) / groups : 1;
  int64_t cap = p.n_tiles / 8;                                   // >= 8 tiles per chunk
  if (chunks > cap) chunks = cap;
  if (chunks > 4096) chunks = 4096;
  if (chunks < 1) chunks = 1;
  p.tiles_per_chunk = p.n_tiles > 0 ? (p.n_tiles + chunks - 1) / chunks : 1;
  p.n_chunks = p.n_tiles > 0 ? (int)((p.n_tiles + p.tiles_per_chunk - 1) / p.tiles_per_chunk) : 1;
  size_t off = 0;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t kc = (size_t)p.kc, nqp = (size_t)p.nqb * 8;
  p.off_qop = off; off = al(off + (size_t)p.nqb * (p.nu + p.ns) * 64 * 16);
  p.off_cinit = off; off = al(off + nqp * 4);
  const size_t nc = nqp * p.n_chunks * kc;
  p.off_cand_s = off; off = al(off + nc * 4);
  p.off_cand_i = off; off = al(off + nc * 4);
  // sample pass (shared-tile kernel, large databases): every 64th tile,
  // 32 chunks, merged into the top kc of the sample per query
  p.sample_stride = (p.shared && p.n_tiles >= 64 * 256) ? 64 : 0;
  if (p.sample_stride) {
    p.sample_tiles = p.n_tiles / p.sample_stride;
    p.sample_chunks = 32;
    const size_t ns2 = nqp * p.sample_chunks * kc;
    p.off_s_cand_s = off; off = al(off + ns2 * 4);
    p.off_s_cand_i = off; off = al(off + ns2 * 4);
    p.off_s_idx = off; off = al(off + (size_t)nq * kc * 8);
    p.off_s_score = off; off = al(off + (size_t)nq * kc * 4);
  }
  p.off_qt64 = off; off = al(off + nqp * 256 * 8);
  p.off_tt64 = off; off = al(off + nqp * 256 * 8);
  p.off_qinfo = off; off = al(off + nqp * 2 * 8);
  p.off_bounds = off; off = al(off + 2 * 4);
  p.off_acand_s = off; off = al(off + (size_t)nq * kc * 4);
  p.off_acand_i = off; off = al(off + (size_t)nq * kc * 4);
  p.off_flags = off; off = al(off + (size_t)nq * 4);
  p.off_fb_s = off; off = al(off + (size_t)nq * kIpFbChunks * k * 8);
  p.off_fb_i = off; off = al(off + (size_t)nq * kIpFbChunks * k * 4);
  p.bytes = off;
  return p;
}

hipError_t launch_topk(const tq_codebook* cb, const float* queries, const TopkPlan& plan,
                       const tq_codes& db, int64_t* out_idx, float* out_score, void* ws,
                       hipStream_t stream, bool force_scan) {
  if (plan.nq == 0 || plan.k == 0) return hipSuccess;
  char* w = static_cast<char*>(ws);
  uint32_t* qop = reinterpret_cast<uint32_t*>(w + plan.off_qop);
  float* cinit = reinterpret_cast<float*>(w + plan.off_cinit);
  float* cand_s = reinterpret_cast<float*>(w + plan.off_cand_s);
  int32_t* cand_i = reinterpret_cast<int32_t*>(w + plan.off_cand_i);
  uint32_t* bounds = reinterpret_cast<uint32_t*>(w + plan.off_bounds);
  const bool qjl = cb->p.qjl_m > 0;

  IPArgs pa{};
  pa.q = queries; pa.nq = plan.nq;
  pa.d = cb->p.d; pa.m = cb->p.qjl_m; pa.dp = cb->dp; pa.mp = cb->mp;
  pa.nu = plan.nu; pa.ns = plan.ns;
  pa.rotT64 = cb->dev.rotT64; pa.qjlT64 = cb->dev.qjlT64;
  pa.qop = qop; pa.cinit = cinit;
  pa.qt64 = reinterpret_cast<double*>(w + plan.off_qt64);
  pa.tt64 = reinterpret_cast<double*>(w + plan.off_tt64);
  pa.qinfo = reinterpret_cast<double*>(w + plan.off_qinfo);
  pa.bounds = bounds;
  hipLaunchKernelGGL(k_ip_prologue, dim3((unsigned)(plan.nqb * 8)), dim3(256), 0, stream, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (plan.n_db > 0) {
    int64_t nb = (plan.n_db + 255) / 256;
    if (nb > 1024) nb = 1024;
    hipLaunchKernelGGL(k_ip_bounds, dim3((unsigned)nb), dim3(256), 0, stream, db.scale, qjl ? db.rnorm : nullptr,
                       plan.n_db, bounds);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  float* acand_s = reinterpret_cast<float*>(w + plan.off_acand_s);
  int32_t* acand_i = reinterpret_cast<int32_t*>(w + plan.off_acand_i);
  ISArgs sa{};
  sa.qop = qop; sa.cinit = cinit;
  sa.idx = static_cast<const uint32_t*>(db.idx);
  sa.sign = static_cast<const uint32_t*>(db.sign);
  sa.scale = db.scale; sa.rnorm = db.rnorm;
  sa.tab = cb->dev.pair_tab;
  sa.n_db = plan.n_db; sa.n_tiles = plan.n_tiles; sa.tiles_per_chunk = plan.tiles_per_chunk;
  sa.rw = (int)(db.idx_row_bytes / 4);
  sa.sw = qjl ? (int)(db.sign_row_bytes / 4) : 0;
  sa.nu = plan.nu; sa.ns = plan.ns; sa.k = plan.kc; sa.n_chunks = plan.n_chunks;
  sa.cand_s = cand_s; sa.cand_i = cand_i;
  {
    ProfileScope prof(TQ_KERNEL_TOPK, stream);
    if (plan.shared) {
      IS2Args s2{};
      s2.qop = qop; s2.cinit = cinit;
      s2.idx = sa.idx; s2.sign = sa.sign; s2.scale = sa.scale; s2.rnorm = qjl ? sa.rnorm : sa.scale;
      s2.tab = sa.tab;
      s2.n_db = plan.n_db; s2.n_tiles = plan.n_tiles; s2.tiles_per_chunk = plan.tiles_per_chunk;
      s2.rw = sa.rw; s2.sw = sa.sw; s2.bits = cb->p.bits; s2.nu = plan.nu; s2.ns = plan.ns;
      s2.k = plan.kc; s2.n_chunks = plan.n_chunks;
      s2.cand_s = cand_s; s2.cand_i = cand_i;
      s2.tstride = 1;
      s2.nq = plan.nq;
      s2.floor_s = nullptr;
      const unsigned groups = (unsigned)(plan.nqb / (kIp2Queries / 8));
      if (plan.sample_stride) {
        IS2Args sp = s2;
        sp.tstride = plan.sample_stride;
        sp.n_tiles = plan.sample_tiles;
        sp.n_chunks = plan.sample_chunks;
        sp.tiles_per_chunk = (plan.sample_tiles + plan.sample_chunks - 1) / plan.sample_chunks;
        sp.cand_s = reinterpret_cast<float*>(w + plan.off_s_cand_s);
        sp.cand_i = reinterpret_cast<int32_t*>(w + plan.off_s_cand_i);
        launch_score2<2>(sp, dim3((unsigned)plan.sample_chunks, groups), stream);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        IMArgs sm{};
        sm.cand_s = sp.cand_s; sm.cand_i = sp.cand_i;
        sm.nq = plan.nq; sm.n_chunks = plan.sample_chunks; sm.k = plan.kc;
        sm.out_idx = reinterpret_cast<int64_t*>(w + plan.off_s_idx);
        sm.out_score = reinterpret_cast<float*>(w + plan.off_s_score);
        hipLaunchKernelGGL(k_ip_merge, dim3((unsigned)plan.nq), dim3(64), 0, stream, sm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        s2.floor_s = sm.out_score;
      }
      launch_score2<2>(s2, dim3((unsigned)plan.n_chunks, groups), stream);
    } else {
      const dim3 grid((unsigned)plan.n_chunks, (unsigned)plan.nqb);
      switch (cb->p.bits) {
        case 1: launch_score_b<1>(sa, qjl, grid, stream); break;
        case 2: launch_score_b<2>(sa, qjl, grid, stream); break;
        case 3: launch_score_b<3>(sa, qjl, grid, stream); break;
        case 4: launch_score_b<4>(sa, qjl, grid, stream); break;
        case 5: launch_score_b<5>(sa, qjl, grid, stream); break;
        case 6: launch_score_b<6>(sa, qjl, grid, stream); break;
        case 7: launch_score_b<7>(sa, qjl, grid, stream); break;
        default: launch_score_b<8>(sa, qjl, grid, stream); break;
      }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  IMArgs ma{};
  ma.cand_s = cand_s; ma.cand_i = cand_i;
  ma.nq = plan.nq; ma.n_chunks = plan.n_chunks; ma.k = plan.kc;
  ma.out_idx = nullptr; ma.out_score = acand_s; ma.out_i32 = acand_i;
  hipLaunchKernelGGL(k_ip_merge, dim3((unsigned)plan.nq), dim3(64), 0, stream, ma);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  IRArgs ra{};
  ra.acand_s = acand_s; ra.acand_i = acand_i;
  ra.qt64 = pa.qt64; ra.tt64 = pa.tt64; ra.qinfo = pa.qinfo; ra.bounds = bounds;
  ra.cent64 = cb->dev.cent64;
  ra.idx = sa.idx; ra.sign = sa.sign; ra.scale = db.scale; ra.rnorm = db.rnorm;
  ra.nq = plan.nq; ra.n_db = plan.n_db;
  ra.d = cb->p.d; ra.m = cb->p.qjl_m; ra.bits = cb->p.bits; ra.rw = sa.rw; ra.sw = sa.sw;
  ra.nu = plan.nu; ra.ns = plan.ns; ra.k = plan.k; ra.kc = plan.kc;
  ra.force_scan = force_scan ? 1 : 0;
  ra.out_idx = out_idx; ra.out_score = out_score;
  ra.flags = reinterpret_cast<int32_t*>(w + plan.off_flags);
  ra.fb_s = reinterpret_cast<double*>(w + plan.off_fb_s);
  ra.fb_i = reinterpret_cast<int32_t*>(w + plan.off_fb_i);
  hipLaunchKernelGGL(k_ip_refine, dim3((unsigned)plan.nq), dim3(64), 0, stream, ra);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((int64_t)plan.kc < plan.n_db) {
    const unsigned slots = (unsigned)(plan.nq < 4096 ? plan.nq : 4096);
    hipLaunchKernelGGL(k_ip_fallback, dim3(slots, (unsigned)kIpFbChunks), dim3(256), 0, stream, ra);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_ip_fbmerge, dim3((unsigned)plan.nq), dim3(64), 0, stream, ra);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
