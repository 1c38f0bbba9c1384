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
// The result is the exact top-k of s_j evaluated in float64 from the codes.
// One call launches, in order:
// k_ip_prologue  four queries per workgroup: q~ = Pi q and t = sqrt(pi/2)/m
//                S q~ in float64, the norms the error bound needs, and the
//                MFMA B operands: fp16, each query scaled by a power of two
//                (k <= 16), or bf16 hi/lo (k > 16).
// k_ip_bounds    one pass over the codes: per-workgroup maxima of |scale|,
//                |rnorm| and |c[idx]|_2, reduced by k_ip_refine.
// k_ip_score16   (topk_common.hpp; k <= 16) 256 (or 128) queries per
//                workgroup, 8 waves x 2 (or 1) blocks of 16 queries as fp16
//                B operands in registers; each 16-row database tile is
//                unpacked once into LDS A operands (fp16 hi/lo centroids from
//                a pair table, +-1 signs from a byte table) and feeds every
//                block through v_mfma_f32_16x16x32_f16.  Candidates above
//                the query's floor are appended to LDS buffers with an LDS
//                atomic; a refresh keeps the best kc when a buffer fills.
//                For large databases a sample pass over every 64th tile
//                first writes the score of every sampled row, and
//                k_ip_floor takes each query's kc-th best of them by a radix
//                select: the full pass starts from that floor.
// k_ip_score     (16 < k <= 32) the bf16 hi/lo product, one 8-query block
//                per workgroup, each wave unpacking its own tiles.
// k_ip_merge     the kc best candidates of each query over the chunks.
// k_ip_refine    rescores the candidates in float64 from the codes, ranks
//                them (ties to the lower index) and keeps the top k when the
//                kc-th approximate score plus the bound on the approximate
//                score's error is below the k-th exact score; other queries
//                go to a list.
// k_ip_fallback, k_ip_fbmerge  the exact float64 scan of the listed queries
//                over 64 database chunks, and the merge of its lists.
#include "topk_common.hpp"

namespace tq {
namespace {

// ------------------------------------------------------------ prologue

struct IPArgs {
  const float* q;       // [nq][d]
  int64_t nq;
  int d, m, dp, mp, nu, ns;
  int half;             // 1: fp16 operands of k_ip_score16; 0: bf16 hi/lo operands of k_ip_score
  const double* rotT64; // [d][d], rotT64[k][i] = Pi[i][k]
  const double* qjlT64; // [d][m], qjlT64[i][j] = S[j][i]
  uint32_t* qop;        // operand records (layout of the mode)
  float* cinit;         // bf16 mode: [nqp] QJL accumulator offsets; fp16 mode: [nqp][2] 2^-(6+sq), 2^-st
  double* qt64;         // [nq][256] q~ = Pi q (float64)
  double* tt64;         // [nq][256] t = sqrt(pi/2)/m S q~ (float64)
  double* qinfo;        // [nq][kQInfo] norms for the error bound
  uint32_t* bounds;     // [4] bounds[3]: count of queries for the exact scan (zeroed here)
};

// qinfo fields: |q~|_2, |t|_1, and in fp16 mode |q~ - q^|_2, |q^|_2,
// |t - t^|_1, |t^|_1 where q^, t^ are the operand values (unscaled)
constexpr int kQInfo = 6;

__device__ inline uint16_t f16_bits(float x) {
  const _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ inline float f16_value(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
// x rounded to fp16, with results below the fp16 normal range taken as 0
// (so the operand is the same whether or not the matrix unit flushes them)
__device__ inline uint16_t f16_operand(double x) {
  const uint16_t b = f16_bits((float)x);
  return ((b & 0x7C00u) == 0u) ? (uint16_t)0u : b;
}

// Operand layouts.  bf16 mode (blocks of 8 queries; lane = column j + 16 g4
// of the B operand, columns 0-7 the hi parts of the block's queries, 8-15
// their lo parts):
//  MSE MFMA u: element el of lane group g4 is coordinate
//    16 u + 4 g4 + 2 (el / 4) + el % 2, matching the key operand dwords
//    {hi pair, lo pair} of coordinate pairs (a, b) and (c, d);
//  sign MFMA v: element el is sketch row 32 v + 8 g4 + el, scaled by
//    2^(128 - 2^el - 64): the sign operand leaves bit el of the lane's sign
//    byte at bf16 bit 7 + el, the normal value 2^(2^el - 127).
// fp16 mode (blocks of 16 queries, column j = query j of the block): record
// u < nu / 2 holds coordinates 32 u + 8 g4 + el (one operand that meets the
// hi and then the lo parts of the centroids in two MFMAs), record nu / 2 + v
// sketch rows 32 v + 8 g4 + el; q~ is scaled by 2^sq and t by 2^st, powers
// of two that bring the largest component to [2^14, 2^15).
// q~ and t are formed in float64 (kept for the exact refinement).
constexpr int kProQ = 4;              // queries per prologue workgroup

__global__ void __launch_bounds__(256) k_ip_prologue(IPArgs a) {
  __shared__ double qs[kProQ][256], qtq[kProQ][256], ttq[kProQ][256];
  __shared__ double red[6][4];
  __shared__ int sexp[2];
  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * kProQ;   // over the padded query count
  if (blockIdx.x == 0 && tid < 4) a.bounds[tid] = 0u;
#pragma unroll
  for (int j = 0; j < kProQ; ++j)
    qs[j][tid] = (q0 + j < a.nq && tid < a.d) ? (double)a.q[(q0 + j) * a.d + tid] : 0.0;
  __syncthreads();
  // q~ = Pi q and t = sqrt(pi/2)/m S q~ of the workgroup's queries, one pass
  // over each table
  double zz[kProQ], tv[kProQ];
#pragma unroll
  for (int j = 0; j < kProQ; ++j) { zz[j] = 0.0; tv[j] = 0.0; }
  if (tid < a.d) {
    for (int k = 0; k < a.d; ++k) {
      const double r = a.rotT64[(int64_t)k * a.d + tid];
#pragma unroll
      for (int j = 0; j < kProQ; ++j) zz[j] = fma(r, qs[j][k], zz[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < kProQ; ++j) qtq[j][tid] = zz[j];
  __syncthreads();
  if (tid < a.m) {
    for (int i = 0; i < a.d; ++i) {
      const double sv = a.qjlT64[(int64_t)i * a.m + tid];
#pragma unroll
      for (int j = 0; j < kProQ; ++j) tv[j] = fma(sv, qtq[j][i], tv[j]);
    }
#pragma unroll
    for (int j = 0; j < kProQ; ++j) tv[j] *= 1.2533141373155002512 / (double)a.m;   // sqrt(pi/2) / m
  }
#pragma unroll
  for (int j = 0; j < kProQ; ++j) ttq[j][tid] = tv[j];
  __syncthreads();
  for (int j = 0; j < kProQ; ++j) {
  const int64_t qi = q0 + j;
  const bool valid = qi < a.nq;
  const double z = zz[j], t = tv[j];
  const double* qt = qtq[j];
  const double* tt = ttq[j];
  if (valid) {
    a.qt64[qi * 256 + tid] = z;
    a.tt64[qi * 256 + tid] = t;
  }
  // operand scales (fp16 mode): exponents of the largest |q~_i|, |t_j|
  double mz = fabs(z), mt = fabs(t);
  for (int o = 32; o >= 1; o >>= 1) {
    mz = fmax(mz, __shfl_xor(mz, o));
    mt = fmax(mt, __shfl_xor(mt, o));
  }
  if ((tid & 63) == 0) { red[4][tid >> 6] = mz; red[5][tid >> 6] = mt; }
  __syncthreads();
  if (tid < 2) {
    const double mx = fmax(fmax(red[4 + tid][0], red[4 + tid][1]), fmax(red[4 + tid][2], red[4 + tid][3]));
    int e = 0;
    if (mx > 0.0) (void)frexp(mx, &e);       // mx in [2^(e-1), 2^e)
    int sc = 15 - e;                          // mx 2^sc in [2^14, 2^15)
    sexp[tid] = sc < -100 ? -100 : (sc > 100 ? 100 : sc);
  }
  __syncthreads();
  const int sq = sexp[0], st = sexp[1];
  // operand values and the norms of the error bound
  double zh = 0.0, th = 0.0;
  if (a.half) {
    zh = ldexp((double)f16_value(f16_operand(ldexp(z, sq))), -sq);
    th = ldexp((double)f16_value(f16_operand(ldexp(t, st))), -st);
  }
  {
    double v0 = z * z, v1 = fabs(t), v2 = (z - zh) * (z - zh), v3 = zh * zh, v4 = fabs(t - th), v5 = fabs(th);
    for (int o = 32; o >= 1; o >>= 1) {
      v0 += __shfl_xor(v0, o); v1 += __shfl_xor(v1, o); v2 += __shfl_xor(v2, o);
      v3 += __shfl_xor(v3, o); v4 += __shfl_xor(v4, o); v5 += __shfl_xor(v5, o);
    }
    __syncthreads();
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = v0; red[1][tid >> 6] = v1; red[2][tid >> 6] = v2;
      red[3][tid >> 6] = v3; red[4][tid >> 6] = v4; red[5][tid >> 6] = v5;
    }
  }
  __syncthreads();
  if (valid && tid < kQInfo) {
    const double sum = red[tid][0] + red[tid][1] + red[tid][2] + red[tid][3];
    a.qinfo[qi * kQInfo + tid] = (tid == 0 || tid == 2 || tid == 3) ? sqrt(sum) : sum;
  }
  if (a.half) {
    const int64_t qb = qi >> 4;
    const int c = (int)(qi & 15);
    const int nh = a.nu / 2;                  // 32-coordinate groups
    uint32_t* rec = a.qop + qb * (int64_t)(nh + a.ns) * 256;
    for (int e = tid; e < (nh + a.ns) * 16; e += 256) {
      const int dw = e & 3, g4 = (e >> 2) & 3, u = e >> 4;
      uint32_t hv[2];
      for (int h2 = 0; h2 < 2; ++h2) {
        const int el = 2 * dw + h2;
        hv[h2] = (u < nh) ? f16_operand(ldexp(qt[32 * u + 8 * g4 + el], sq))
                          : f16_operand(ldexp(tt[32 * (u - nh) + 8 * g4 + el], st));
      }
      rec[(u * 64 + c + 16 * g4) * 4 + dw] = hv[0] | (hv[1] << 16);
    }
    if (tid < 2) a.cinit[qi * 2 + tid] = ldexpf(1.f, tid == 0 ? -(kTabScaleLog2 + sq) : -st);
    __syncthreads();                  // red and sexp are reused by the next query
    continue;
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
    for (int jj = tid; jj < 256; jj += 64) {
      const float v = (float)tt[jj];
      const float fh = __uint_as_float(bf16_rne_bits(v) << 16);
      s += fh + __uint_as_float(bf16_rne_bits(v - fh) << 16);
    }
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (tid == 0) a.cinit[qi] = -ldexpf(s, -kSignShiftIp);
  }
  __syncthreads();                    // red and sexp are reused by the next query
  }
}

// Database bounds of the refinement's error bound: max |scale|, max |rnorm|
// and max_j |c[idx_j]|_2 (float bits; non-negative floats order as their
// bits).  Each workgroup stages 256 rows of codes in LDS with coalesced
// loads; one thread per row then sums c^2 over its codes in float, 32 codes
// (B words) at a time (the result is enlarged by 2^-12 relative where it is
// used).
struct IBArgs {
  const float* scale;
  const float* rnorm;       // or null
  const uint32_t* idx;      // row layout, rw words per vector
  const double* cent64;
  int64_t n;
  int d, bits, rw;
  float* bpart;             // [gridDim.x][3] per-workgroup maxima
};

constexpr int kBoundRows = 256;
constexpr int kBoundBlocks = 1024;    // most workgroups of k_ip_bounds

template <int B, bool WIDE>
__global__ void __launch_bounds__(256) k_ip_bounds(IBArgs a) {
  // widths that divide a byte read |c|^2 sums byte by byte: bt[v] is the sum
  // of c^2 over the codes of byte value v
  constexpr bool kBytes = B == 1 || B == 2 || B == 4 || B == 8;
  __shared__ float c2[1 << B];
  __shared__ float bt[kBytes ? 256 : 1];
  // a minimal row holds B ceil(d/32) <= 8 B words (d <= 256): the buffer is
  // sized for that, so narrow codes leave room for more resident workgroups;
  // WIDE takes rows padded up to the largest pitch
  constexpr int kRowWords = WIDE ? kIpMaxRowBytes / 4 : 8 * B;
  __shared__ __align__(16) uint32_t rows[kBoundRows * kRowWords + 8];
  const int tid = threadIdx.x;
  if (tid < (1 << B)) {
    const double c = a.cent64[tid];
    c2[tid] = (float)(c * c);
  }
  if constexpr (kBytes) {
    float sb = 0.f;
#pragma unroll
    for (int k = 0; k < 8 / B; ++k) {
      const double c = a.cent64[(tid >> (k * B)) & ((1 << B) - 1)];
      sb += (float)(c * c);
    }
    bt[tid] = sb;
  }
  constexpr uint32_t mask = (1u << B) - 1u;
  const int groups = (a.d + 31) / 32;
  float ms = 0.f, mr = 0.f, mc = 0.f;
  for (int64_t base = (int64_t)blockIdx.x * kBoundRows; base < a.n; base += (int64_t)gridDim.x * kBoundRows) {
    const int nr = (int)(a.n - base < kBoundRows ? a.n - base : kBoundRows);
    const int nw = nr * a.rw;
    const uint32_t* src = a.idx + base * a.rw;
    __syncthreads();                     // the previous rows are consumed (and c2 is ready)
    if ((reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
      // 16-byte loads, all of a thread's share in flight before the stores
      constexpr int kPer = kBoundRows * kRowWords / 4 / 256;
      const int nw4 = nw >> 2;
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      uint4* r4 = reinterpret_cast<uint4*>(rows);
      uint4 t4[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (tid + 256 * j < nw4) t4[j] = s4[tid + 256 * j];
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (tid + 256 * j < nw4) r4[tid + 256 * j] = t4[j];
      if (tid < (nw & 3)) rows[4 * nw4 + tid] = src[4 * nw4 + tid];
    } else {
#pragma unroll 8
      for (int e = tid; e < nw; e += 256) rows[e] = src[e];
    }
    __syncthreads();
    if (tid < nr) {
      ms = fmaxf(ms, fabsf(a.scale[base + tid]));
      if (a.rnorm) mr = fmaxf(mr, fabsf(a.rnorm[base + tid]));
      const uint32_t* ir = rows + tid * a.rw;
      float s0 = 0.f, s1 = 0.f;
      int gi = 0;
      if constexpr (kBytes) {
        // whole groups of 32 codes (4B bytes) by byte
        for (; gi < a.d / 32; ++gi) {
#pragma unroll
          for (int j = 0; j < B; ++j) {
            const uint32_t w = ir[B * gi + j];
            s0 += bt[w & 0xFFu] + bt[(w >> 8) & 0xFFu];
            s1 += bt[(w >> 16) & 0xFFu] + bt[w >> 24];
          }
        }
      }
      for (; gi < groups; ++gi) {
        // codes 32 gi .. 32 gi + 31 occupy words B gi .. B gi + B - 1 (past
        // the row's words only for codes past d, which count 0)
        uint32_t w[B];
#pragma unroll
        for (int j = 0; j < B; ++j) w[j] = ir[B * gi + j];
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          const int bit = c * B, wj = bit >> 5, sh = bit & 31;
          uint32_t v = w[wj] >> sh;
          if (sh + B > 32) v |= w[wj + 1] << (32 - sh);
          const float t = (32 * gi + c < a.d) ? c2[v & mask] : 0.f;
          if (c & 1) s1 += t; else s0 += t;
        }
      }
      mc = fmaxf(mc, s0 + s1);
    }
  }
  // one partial (max |scale|, max |rnorm|, max |c[idx]|) per workgroup: many
  // atomics on one address serialise, the refinement reduces the partials
  __shared__ float part[3][4];
  for (int o = 32; o >= 1; o >>= 1) {
    ms = fmaxf(ms, __shfl_xor(ms, o));
    mr = fmaxf(mr, __shfl_xor(mr, o));
    mc = fmaxf(mc, __shfl_xor(mc, o));
  }
  if ((tid & 63) == 0) { part[0][tid >> 6] = ms; part[1][tid >> 6] = mr; part[2][tid >> 6] = mc; }
  __syncthreads();
  if (tid < 3) {
    const float v = fmaxf(fmaxf(part[tid][0], part[tid][1]), fmaxf(part[tid][2], part[tid][3]));
    a.bpart[blockIdx.x * 3 + tid] = (tid == 2) ? sqrtf(v) : v;
  }
}

template <int B>
void launch_bounds(const IBArgs& a, bool wide, dim3 g, dim3 b, hipStream_t st) {
  if (wide) hipLaunchKernelGGL((k_ip_bounds<B, true>), g, b, 0, st, a);
  else hipLaunchKernelGGL((k_ip_bounds<B, false>), g, b, 0, st, a);
}

// Order-preserving keys of floats (larger float, larger key) and back.
__device__ inline uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The k-th largest sample score of each query (the floor of its full pass):
// each thread keeps the KS best of its share in registers (an unrolled
// compare-exchange chain), then a radix select over the 256 KS survivors in
// LDS, 8 bits at a time from the top.  k <= KS.
template <int KS>
__global__ void __launch_bounds__(256) k_ip_floor(const float* sample, int64_t ld, int64_t n, int k, float* floor_v) {
  __shared__ uint32_t keys[256 * KS];
  __shared__ uint32_t hist[256];
  __shared__ int sel[2];
  const int tid = threadIdx.x;
  const float* src = sample + (int64_t)blockIdx.x * ld;
  float r[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) r[j] = -INFINITY;
#pragma unroll 4
  for (int64_t e = tid; e < n; e += 256) {
    float v = src[e];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const float hi = fmaxf(v, r[j]);
      v = fminf(v, r[j]);
      r[j] = hi;
    }
  }
#pragma unroll
  for (int j = 0; j < KS; ++j) keys[tid * KS + j] = fkey(r[j]);
  uint32_t prefix = 0u, pmask = 0u;
  int kr = k;
  for (int dgt = 3; dgt >= 0; --dgt) {
    hist[tid] = 0u;
    __syncthreads();
    for (int e = tid; e < 256 * KS; e += 256) {
      const uint32_t u = keys[e];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> (8 * dgt)) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, bsel = 0;
      for (int bb = 255; bb >= 0; --bb) {
        if (acc + (int)hist[bb] >= kr) { bsel = bb; break; }
        acc += (int)hist[bb];
      }
      sel[0] = bsel;
      sel[1] = kr - acc;
    }
    __syncthreads();
    prefix |= (uint32_t)sel[0] << (8 * dgt);
    pmask |= 255u << (8 * dgt);
    kr = sel[1];
    __syncthreads();
  }
  if (tid == 0) floor_v[blockIdx.x] = fkey_inv(prefix);
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
// distinct, so the order is strict.  Up to kMergeLds candidates are staged
// in LDS first.
constexpr int kMergeLds = 4096;

__global__ void __launch_bounds__(64) k_ip_merge(IMArgs a) {
  __shared__ float ms_[kMergeLds];
  __shared__ int32_t mi_[kMergeLds];
  const int64_t q = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = a.n_chunks * a.k;
  const float* cs = a.cand_s + q * n;
  const int32_t* ci = a.cand_i + q * n;
  const bool staged = n <= kMergeLds;
  if (staged) {
    // eight loads of each array in flight per round
    for (int e0 = 0; e0 < n; e0 += 8 * 64) {
      float ts[8];
      int32_t ti[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + 64 * j + lane;
        if (e < n) { ts[j] = cs[e]; ti[j] = ci[e]; }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + 64 * j + lane;
        if (e < n) { ms_[e] = ts[j]; mi_[e] = ti[j]; }
      }
    }
    __syncthreads();
  }
  float ps = INFINITY;
  int32_t pi = -1;
  for (int o = 0; o < a.k; ++o) {
    float bs = -INFINITY;
    int32_t bi = kNoIndex;
    bool have = false;
    for (int e = lane; e < n; e += 64) {
      const float s = staged ? ms_[e] : cs[e];
      const int32_t i = staged ? mi_[e] : ci[e];
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
  int d, m, bits, rw, sw, nu, ns, k, kc, dp, mp;
  int half;                 // candidates from the fp16 kernel (else bf16 hi/lo)
  double emax_c;            // max_l |c_l - (hi + lo)_l| of the fp16 centroid operands
  int force_scan;           // 1: no query is settled by the candidates
  int64_t* out_idx;
  float* out_score;
  int32_t* flags;           // [nq]: 1 settled by the candidates, 0 needs the scan
  int32_t* fblist;          // [nq] queries that need the scan, bounds[3] of them
  uint32_t* nfb;
  const float* bpart;       // [nbpart][3] per-workgroup database maxima
  int nbpart;
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
    if (id < 0 || (int64_t)id >= a.n_db) id = kNoIndex;      // empty slot
    if (id != kNoIndex) e = exact_score(a, id, sq, st, cent);
  }
  es[lane] = e;
  ei[lane] = id;
  if (lane == 0) ek = -INFINITY;
  // database maxima from the bounds kernel's per-workgroup partials
  float pm0 = 0.f, pm1 = 0.f, pm2 = 0.f;
  for (int b = lane; b < a.nbpart; b += 64) {
    pm0 = fmaxf(pm0, a.bpart[b * 3]);
    pm1 = fmaxf(pm1, a.bpart[b * 3 + 1]);
    pm2 = fmaxf(pm2, a.bpart[b * 3 + 2]);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    pm0 = fmaxf(pm0, __shfl_xor(pm0, o));
    pm1 = fmaxf(pm1, __shfl_xor(pm1, o));
    pm2 = fmaxf(pm2, __shfl_xor(pm2, o));
  }
  const float dbmax[3] = {pm0, pm1, pm2};
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
  __syncthreads();
  if (lane == 0) {
    bool ok = (int64_t)a.kc >= a.n_db;                    // every row was rescored
    if (!ok && !a.force_scan) {
      const double u = 0x1p-24;
      auto gam = [u](double n) { return n * u / (1.0 - n * u); };
      const double smax = (double)dbmax[0];
      const double rmax = (double)dbmax[1];
      const double cn = (double)dbmax[2] * (1.0 + 0x1p-12);   // >= max_j |c[idx_j]|_2
      const double* qi = a.qinfo + q * kQInfo;
      double delta;
      if (a.half) {
        // fp16 operands: exact rounding residuals of the query operands,
        // the centroid table's rounding, accumulation and the final combination
        const double sd = sqrt((double)a.d);
        const double cc = (1.0 + 0x1p-9) * (cn + sd * a.emax_c);   // >= | |c^hi| + |c^lo| |_2
        const double em = smax * (cn * qi[2] + sd * a.emax_c * qi[3]);
        const double et = rmax * qi[4];
        const double ea = 2.0 * (gam(2.0 * a.dp + 16.0) * smax * cc * qi[3] + gam(a.mp + 16.0) * rmax * qi[5]);
        const double ef = 4.0 * u * (smax * cc * qi[3] + rmax * qi[5]);
        delta = 1.5 * (em + et + ea + ef);
      } else {
        const double rel = 0x1p-16 + 0x1p-24;
        const double bm = smax * cn * qi[0];
        const double bq = rmax * qi[1];
        const double nm = 32.0 * a.nu + 16.0, nsk = 32.0 * a.ns + 16.0;
        delta = 2.0 * ((2.0 * rel + rel * rel + gam(nm)) * (1.0 + 2.0 * rel) * bm +
                       (rel + gam(320.0) + 3.0 * gam(nsk)) * bq + 4.0 * u * (bm + bq));
      }
      const float akc = a.acand_s[q * a.kc + a.kc - 1];
      ok = (double)akc + delta < ek;
    }
    a.flags[q] = ok ? 1 : 0;
    if (!ok) a.fblist[atomicAdd(a.nfb, 1u)] = (int32_t)q;
  }
}

// Exact scan for the queries the candidates did not settle: grid
// (slots, kIpFbChunks); each workgroup keeps the k best rows of its share of
// the database by float64 score, for entries blockIdx.x, blockIdx.x +
// gridDim.x, ... of the list of unsettled queries
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
  const int64_t nfb = (int64_t)*a.nfb;
  for (int64_t f = blockIdx.x; f < nfb; f += gridDim.x) {
    const int64_t q = a.fblist[f];
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

__device__ void fbmerge_one(const IRArgs& a, int64_t q) {
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

// One wave per unsettled query (list entries blockIdx.x, blockIdx.x +
// gridDim.x, ...): the k best of its kIpFbChunks scan lists.
__global__ void __launch_bounds__(64) k_ip_fbmerge(IRArgs a) {
  const int64_t nfb = (int64_t)*a.nfb;
  for (int64_t f = blockIdx.x; f < nfb; f += gridDim.x) fbmerge_one(a, a.fblist[f]);
}

}  // namespace

// candidates of the approximate pass: k <= 10 keeps 16, larger k twice k
// (at most kIpCandMax)
static int topk_candidates(int k) { return k <= 10 ? 16 : (2 * k < kIpCandMax ? 2 * k : kIpCandMax); }

TopkPlan plan_topk(int64_t nq, int64_t n_db, int k, int d, int m) {
  TopkPlan p{};
  p.nq = nq; p.n_db = n_db; p.k = k;
  p.kc = topk_candidates(k);
  p.nu = (pad32(d) + 15) / 16;
  p.ns = m > 0 ? (m + 31) / 32 : 0;
  // kc <= 32: fp16 shared-tile kernel, 256 (kc <= 16) or 128 queries per
  // workgroup in blocks of 16; else the bf16 kernel with blocks of 8
  p.shared = p.kc <= 32;
  const int qw = p.kc <= 16 ? 256 : 128;
  p.nqb = p.shared ? (nq + qw - 1) / qw * (qw / 16) : (nq + 7) / 8;
  const int64_t nqp = p.nqb * (p.shared ? 16 : 8);
  p.n_tiles = (n_db + 15) / 16;
  const int64_t groups = p.shared ? p.nqb / (qw / 16) : p.nqb;
  // workgroups: the shared-tile kernel holds one workgroup per CU (one wave
  // per SIMD), so 256 is one round over the CUs
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
  const size_t kc = (size_t)p.kc;
  p.off_qop = off; off = al(off + (size_t)p.nqb * (p.nu + p.ns) * 64 * 16);
  p.off_cinit = off; off = al(off + (size_t)nqp * 2 * 4);
  const size_t nc = (size_t)nqp * p.n_chunks * kc;
  p.off_cand_s = off; off = al(off + nc * 4);
  p.off_cand_i = off; off = al(off + nc * 4);
  // sample pass (shared-tile kernel, databases of 4096 tiles or more):
  // every 64th tile (or a wider stride that keeps the sample scores within
  // 512 MB), whose scores give each query's floor
  p.sample_stride = 0;
  if (p.shared && p.n_tiles >= 64 * 64) {
    int64_t stride = 64;
    while ((size_t)nqp * (p.n_tiles / stride) * 16 * 4 > ((size_t)512 << 20) && p.n_tiles / (stride * 2) >= 64)
      stride *= 2;
    p.sample_stride = stride;
    p.sample_tiles = p.n_tiles / stride;
    int64_t sc = groups > 0 ? (256 + groups - 1) / groups : 1;
    if (sc > p.sample_tiles / 4) sc = p.sample_tiles / 4;
    if (sc < 1) sc = 1;
    p.sample_chunks = (int)sc;
    p.sample_ld = (p.sample_tiles * 16 + 3) / 4 * 4;
    p.off_sample = off; off = al(off + (size_t)nqp * p.sample_ld * 4);
    p.off_floor = off; off = al(off + (size_t)nq * 4);
  }
  p.off_qt64 = off; off = al(off + (size_t)nqp * 256 * 8);
  p.off_tt64 = off; off = al(off + (size_t)nqp * 256 * 8);
  p.off_qinfo = off; off = al(off + (size_t)nqp * kQInfo * 8);
  p.off_bounds = off; off = al(off + 4 * 4);
  p.off_acand_s = off; off = al(off + (size_t)nq * kc * 4);
  p.off_acand_i = off; off = al(off + (size_t)nq * kc * 4);
  p.off_flags = off; off = al(off + (size_t)nq * 4);
  p.off_fb_s = off; off = al(off + (size_t)nq * kIpFbChunks * k * 8);
  p.off_fb_i = off; off = al(off + (size_t)nq * kIpFbChunks * k * 4);
  p.off_fblist = off; off = al(off + (size_t)nq * 4);
  p.off_bpart = off; off = al(off + (size_t)kBoundBlocks * 3 * 4);
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
  const int64_t nqp = plan.nqb * (plan.shared ? 16 : 8);
  int nbp = 1;                          // workgroups of k_ip_bounds

  IPArgs pa{};
  pa.q = queries; pa.nq = plan.nq;
  pa.d = cb->p.d; pa.m = cb->p.qjl_m; pa.dp = cb->dp; pa.mp = cb->mp;
  pa.nu = plan.nu; pa.ns = plan.ns;
  pa.half = plan.shared ? 1 : 0;
  pa.rotT64 = cb->dev.rotT64; pa.qjlT64 = cb->dev.qjlT64;
  pa.qop = qop; pa.cinit = cinit;
  pa.qt64 = reinterpret_cast<double*>(w + plan.off_qt64);
  pa.tt64 = reinterpret_cast<double*>(w + plan.off_tt64);
  pa.qinfo = reinterpret_cast<double*>(w + plan.off_qinfo);
  pa.bounds = bounds;
  hipLaunchKernelGGL(k_ip_prologue, dim3((unsigned)(nqp / kProQ)), dim3(256), 0, stream, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t* idxw = static_cast<const uint32_t*>(db.idx);
  const int rw = (int)(db.idx_row_bytes / 4);
  {
    IBArgs ba{};
    ba.scale = db.scale; ba.rnorm = qjl ? db.rnorm : nullptr;
    ba.idx = idxw; ba.cent64 = cb->dev.cent64;
    ba.n = plan.n_db; ba.d = cb->p.d; ba.bits = cb->p.bits; ba.rw = rw;
    ba.bpart = reinterpret_cast<float*>(w + plan.off_bpart);
    int64_t nb = (plan.n_db + kBoundRows - 1) / kBoundRows;
    if (nb > kBoundBlocks) nb = kBoundBlocks;
    if (nb < 1) nb = 1;
    nbp = (int)nb;
    const dim3 g((unsigned)nb), b(256);
    // rows padded past 8 B words take the buffer for the largest pitch
    const bool wide = rw > 8 * cb->p.bits;
    switch (cb->p.bits) {
      case 1: launch_bounds<1>(ba, wide, g, b, stream); break;
      case 2: launch_bounds<2>(ba, wide, g, b, stream); break;
      case 3: launch_bounds<3>(ba, wide, g, b, stream); break;
      case 4: launch_bounds<4>(ba, wide, g, b, stream); break;
      case 5: launch_bounds<5>(ba, wide, g, b, stream); break;
      case 6: launch_bounds<6>(ba, wide, g, b, stream); break;
      case 7: launch_bounds<7>(ba, wide, g, b, stream); break;
      default: launch_bounds<8>(ba, wide, g, b, stream); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  float* acand_s = reinterpret_cast<float*>(w + plan.off_acand_s);
  int32_t* acand_i = reinterpret_cast<int32_t*>(w + plan.off_acand_i);
  const int sw = qjl ? (int)(db.sign_row_bytes / 4) : 0;
  {
    ProfileScope prof(TQ_KERNEL_TOPK, stream);
    if (plan.shared) {
      IS2Args s2{};
      s2.qop = qop; s2.qsc = cinit;
      s2.idx = idxw; s2.sign = static_cast<const uint32_t*>(db.sign);
      s2.scale = db.scale; s2.rnorm = qjl ? db.rnorm : db.scale;
      s2.tab = cb->dev.pair_tab16;
      s2.n_db = plan.n_db; s2.n_tiles = plan.n_tiles; s2.tiles_per_chunk = plan.tiles_per_chunk;
      s2.rw = rw; s2.sw = sw; s2.bits = cb->p.bits; s2.nu = plan.nu; s2.ns = plan.ns;
      s2.k = plan.kc; s2.n_chunks = plan.n_chunks;
      s2.cand_s = cand_s; s2.cand_i = cand_i;
      s2.tstride = 1;
      s2.nq = plan.nq;
      s2.floor_v = nullptr;
      s2.sample_out = nullptr;
      const bool wide = plan.kc <= 16;
      const unsigned groups = (unsigned)(plan.nqb / (wide ? 16 : 8));
      auto score = [&](const IS2Args& x, dim3 grid) {
        switch (x.nu) {
          case 2: launch_score16_2(x, !wide, grid, stream); break;
          case 4: launch_score16_4(x, !wide, grid, stream); break;
          case 6: launch_score16_6(x, !wide, grid, stream); break;
          case 8: launch_score16_8(x, !wide, grid, stream); break;
          case 10: launch_score16_10(x, !wide, grid, stream); break;
          case 12: launch_score16_12(x, !wide, grid, stream); break;
          case 14: launch_score16_14(x, !wide, grid, stream); break;
          default: launch_score16_16(x, !wide, grid, stream); break;
        }
      };
      if (plan.sample_stride) {
        IS2Args sp = s2;
        sp.tstride = plan.sample_stride;
        sp.n_tiles = plan.sample_tiles;
        sp.n_chunks = plan.sample_chunks;
        sp.tiles_per_chunk = (plan.sample_tiles + plan.sample_chunks - 1) / plan.sample_chunks;
        sp.sample_out = reinterpret_cast<float*>(w + plan.off_sample);
        sp.sample_ld = plan.sample_ld;
        score(sp, dim3((unsigned)plan.sample_chunks, groups));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        float* floor_v = reinterpret_cast<float*>(w + plan.off_floor);
        if (plan.kc <= 16)
          hipLaunchKernelGGL(k_ip_floor<16>, dim3((unsigned)plan.nq), dim3(256), 0, stream, sp.sample_out,
                             plan.sample_ld, plan.sample_tiles * 16, plan.kc, floor_v);
        else
          hipLaunchKernelGGL(k_ip_floor<32>, dim3((unsigned)plan.nq), dim3(256), 0, stream, sp.sample_out,
                             plan.sample_ld, plan.sample_tiles * 16, plan.kc, floor_v);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        s2.floor_v = floor_v;
      }
      score(s2, dim3((unsigned)plan.n_chunks, groups));
    } else {
      ISArgs sa{};
      sa.qop = qop; sa.cinit = cinit;
      sa.idx = idxw;
      sa.sign = static_cast<const uint32_t*>(db.sign);
      sa.scale = db.scale; sa.rnorm = db.rnorm;
      sa.tab = cb->dev.pair_tab;
      sa.n_db = plan.n_db; sa.n_tiles = plan.n_tiles; sa.tiles_per_chunk = plan.tiles_per_chunk;
      sa.rw = rw; sa.sw = sw;
      sa.nu = plan.nu; sa.ns = plan.ns; sa.k = plan.kc; sa.n_chunks = plan.n_chunks;
      sa.cand_s = cand_s; sa.cand_i = cand_i;
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
  ra.idx = idxw; ra.sign = static_cast<const uint32_t*>(db.sign); ra.scale = db.scale; ra.rnorm = db.rnorm;
  ra.nq = plan.nq; ra.n_db = plan.n_db;
  ra.d = cb->p.d; ra.m = cb->p.qjl_m; ra.bits = cb->p.bits; ra.rw = rw; ra.sw = sw;
  ra.dp = cb->dp; ra.mp = cb->mp; ra.half = plan.shared ? 1 : 0; ra.emax_c = cb->emax_c16;
  ra.nu = plan.nu; ra.ns = plan.ns; ra.k = plan.k; ra.kc = plan.kc;
  ra.force_scan = force_scan ? 1 : 0;
  ra.out_idx = out_idx; ra.out_score = out_score;
  ra.flags = reinterpret_cast<int32_t*>(w + plan.off_flags);
  ra.fblist = reinterpret_cast<int32_t*>(w + plan.off_fblist);
  ra.nfb = bounds + 3;
  ra.bpart = reinterpret_cast<const float*>(w + plan.off_bpart);
  ra.nbpart = nbp;
  ra.fb_s = reinterpret_cast<double*>(w + plan.off_fb_s);
  ra.fb_i = reinterpret_cast<int32_t*>(w + plan.off_fb_i);
  hipLaunchKernelGGL(k_ip_refine, dim3((unsigned)plan.nq), dim3(64), 0, stream, ra);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((int64_t)plan.kc < plan.n_db) {
    const unsigned slots = (unsigned)(plan.nq < 64 ? plan.nq : 64);
    hipLaunchKernelGGL(k_ip_fallback, dim3(slots, (unsigned)kIpFbChunks), dim3(256), 0, stream, ra);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_ip_fbmerge, dim3((unsigned)(plan.nq < 1024 ? plan.nq : 1024)), dim3(64), 0, stream, ra);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
