// Shared pieces of the inner-product top-k kernels (gfx950): helpers and
// the fp16 score kernel template, instantiated over the operand counts in
// the topk_s16_*.hip units.
#pragma once
#include "tq_internal.hpp"

namespace tq {

struct IS2Args {
  const uint32_t* qop;     // [nqb16][nu + ns][64][4] fp16 query operands
  const float* qsc;        // [nqp][2] 2^-(6+sq), 2^-st
  const uint32_t* idx;     // row layout, rw words per vector
  const uint32_t* sign;    // sw words per vector (or null)
  const float* scale;
  const float* rnorm;      // (scale when there is no sketch)
  const uint32_t* tab;     // fp16 centroid operand table
  int64_t n_db, n_tiles, tiles_per_chunk;
  int64_t tstride;         // tile i of a chunk is database tile (t_begin + i) * tstride
  int64_t nq;
  const float* floor_v;    // [nq] the sample floor of each query, or null
  int rw, sw, bits, nu, ns, k, n_chunks;
  float* cand_s;           // [nqp][n_chunks][k]
  int32_t* cand_i;
  float* sample_out;       // sample pass: [nqp][sample_ld] the score of every sampled row
  int64_t sample_ld;
};

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

constexpr int kTabScaleLog2 = 6;     // fp16 centroid operands carry 2^6

// ------------------------------------------------------------ scores, fp16 operands

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kHWaves = 8;          // two waves per SIMD
constexpr int kHRaw = 16 * (kIpMaxRowBytes / 4) + 16 * (kIpMaxSignRowBytes / 4) + 32;  // words of a raw tile
constexpr int kHPer = (kHRaw + 64 * kHWaves - 1) / (64 * kHWaves);                     // raw words per thread

// the largest float below x (x itself for -inf)
__device__ inline float prev_float(float x) {
  if (x == -INFINITY) return x;
  const int32_t b = __float_as_int(x);
  if (x == 0.f) return -__int_as_float(1);
  return __int_as_float(x > 0.f ? b - 1 : b + 1);
}

__device__ inline f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}


// One workgroup: 8 waves x QB blocks of 16 queries, a chunk of 16-row
// database tiles.  Each wave keeps its queries' operands in registers (one
// record per 32 coordinates, met by the hi and the lo centroid operands, and
// one per 32 sketch rows); a tile's A operands are unpacked once into LDS
// (centroid hi/lo parts from the pair table, +-1 sign elements from a
// 256-entry byte table) and read by all eight waves.  Per tile: MFMAs of
// tile i, the unpack of tile i + 1, the scores of tile i, the LDS store of
// raw tile i + 2 (loaded two tiles earlier) and the global loads of raw tile
// i + 4; one barrier.  A lane appends its rows that score above its query's
// threshold to the query's LDS buffer (an LDS atomic gives the slot); when a
// buffer may overflow in the next tile, a refresh (one thread per query)
// keeps each buffer's best k and raises the threshold to the k-th score.
// Thresholds start at the sample floor of the query when one is given.
// WIDE: codes of more than 4 bits (one table entry per code).  SAMPLE: the
// sample pass, which writes the score of every row it visits (sample tile t
// of the chunk sequence gives rows 16 t .. 16 t + 15 of sample_out) and keeps
// no candidates.
template <int NU, int NS, int QB, int LC, bool WIDE, bool SAMPLE>
__global__ void __launch_bounds__(64 * kHWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_ip_score16(IS2Args a) {
  constexpr int NUS = NU + NS;
  constexpr int QW = kHWaves * QB * 16;                    // queries per workgroup
  __shared__ __align__(16) uint4 s_a[2][NUS][64];          // A operands of a tile
  __shared__ float s_sr[2][2][16];                         // its scale and rnorm
  __shared__ __align__(16) uint32_t s_raw[2][kHRaw];       // raw code rows of a tile
  __shared__ __align__(16) uint32_t s_tab[512];
  __shared__ __align__(16) uint4 s_sgn[256];
  // per-query candidate buffers: up to CAP (score, row) pairs; a refresh
  // keeps the best k and raises the query's threshold to the k-th score
  constexpr int CAP = LC + 24;
  constexpr int QWB = SAMPLE ? 1 : QW;                     // the sample pass keeps no buffers
  __shared__ float s_cs[QWB][CAP];
  __shared__ int32_t s_ci[QWB][CAP];
  __shared__ int s_cnt[QWB];
  __shared__ float s_thr[QWB];                             // a candidate must score above it
  __shared__ int s_need;                                   // some buffer holds more than CAP - 16
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int chunk = blockIdx.x;
  const int64_t qb0 = (int64_t)blockIdx.y * (QW / 16) + wave * QB;   // first 16-query block of the wave
  const int B = a.bits;
  const int tabw = WIDE ? (1 << B) : (2 << (2 * B));
  for (int i = tid; i < tabw; i += 64 * kHWaves) s_tab[i] = a.tab[i];
  for (int bt = tid; bt < 256; bt += 64 * kHWaves) {
    // byte -> eight fp16 elements, +1 where the bit is set, -1 elsewhere
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (((bt >> (2 * j)) & 1) ? 0x3C00u : 0xBC00u) | ((((bt >> (2 * j + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
    s_sgn[bt] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // thresholds start at the sample floor: rows scoring below it cannot be
  // among the final candidates, equal ones can (the test is strict, so the
  // floor's predecessor)
  for (int i = tid; i < QWB; i += 64 * kHWaves) {
    const int64_t q = (int64_t)blockIdx.y * QW + i;
    s_cnt[i] = 0;
    s_thr[i] = (a.floor_v && q < a.nq) ? prev_float(a.floor_v[q]) : -INFINITY;
  }
  if (tid == 0) s_need = 0;
  // this wave's query operands (registers), output scales and floors
  constexpr int NH = NU / 2;                // 32-coordinate groups
  constexpr int NB = NH + NS;               // operand records per block
  f16x8 bq[QB][NB];
  float fm[QB], fq[QB], thq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint4* src = reinterpret_cast<const uint4*>(a.qop) + (qb0 + qb) * (int64_t)NB * 64;
#pragma unroll
    for (int u = 0; u < NB; ++u) bq[qb][u] = __builtin_bit_cast(f16x8, src[u * 64 + lane]);
    const int64_t q = (qb0 + qb) * 16 + c16;
    fm[qb] = a.qsc[q * 2];
    fq[qb] = a.qsc[q * 2 + 1];
    thq[qb] = (a.floor_v && q < a.nq) ? prev_float(a.floor_v[q]) : -INFINITY;
  }

  // fixed share of the raw tile words of this thread, word e = tid + 512 j:
  // idx words [0, 16 rw), sign words [16 rw, 16 rw + 16 sw), scale [.., +16),
  // rnorm [.., +16); wrc[j] = row << 16 | word within the row
  const int n_idx = 16 * a.rw, n_sgn = 16 * a.sw, n_raw = n_idx + n_sgn + 32;
  uint32_t wrc[kHPer];
#pragma unroll
  for (int j = 0; j < kHPer; ++j) {
    const int e = tid + 64 * kHWaves * j;
    int row = 0, col = 0;
    if (e < n_idx) { row = e / a.rw; col = e - row * a.rw; }
    else if (e < n_idx + n_sgn) { row = (e - n_idx) / a.sw; col = e - n_idx - row * a.sw; }
    else if (e < n_raw - 16) row = e - n_idx - n_sgn;
    else if (e < n_raw) row = e - n_raw + 16;
    wrc[j] = (uint32_t)row << 16 | (uint32_t)col;
  }
  const int64_t last = a.n_db - 1;
  struct Pre { uint32_t w[kHPer]; };
  auto raw_load = [&](Pre& P, int64_t tile) {
    const int64_t r0 = tile * 16;
#pragma unroll
    for (int j = 0; j < kHPer; ++j) {
      const int e = tid + 64 * kHWaves * j;
      const int64_t row = min(r0 + (int64_t)(wrc[j] >> 16), last);   // rows past the end repeat the last one
      const int col = (int)(wrc[j] & 0xFFFFu);
      P.w[j] = 0u;
      if (e < n_idx) P.w[j] = a.idx[row * a.rw + col];
      else if (e < n_idx + n_sgn) P.w[j] = a.sign[row * a.sw + col];
      else if (e < n_raw - 16) P.w[j] = __float_as_uint(a.scale[row]);
      else if (e < n_raw) P.w[j] = __float_as_uint(a.rnorm[row]);
    }
  };
  auto raw_store = [&](const Pre& P, int buf) {
#pragma unroll
    for (int j = 0; j < kHPer; ++j)
      if (tid + 64 * kHWaves * j < n_raw) s_raw[buf][tid + 64 * kHWaves * j] = P.w[j];
  };
  // unpack raw slot rs into operand slot os: task (w, lane) = tid + 512 j;
  // w < NH: coordinates 32 w + 8 g + 0..7 of row r into operand slots 2w
  // (hi parts) and 2w + 1 (lo parts); else sign byte g of word w - NH of
  // row r into slot NU + w - NH
  auto build = [&](int rs, int os) {
    const uint32_t* raw = s_raw[rs];
    const char* tab = reinterpret_cast<const char*>(s_tab);
#pragma unroll
    for (int jj = 0; jj < (NB * 64 + 64 * kHWaves - 1) / (64 * kHWaves); ++jj) {
      const int t = tid + 64 * kHWaves * jj;
      if (NB * 64 % (64 * kHWaves) != 0 && t >= NB * 64) break;
      const int w = t >> 6, l = t & 63, r = l & 15, g = l >> 4;
      if (w < NH) {
        const int o = (32 * w + 8 * g) * B;
        const int i0 = o >> 5, sh = o & 31;
        const int i1 = (i0 + 1 < a.rw) ? i0 + 1 : i0;
        const uint32_t lo32 = raw[r * a.rw + i0], hi32 = raw[r * a.rw + i1];
        uint32_t hv[4], lv[4];
        if constexpr (!WIDE) {
          // 8 codes of B <= 4 bits: 8B <= 32 bits from bit sh of the pair of words
          const uint32_t f = __builtin_amdgcn_alignbit(hi32, lo32, sh);
          const uint32_t pm = (1u << (2 * B)) - 1u;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint2 e = *reinterpret_cast<const uint2*>(tab + (((f >> (2 * B * p)) & pm) << 3));
            hv[p] = e.x;
            lv[p] = e.y;
          }
        } else {
          // 8 codes of 5..8 bits span up to three words
          const int i2 = (i0 + 2 < a.rw) ? i0 + 2 : i1;
          const uint64_t f = ((uint64_t)__builtin_amdgcn_alignbit(raw[r * a.rw + i2], hi32, sh) << 32) |
                             __builtin_amdgcn_alignbit(hi32, lo32, sh);
          const uint32_t cm = (1u << B) - 1u;
          const uint32_t* t32 = reinterpret_cast<const uint32_t*>(tab);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t ca = t32[(uint32_t)(f >> (2 * B * p)) & cm];
            const uint32_t cb = t32[(uint32_t)(f >> (2 * B * p + B)) & cm];
            hv[p] = __builtin_amdgcn_perm(cb, ca, 0x05040100u);
            lv[p] = __builtin_amdgcn_perm(cb, ca, 0x07060302u);
          }
        }
        s_a[os][2 * w][l] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
        s_a[os][2 * w + 1][l] = make_uint4(lv[0], lv[1], lv[2], lv[3]);
      } else {
        const uint32_t sb = (raw[n_idx + r * a.sw + (w - NH)] >> (8 * g)) & 0xFFu;
        s_a[os][NU + w - NH][l] = s_sgn[sb];
      }
    }
    if (tid < 32) s_sr[os][tid >> 4][tid & 15] = __uint_as_float(raw[n_idx + n_sgn + tid]);
  };

  const int64_t t_begin = (int64_t)chunk * a.tiles_per_chunk;
  int64_t t_end = t_begin + a.tiles_per_chunk;
  if (t_end > a.n_tiles) t_end = a.n_tiles;
  const int64_t nt = t_end > t_begin ? t_end - t_begin : 0;
  auto dbt = [&](int64_t i) { return (t_begin + i) * a.tstride; };   // database tile of step i

  // MFMAs of the tile in operand slot cs
  auto mfma_phase = [&](const int cs, f32x4 (&am)[QB], f32x4 (&aq)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      am[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      aq[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    // A operands PF steps ahead of their MFMAs
    constexpr int PF = 4;
    f16x8 aw[NUS];
#pragma unroll
    for (int u = 0; u < PF && u < NUS; ++u) aw[u] = __builtin_bit_cast(f16x8, s_a[cs][u][lane]);
#pragma unroll
    for (int u = 0; u < NUS; ++u) {
      if (u + PF < NUS) aw[u + PF] = __builtin_bit_cast(f16x8, s_a[cs][u + PF][lane]);
      if (u < NU) {
        // operand slots 2w, 2w + 1: hi, lo parts of coordinate group w
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) am[qb] = mfma16(aw[u], bq[qb][u >> 1], am[qb]);
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) aq[qb] = mfma16(aw[u], bq[qb][NH + u - NU], aq[qb]);
      }
    }
  };
  // scale and rnorm of this lane's rows of the tile in slot cs
  auto load_sr = [&](const int cs, float (&sc)[4], float (&rn)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = s_sr[cs][0][4 * g4 + r];
      rn[r] = s_sr[cs][1][4 * g4 + r];
    }
  };
  // scores of the tile starting at row0 and the appends of those above the
  // thresholds
  auto epilogue = [&](const f32x4 (&am)[QB], const f32x4 (&aq)[QB], const float (&sc)[4], const float (&rn)[4],
                      const int64_t row0, const int64_t srow0) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = (sc[r] * fm[qb]) * am[qb][r];
        if constexpr (NS > 0) v = fmaf(rn[r] * fq[qb], aq[qb][r], v);
        sv[r] = (row0 + 4 * g4 + r < a.n_db) ? v : -INFINITY;
      }
      if constexpr (SAMPLE) {
        const int64_t q = (qb0 + qb) * 16 + c16;
        *reinterpret_cast<float4*>(a.sample_out + q * a.sample_ld + srow0 + 4 * g4) =
            make_float4(sv[0], sv[1], sv[2], sv[3]);
      } else {
        uint32_t pm = 0u;               // rows of this lane above the query's threshold
#pragma unroll
        for (int r = 0; r < 4; ++r) pm |= (sv[r] > thq[qb]) ? (1u << r) : 0u;
        if (pm) {
          // append (at most 16 rows per query and step; the buffer holds at
          // most CAP - 16 before the step)
          const int li = (wave * QB + qb) * 16 + c16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if ((pm >> r) & 1u) {
              const int slot = atomicAdd(&s_cnt[li], 1);
              s_cs[li][slot] = sv[r];
              s_ci[li][slot] = (int32_t)(row0 + 4 * g4 + r);
              if (slot >= CAP - 16) s_need = 1;
            }
          }
        }
      }
    }
  };
  // The two waves of a SIMD work out of phase so that one's MFMAs overlap the
  // other's unpack and scores.  Step i, tile i in operand slot cs, tile
  // i + 1 in raw slot cs ^ 1:
  //  waves 0-3: MFMAs of tile i, unpack of tile i + 1, scores of tile i;
  //  waves 4-7: unpack of tile i + 1, scores of tile i - 1 (accumulators
  //             kept from the previous step), MFMAs of tile i.
  const bool lead = wave < kHWaves / 2;
  f32x4 pam[QB], paq[QB];
  float psc[4], prn[4];
  int64_t prow0 = -1;                   // row0 of the tile held in pam, paq (-1: none)
  int64_t psrow0 = 0;
  auto tile_step = [&](const int cs, const int64_t i) __attribute__((always_inline)) {
    const int64_t row0 = dbt(i) * 16, srow0 = (t_begin + i) * 16;
    if (lead) {
      f32x4 am[QB], aq[QB];
      float sc[4], rn[4];
      mfma_phase(cs, am, aq);
      build(cs ^ 1, cs ^ 1);          // past the last tile it rebuilds a slot nobody reads
      load_sr(cs, sc, rn);
      epilogue(am, aq, sc, rn, row0, srow0);
    } else {
      build(cs ^ 1, cs ^ 1);
      if (prow0 >= 0) epilogue(pam, paq, psc, prn, prow0, psrow0);
      mfma_phase(cs, pam, paq);
      load_sr(cs, psc, prn);
      prow0 = row0;
      psrow0 = srow0;
    }
  };

  // keep the best `keep` entries of buffer li in slots [0, keep), in
  // (score desc, index asc) order; empty slots read (-inf, no index)
  auto select_top = [&](int li, int keep) {
    const int n = s_cnt[li];
    for (int o = 0; o < keep; ++o) {
      float bs = -INFINITY;
      int32_t bi = kNoIndex;
      int bj = -1;
      for (int j = o; j < n; ++j) {
        const float hs = s_cs[li][j];
        const int32_t hi = s_ci[li][j];
        if (bj < 0 || better(hs, hi, bs, bi)) { bs = hs; bi = hi; bj = j; }
      }
      if (bj >= 0) {
        s_cs[li][bj] = s_cs[li][o];
        s_ci[li][bj] = s_ci[li][o];
      }
      s_cs[li][o] = bs;
      s_ci[li][o] = bi;
    }
  };
  // after a barrier: when some buffer may overflow in the next tile, every
  // buffer above k entries keeps its best k (k <= LC) and its threshold
  // rises to the k-th score (uniform branch: s_need is read after the barrier)
  auto refresh = [&]() {
    if constexpr (!SAMPLE) {
      if (s_need) {
        __syncthreads();
        if (tid < QW && s_cnt[tid] > a.k) {
          select_top(tid, a.k);
          s_cnt[tid] = a.k;
          s_thr[tid] = fmaxf(s_thr[tid], s_cs[tid][a.k - 1]);
        }
        if (tid == 0) s_need = 0;
        __syncthreads();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) thq[qb] = s_thr[(wave * QB + qb) * 16 + c16];
      }
    }
  };

  // prologue: raw tiles 0, 1 -> raw slots 0, 1; tile 0 -> operand slot 0;
  // raw tiles 2, 3 in registers
  Pre p0, p1;
  raw_load(p0, dbt(0));
  raw_load(p1, dbt(1));
  raw_store(p0, 0);
  raw_store(p1, 1);
  raw_load(p0, dbt(2));
  raw_load(p1, dbt(3));
  __syncthreads();
  build(0, 0);
  __syncthreads();

  // step i: tile i in operand slot i & 1, tile i + 1 in raw slot (i + 1) & 1,
  // tile i + 2 in registers (p0 for even i, p1 for odd i)
  for (int64_t i = 0; i < nt; i += 2) {
    tile_step(0, i);
    raw_store(p0, 0);
    raw_load(p0, dbt(i + 4));
    __syncthreads();
    refresh();
    if (i + 1 < nt) {
      tile_step(1, i + 1);
      raw_store(p1, 1);
      raw_load(p1, dbt(i + 5));
      __syncthreads();
      refresh();
    }
  }
  // the trailing waves' last tile
  if (!lead && prow0 >= 0) epilogue(pam, paq, psc, prn, prow0, psrow0);
  if constexpr (!SAMPLE) {
    __syncthreads();
    refresh();

    // each query's best k of the chunk, (score desc, index asc)
    if (tid < QW) {
      select_top(tid, a.k);
      const int64_t q = (int64_t)blockIdx.y * QW + tid;
      const int64_t base = (q * a.n_chunks + chunk) * (int64_t)a.k;
      for (int o = 0; o < a.k; ++o) {
        a.cand_s[base + o] = s_cs[tid][o];
        a.cand_i[base + o] = s_ci[tid][o];
      }
    }
  }
}

template <int NU, int NS, int QB, int LC>
void launch_score16_ns(const IS2Args& a, int ns, dim3 grid, hipStream_t st) {
  if constexpr (NS > kIpNsMax) {
    (void)a; (void)ns; (void)grid; (void)st;
  } else {
    if (ns != NS) launch_score16_ns<NU, NS + 1, QB, LC>(a, ns, grid, st);
    else if (a.sample_out) {
      if (a.bits > 4) hipLaunchKernelGGL((k_ip_score16<NU, NS, QB, LC, true, true>), grid, dim3(64 * kHWaves), 0, st, a);
      else hipLaunchKernelGGL((k_ip_score16<NU, NS, QB, LC, false, true>), grid, dim3(64 * kHWaves), 0, st, a);
    } else if (a.bits > 4) {
      hipLaunchKernelGGL((k_ip_score16<NU, NS, QB, LC, true, false>), grid, dim3(64 * kHWaves), 0, st, a);
    } else {
      hipLaunchKernelGGL((k_ip_score16<NU, NS, QB, LC, false, false>), grid, dim3(64 * kHWaves), 0, st, a);
    }
  }
}

// QB 2 with lists of 16 (narrow false) or QB 1 with lists of 32
template <int NU>
void launch_score16_fixed(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  if (narrow) launch_score16_ns<NU, 0, 1, 32>(a, a.ns, grid, st);
  else launch_score16_ns<NU, 0, 2, 16>(a, a.ns, grid, st);
}

}  // namespace

// k_ip_score16 for a.nu == 2, 4, ..., 16 (one per unit topk_s16_*.hip)
void launch_score16_2(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);
void launch_score16_4(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);
void launch_score16_6(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);
void launch_score16_8(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);
void launch_score16_10(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);
void launch_score16_12(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);
void launch_score16_14(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);
void launch_score16_16(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st);

}  // namespace tq
