// Decode attention computed from packed codes (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog), "如何实现 TurboQuant" item 1
// and "专业提示": the query is rotated once and attention dot products are
// taken straight from the stored indices; "第二阶段" supplies the QJL
// correction of the inner product.
//
// Three launches:
//  1. prologue, one workgroup per (batch, KV head, group of <= 8 query
//     heads): q~ = Pi_K q scaled by sm_scale*log2(e), t = sqrt(pi/2)/m S_K q~;
//     both are split into bf16 hi + lo and written in the lane order of the
//     B operand of v_mfma_f32_16x16x32_bf16 (columns 0-7 = hi of the 8
//     queries, 8-15 = lo).
//  2. split: each wave streams 32-token tiles of one KV head's codes and
//     computes, on MFMA, S^T = K^ Q~^T (tokens x query columns), the QJL term
//     T^ (2 sigma) - sum(t) (the -sum(t) enters as the accumulator's initial
//     value), the online softmax in base 2, and O^T += V^T P^T in the
//     rotated value domain.  Code operands are expanded through bf16 hi/lo
//     tables in LDS indexed by pairs of packed indices.  hi and lo query
//     columns are summed with one DPP row rotation.
//  3. combine, one workgroup per (batch, query head): log-sum-exp merge of
//     the waves' partials in a fixed order, then out = Pi_V^T o~ / l.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int D = 128;           // head dimension of this kernel family
constexpr int QOP_DWORDS = 2 * 4 * 64 * 4 + 16;   // Q op, T op, 16 C-init floats
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ inline uint32_t bf16_rne_bits(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ inline bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------ 1. prologue

struct PArgs {
  const void* q;
  int qdt;
  int Hq, Hkv, g, qgroups;
  int m;
  float qscale;           // sm_scale * log2(e)
  const float* rotK;      // [D][D]
  const float* qjlK;      // [mp][D] or null
  uint32_t* qop;          // [rows][QOP_DWORDS]
};

__device__ inline float load_q(const void* p, int dt, int64_t i) {
  if (dt == TQ_F32) return static_cast<const float*>(p)[i];
  if (dt == TQ_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
  return (float)static_cast<const _Float16*>(p)[i];
}

__global__ void __launch_bounds__(256) k_prologue(PArgs a) {
  __shared__ float qs[8][D];
  __shared__ float qt[8][D];
  __shared__ float tt[8][D];
  const int row = blockIdx.x;
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;          // b * Hkv + h
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int tid = threadIdx.x;
  for (int e = tid; e < 8 * D; e += 256) {
    const int c = e / D, i = e % D;
    const int j = qg * 8 + c;
    float v = 0.f;
    if (j < a.g) v = load_q(a.q, a.qdt, ((int64_t)b * a.Hq + h * a.g + j) * D + i);
    qs[c][i] = v;
  }
  __syncthreads();
  for (int e = tid; e < 8 * D; e += 256) {
    const int c = e / D, i = e % D;
    float s = 0.f;
    for (int k = 0; k < D; ++k) s += a.rotK[i * D + k] * qs[c][k];
    qt[c][i] = s * a.qscale;
  }
  __syncthreads();
  const float cq = a.m > 0 ? 1.2533141373155003f / (float)a.m : 0.f;   // sqrt(pi/2)/m
  for (int e = tid; e < 8 * D; e += 256) {
    const int c = e / D, j = e % D;
    float s = 0.f;
    if (j < a.m)
      for (int i = 0; i < D; ++i) s += a.qjlK[j * D + i] * qt[c][i];
    tt[c][j] = s * cq;
  }
  __syncthreads();
  uint32_t* dst = a.qop + (int64_t)row * QOP_DWORDS;
  // operand dwords: [op][chunk][lane][4]
  for (int e = tid; e < 2 * 4 * 64 * 4; e += 256) {
    const int p = e & 3, lane = (e >> 2) & 63, chunk = (e >> 8) & 3, op = e >> 10;
    const int col = lane & 15, g4 = lane >> 4;
    const int c = col & 7;
    const bool lo = col >= 8;
    uint32_t halves[2];
    for (int h2 = 0; h2 < 2; ++h2) {
      const int el = 2 * p + h2;           // element 0..7 of the lane's operand
      float v;
      if (op == 0) {
        v = qt[c][32 * g4 + 8 * chunk + el];
      } else {
        const int j = 32 * g4 + 4 * chunk + (el >> 1) + 16 * (el & 1);
        v = tt[c][j];
      }
      const uint32_t hi = bf16_rne_bits(v);
      halves[h2] = lo ? bf16_rne_bits(v - __uint_as_float(hi << 16)) : hi;
    }
    dst[e] = halves[0] | (halves[1] << 16);
  }
  if (tid < 16) {
    float s = 0.f;
    if (tid < 8) {
      for (int j = 0; j < D; ++j) {
        const float v = tt[tid][j];
        const uint32_t hi = bf16_rne_bits(v);
        const float fh = __uint_as_float(hi << 16);
        const float fl = __uint_as_float(bf16_rne_bits(v - fh) << 16);
        s += fh + fl;
      }
    }
    reinterpret_cast<float*>(dst)[2 * 4 * 64 * 4 + tid] = -s;
  }
}

// ------------------------------------------------------------ 2. split

struct SArgs {
  const uint32_t* qop;
  const uint8_t* kidx;
  const uint32_t* ksign;
  const float* kscale;
  const float* krnorm;
  int64_t k_pitch, ks_pitch, k_stride;
  const uint32_t* vidx;
  const float* vscale;
  int64_t v_stride;
  const uint32_t* ktab;
  const uint32_t* vtab;
  int ktab_dwords, vtab_dwords;
  const int32_t* seq_lens;
  int64_t n_ctx;
  int Hq, Hkv, g, qgroups, m;
  int chunk, n_parts;
  float* part_o;     // [rows][n_parts][8][D]
  float* part_ml;    // [rows][n_parts][8][2]
  float* logits;     // [B][Hq][n_ctx] or null
};

// Bits [off, off+w) of a little-endian multi-word field (w <= 32).
template <int NW>
__device__ inline uint32_t field(const uint32_t (&wd)[NW], int off, int w) {
  const int i = off >> 5, s = off & 31;
  uint64_t v = wd[i];
  if (i + 1 < NW) v |= (uint64_t)wd[i + 1] << 32;
  return (uint32_t)(v >> s) & (w >= 32 ? 0xFFFFFFFFu : ((1u << w) - 1u));
}

// Two bf16 hi/lo dwords for codes (a at element 2p, b at 2p+1) from a pair
// field of 2*B bits.
template <int B>
__device__ inline void expand_pair(const uint32_t* tab, uint32_t pair, uint32_t& hi, uint32_t& lo) {
  if constexpr (B <= 4) {
    const uint2 e = reinterpret_cast<const uint2*>(tab)[pair];
    hi = e.x;
    lo = e.y;
  } else {
    const uint32_t e0 = tab[pair & ((1u << B) - 1u)];
    const uint32_t e1 = tab[pair >> B];
    hi = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
    lo = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
  }
}

template <int BK, int BV, bool QJL>
__global__ void __launch_bounds__(256) k_split(SArgs a) {
  __shared__ uint32_t s_ktab[(BK <= 4) ? (2 << (2 * BK)) : (1 << BK)];
  __shared__ uint32_t s_vtab[(BV <= 4) ? (2 << (2 * BV)) : (1 << BV)];
  const int tid = threadIdx.x;
  for (int i = tid; i < a.ktab_dwords; i += 256) s_ktab[i] = a.ktab[i];
  for (int i = tid; i < a.vtab_dwords; i += 256) s_vtab[i] = a.vtab[i];
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int part = blockIdx.x * 4 + wave;
  if (part >= a.n_parts) return;
  const int row = blockIdx.y;
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int64_t seq = bh;                                   // b * Hkv + h
  int64_t n_valid = a.n_ctx;
  if (a.seq_lens) n_valid = a.seq_lens[b];
  const int64_t t_begin = (int64_t)part * a.chunk;
  int64_t t_end = t_begin + a.chunk;
  if (t_end > n_valid) t_end = n_valid;

  // query operands
  const uint32_t* qop = a.qop + (int64_t)row * QOP_DWORDS;
  bf16x8 qa[4], ta[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 v = reinterpret_cast<const u32x4*>(qop)[(0 * 4 + c) * 64 + lane];
    qa[c] = __builtin_bit_cast(bf16x8, v);
    const u32x4 w = reinterpret_cast<const u32x4*>(qop)[(1 * 4 + c) * 64 + lane];
    ta[c] = __builtin_bit_cast(bf16x8, w);
  }
  const float cinit = reinterpret_cast<const float*>(qop)[2 * 4 * 64 * 4 + c16];

  float M = -INFINITY, l = 0.f;
  f32x4 acc_o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc_o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int hq_lane = h * a.g + qg * 8 + (c16 & 7);
  const bool q_valid = qg * 8 + (c16 & 7) < a.g;
  const float* kscale = a.kscale + seq * a.k_stride;
  const float* krnorm = QJL ? a.krnorm + seq * a.k_stride : nullptr;
  const float* vscale = a.vscale + seq * a.v_stride;

  int64_t t0 = t_begin;
  for (; t0 < t_end; t0 += 32) {
    // ---- loads
    uint32_t kw[2][BK];
    uint32_t sw[2] = {0u, 0u};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int64_t r = seq * a.k_stride + t0 + 16 * blk + c16;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.kidx + r * a.k_pitch) + g4 * BK;
#pragma unroll
      for (int i = 0; i < BK; ++i) kw[blk][i] = src[i];
      if constexpr (QJL) {
        if (32 * g4 < a.m) sw[blk] = a.ksign[(r * a.ks_pitch >> 2) + g4];
      }
    }
    f32x4 ks[2], kr[2], vs[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int64_t t = t0 + 16 * blk + 4 * g4;
      ks[blk] = *reinterpret_cast<const f32x4*>(kscale + t);
      vs[blk] = *reinterpret_cast<const f32x4*>(vscale + t);
      if constexpr (QJL) kr[blk] = *reinterpret_cast<const f32x4*>(krnorm + t);
    }
    constexpr int VW = (8 * BV + 31) / 32 + 1 > BV ? BV : (8 * BV + 31) / 32 + 1;
    uint32_t vw[8][2];
    {
      const uint32_t* vb = a.vidx + (seq * (a.v_stride / 32) + t0 / 32) * (int64_t)(D * BV);
      const int off = 8 * BV * g4;
      const int w0 = off >> 5;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint32_t* src = vb + (16 * db + c16) * BV;
        vw[db][0] = src[w0];
        vw[db][1] = (w0 + 1 < BV) ? src[w0 + 1] : 0u;
      }
      (void)VW;
    }

    // ---- logits S^T (tokens x 16 query columns)
    float lg[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t ah[4], al[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t pr = field<BK>(kw[blk], (8 * c + 2 * p) * BK, 2 * BK);
          expand_pair<BK>(s_ktab, pr, ah[p], al[p]);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah[0], ah[1], ah[2], ah[3]), qa[c], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al[0], al[1], al[2], al[3]), qa[c], acc, 0, 0, 0);
      }
      f32x4 accq = {cinit, cinit, cinit, cinit};
      if constexpr (QJL) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t as[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int x = 4 * c + p;
            as[p] = ((sw[blk] >> x) & 0x00010001u) << 14;   // bf16 2.0 or 0 at j, j+16
          }
          accq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(as[0], as[1], as[2], as[3]), ta[c], accq, 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mse = acc[r] + dpp_ror8(acc[r]);
        float v = ks[blk][r] * mse;
        if constexpr (QJL) {
          const float qj = accq[r] + dpp_ror8(accq[r]);
          v += kr[blk][r] * qj;
        }
        const int64_t t = t0 + 16 * blk + 4 * g4 + r;
        lg[blk][r] = (t < t_end) ? v : -INFINITY;
      }
    }
    if (a.logits && c16 < 8 && q_valid) {
      float* dst = a.logits + ((int64_t)b * a.Hq + hq_lane) * a.n_ctx;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t t = t0 + 16 * blk + 4 * g4 + r;
          if (t < a.n_ctx) dst[t] = lg[blk][r] * LN2;
        }
    }

    // ---- online softmax (base 2), per query column
    float mt = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                     fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float Mn = fmaxf(M, mt);
    const float alpha = (Mn == -INFINITY) ? 1.f : exp2f(M - Mn);
    M = Mn;
    float w[2][4];
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (lg[blk][r] == -INFINITY) ? 0.f : exp2f(lg[blk][r] - Mn);
        psum += p;
        w[blk][r] = (p == 0.f) ? 0.f : p * vs[blk][r];
      }
    l = l * alpha + psum;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc_o[db] *= alpha;

    // ---- P^T operand: slot 8*g4+e <-> this lane's tokens; hi or lo column
    uint32_t pb[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t hv[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int e = 2 * p + h2;
        const float x = w[e >> 2][e & 3];
        const float xh = __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
        const float v = (c16 < 8) ? x : (x - xh);
        hv[h2] = __float_as_uint(v) >> 16;
      }
      pb[p] = hv[0] | (hv[1] << 16);
    }
    const bf16x8 pop = as_bf16x8(pb[0], pb[1], pb[2], pb[3]);

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int off = 8 * BV * g4;
      const int s = off & 31;
      const uint64_t fld = (((uint64_t)vw[db][1] << 32) | vw[db][0]) >> s;
      uint32_t ah[4], al[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t pr = (uint32_t)(fld >> (2 * p * BV)) & ((1u << (2 * BV)) - 1u);
        expand_pair<BV>(s_vtab, pr, ah[p], al[p]);
      }
      acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah[0], ah[1], ah[2], ah[3]), pop, acc_o[db], 0, 0, 0);
      acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al[0], al[1], al[2], al[3]), pop, acc_o[db], 0, 0, 0);
    }
  }

  // positions of this wave's range that no tile covered (beyond len_b)
  if (a.logits) {
    int64_t to = t_begin + a.chunk;
    if (to > a.n_ctx) to = a.n_ctx;
    for (int c = 0; c < 8; ++c) {
      if (qg * 8 + c >= a.g) break;
      float* dst = a.logits + ((int64_t)b * a.Hq + h * a.g + qg * 8 + c) * a.n_ctx;
      for (int64_t t = t0 + lane; t < to; t += 64) dst[t] = -INFINITY;
    }
  }

  // ---- wave partial: (M, l, o~) per query column
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int64_t rec = ((int64_t)row * a.n_parts + part) * 8 + (c16 & 7);
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = acc_o[db][r] + dpp_ror8(acc_o[db][r]);
    if (c16 < 8) *reinterpret_cast<f32x4*>(a.part_o + rec * D + 16 * db + 4 * g4) = o;
  }
  if (c16 < 8 && g4 == 0) {
    a.part_ml[rec * 2 + 0] = M;
    a.part_ml[rec * 2 + 1] = l;
  }
}

// ------------------------------------------------------------ 3. combine

struct CArgs {
  const float* part_o;
  const float* part_ml;
  const float* rotV;   // [D][D]
  int Hq, Hkv, g, qgroups, n_parts;
  float* out;          // [B][Hq][D]
};

__global__ void __launch_bounds__(D) k_combine(CArgs a) {
  __shared__ float ov[D];
  const int bq = blockIdx.x;                  // b * Hq + hq
  const int b = bq / a.Hq, hq = bq % a.Hq;
  const int h = hq / a.g, j = hq % a.g;
  const int row = (b * a.Hkv + h) * a.qgroups + j / 8;
  const int c = j % 8;
  const int i = threadIdx.x;
  float Mx = -INFINITY;
  for (int p = 0; p < a.n_parts; ++p)
    Mx = fmaxf(Mx, a.part_ml[(((int64_t)row * a.n_parts + p) * 8 + c) * 2]);
  float lsum = 0.f, o = 0.f;
  if (Mx != -INFINITY) {
    for (int p = 0; p < a.n_parts; ++p) {
      const int64_t rec = ((int64_t)row * a.n_parts + p) * 8 + c;
      const float Mp = a.part_ml[rec * 2];
      if (Mp == -INFINITY) continue;
      const float s = exp2f(Mp - Mx);
      lsum += s * a.part_ml[rec * 2 + 1];
      o += s * a.part_o[rec * D + i];
    }
  }
  ov[i] = (lsum > 0.f) ? o / lsum : 0.f;
  __syncthreads();
  float r = 0.f;
  for (int k = 0; k < D; ++k) r += a.rotV[k * D + i] * ov[k];
  a.out[(int64_t)bq * D + i] = r;
}

template <int BK, int BV>
void launch_split_bits(const SArgs& a, bool qjl, dim3 grid, hipStream_t st) {
  if (qjl) hipLaunchKernelGGL((k_split<BK, BV, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_split<BK, BV, false>), grid, dim3(256), 0, st, a);
}

template <int BK>
void launch_split_bv(const SArgs& a, int bv, bool qjl, dim3 grid, hipStream_t st) {
  switch (bv) {
    case 2: launch_split_bits<BK, 2>(a, qjl, grid, st); break;
    case 3: launch_split_bits<BK, 3>(a, qjl, grid, st); break;
    case 4: launch_split_bits<BK, 4>(a, qjl, grid, st); break;
    default: launch_split_bits<BK, 8>(a, qjl, grid, st); break;
  }
}

bool bits_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 8; }

}  // namespace

bool decode_supported(const tq_codebook* kcb, const tq_codebook* vcb) {
  return kcb->p.d == D && vcb->p.d == D && bits_ok(kcb->p.bits) && bits_ok(vcb->p.bits) &&
         kcb->p.qjl_m <= 128;
}

DecodePlan plan_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_ctx, int d) {
  DecodePlan p{};
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.n_ctx = n_ctx; p.d = d;
  p.g = Hkv > 0 ? (int)(Hq / Hkv) : 0;
  p.qgroups = (p.g + 7) / 8;
  p.rows = B * Hkv * p.qgroups;
  const int64_t target_waves = 2048;
  int64_t parts = p.rows > 0 ? (target_waves + p.rows - 1) / p.rows : 1;
  if (parts < 1) parts = 1;
  int64_t chunk = (n_ctx + parts - 1) / parts;
  chunk = (chunk + 31) / 32 * 32;
  if (chunk < 32) chunk = 32;
  p.chunk = (int)chunk;
  p.n_parts = n_ctx > 0 ? (int)((n_ctx + chunk - 1) / chunk) : 0;
  size_t off = 0;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  p.off_qop = off; off = al(off + (size_t)p.rows * QOP_DWORDS * 4);
  p.off_part_o = off; off = al(off + (size_t)p.rows * p.n_parts * 8 * D * 4);
  p.off_part_ml = off; off = al(off + (size_t)p.rows * p.n_parts * 8 * 2 * 4);
  p.bytes = off;
  return p;
}

hipError_t launch_decode(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                         tq_dtype qdt, const DecodePlan& plan, const tq_codes& k,
                         const tq_codes& v, const int32_t* seq_lens, float sm_scale,
                         float* out, float* logits, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  uint32_t* qop = reinterpret_cast<uint32_t*>(w + plan.off_qop);
  float* part_o = reinterpret_cast<float*>(w + plan.off_part_o);
  float* part_ml = reinterpret_cast<float*>(w + plan.off_part_ml);
  if (plan.rows == 0) return hipSuccess;

  PArgs pa{};
  pa.q = q; pa.qdt = qdt;
  pa.Hq = (int)plan.Hq; pa.Hkv = (int)plan.Hkv; pa.g = plan.g; pa.qgroups = plan.qgroups;
  pa.m = kcb->p.qjl_m;
  pa.qscale = sm_scale * LOG2E;
  pa.rotK = kcb->dev.rot;
  pa.qjlK = kcb->dev.qjl;
  pa.qop = qop;
  hipLaunchKernelGGL(k_prologue, dim3((unsigned)plan.rows), dim3(256), 0, stream, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (plan.n_parts > 0) {
    SArgs sa{};
    sa.qop = qop;
    sa.kidx = static_cast<const uint8_t*>(k.idx);
    sa.ksign = static_cast<const uint32_t*>(k.sign);
    sa.kscale = k.scale;
    sa.krnorm = k.rnorm;
    sa.k_pitch = k.idx_row_bytes;
    sa.ks_pitch = k.sign_row_bytes;
    sa.k_stride = k.seq_stride;
    sa.vidx = static_cast<const uint32_t*>(v.idx);
    sa.vscale = v.scale;
    sa.v_stride = v.seq_stride;
    sa.ktab = kcb->dev.pair_tab;
    sa.vtab = vcb->dev.pair_tab;
    sa.ktab_dwords = kcb->dev.pair_tab_dwords;
    sa.vtab_dwords = vcb->dev.pair_tab_dwords;
    sa.seq_lens = seq_lens;
    sa.n_ctx = plan.n_ctx;
    sa.Hq = (int)plan.Hq; sa.Hkv = (int)plan.Hkv; sa.g = plan.g; sa.qgroups = plan.qgroups;
    sa.m = kcb->p.qjl_m;
    sa.chunk = plan.chunk;
    sa.n_parts = plan.n_parts;
    sa.part_o = part_o;
    sa.part_ml = part_ml;
    sa.logits = logits;
    const dim3 grid((unsigned)((plan.n_parts + 3) / 4), (unsigned)plan.rows);
    const bool qjl = kcb->p.qjl_m > 0;
    switch (kcb->p.bits) {
      case 2: launch_split_bv<2>(sa, vcb->p.bits, qjl, grid, stream); break;
      case 3: launch_split_bv<3>(sa, vcb->p.bits, qjl, grid, stream); break;
      case 4: launch_split_bv<4>(sa, vcb->p.bits, qjl, grid, stream); break;
      default: launch_split_bv<8>(sa, vcb->p.bits, qjl, grid, stream); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  CArgs ca{};
  ca.part_o = part_o;
  ca.part_ml = part_ml;
  ca.rotV = vcb->dev.rot;
  ca.Hq = (int)plan.Hq; ca.Hkv = (int)plan.Hkv; ca.g = plan.g; ca.qgroups = plan.qgroups;
  ca.n_parts = plan.n_parts;
  ca.out = out;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(plan.B * plan.Hq)), dim3(D), 0, stream, ca);
  return hipGetLastError();
}

}  // namespace tq
