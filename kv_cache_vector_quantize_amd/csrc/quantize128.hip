// Online quantization for head dimension 128 (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog): "第一阶段" items 1-2 (rotate by
// Pi, normalise, Lloyd-Max index per coordinate) and "如何实现 TurboQuant" item 1
// (quantize on every cache update), and "第二阶段：QJL 残差校正" (the sign
// sketch of the residual) for keys with m <= 128 sketch rows.
//
// One workgroup of four waves owns a tile of 32 consecutive positions of one
// sequence (tile32-aligned in absolute position) and loops over tiles.
//
// Rotation.  Wave w computes coordinates 32w .. 32w + 31 of z = Pi x for the
// 32 vectors with v_mfma_f32_32x32x16_bf16.  Pi is split into bf16 parts
// hi + lo (+ lo2) kept in registers (8 k-steps x NP operands); the tile is
// staged in LDS as bf16 parts of x: one for bf16 input (exact), two for fp16
// (exact), three for fp32.  With three parts every product of parts whose
// orders add up to at most 2^-18 is accumulated in fp32 (3, 5 or 6 MFMAs per
// k-step) and y carries fp32-level error.  Two parts (codes of up to 4 bits)
// leave 2^-18 |Pi| per entry, ~2e-7 in y: an index moves only for a
// coordinate that close to a boundary, about 1.5e-5 of the coordinates at 4
// bits against the 1e-4 the zone rule allows (8-bit codebooks have 16x the
// boundaries and need the third part).
//
// Keys with a sketch (row layout) take three parts of Pi, so y and the
// residual r = y - (scale/|x|) c[idx] carry fp32-level error and |r| its
// relative accuracy.  Each wave writes its 32 coordinates of r to LDS as bf16
// hi + lo; after the tile's barrier wave w forms sketch rows 32w .. 32w + 31
// of u = S r with hi.hi + hi.lo + lo.hi products of S (registers) and r
// (about 2^-17 of |S_j| |r|, far inside the 1e-5 zone of the sign rule),
// packs their signs into word w of each sign row and, in wave 0, writes
// rnorm = |x| |r|.
// Row layout codes take z^T (rows = coordinates: a lane holds 16 coordinates
// of one vector); tile32 codes take z (rows = vectors: a lane holds one
// coordinate of 16 vectors, which is how a tile32 record is ordered).
//
// Index.  y = z / |x| lies in [-1, 1]; cell floor((y + 1) G) of a uniform grid
// (cells narrower than the closest pair of decision boundaries, built with
// the codebook) holds the number of boundaries below the cell and the one
// inside it, so idx = count + (y >= boundary).  Both sides of the compare are
// taken in cell coordinates, key = z (G / |x|) + G against (t + 1) G, one FMA
// per coordinate; fp32 rounding of the key only matters when a boundary lies
// within ~3e-7 of y.
//
// Pipeline.  The next tile's input is loaded into registers while the current
// tile is rotated, indexed and packed; the grid holds as many workgroups as
// stay resident, each looping over tiles.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int TILE = 32;
constexpr int XS = 136;   // bf16 row stride of the staged tile (272 bytes: 16-byte lane reads hit distinct banks)

struct Q128Args {
  const void* x;
  int64_t n_tok, tok_off;
  int tiles_per_seq, n_tiles;
  int64_t first_block;
  int bits, nc, ncell;
  float G;
  const uint4* rop;    // Pi operands [4][8][3][64]
  const float* cent;   // [L]
  const int2* qtab;    // [ncell] index cells
  uint8_t* idx;
  float* scale;
  int64_t idx_pitch, seq_stride;
  PageMap pm;          // where a sequence's blocks are written (identity unless paged)
  // keys with a sketch (k_q128<..., true>, row layout): S as hi / lo
  // operands in the layout of rop (rows past m zero), sign rows, residual norms
  const uint4* sop;
  uint32_t* sign;
  float* rnorm;
  int64_t sign_pitch;
  int m;
};

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline uint32_t bf16_bits(float v) {   // round to nearest even
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline float bf16_float(uint32_t h) { return __uint_as_float(h << 16); }

// A thread's share of a tile: row tid/8, 16 consecutive input elements from
// coordinate 16*(tid%8), as raw 16-byte words (zero for rows outside the
// written range).
template <int DT>
struct Share {
  static constexpr int NW = DT == TQ_F32 ? 4 : 2;
  uint4 w[NW];
};

template <int DT>
__device__ inline void share_load(Share<DT>& sh, const void* x, int64_t e0, bool valid, bool vec_ok) {
  constexpr int EB = DT == TQ_F32 ? 4 : 2;
  if (!valid) {
#pragma unroll
    for (int c = 0; c < Share<DT>::NW; ++c) sh.w[c] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const char* p = static_cast<const char*>(x) + e0 * EB;
  if (vec_ok) {
#pragma unroll
    for (int c = 0; c < Share<DT>::NW; ++c) sh.w[c] = reinterpret_cast<const uint4*>(p)[c];
  } else {
    uint32_t t[4 * Share<DT>::NW];
    if constexpr (DT == TQ_F32) {
#pragma unroll
      for (int k = 0; k < 16; ++k) t[k] = reinterpret_cast<const uint32_t*>(p)[k];
    } else {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = (uint32_t)h[2 * k] | ((uint32_t)h[2 * k + 1] << 16);
    }
#pragma unroll
    for (int c = 0; c < Share<DT>::NW; ++c) sh.w[c] = make_uint4(t[4 * c], t[4 * c + 1], t[4 * c + 2], t[4 * c + 3]);
  }
}

template <int DT, bool T32, int NP, bool QJ>
__global__ void __launch_bounds__(256) k_q128(Q128Args a) {
  static_assert(!(QJ && T32), "sketch signs are written in the row layout only");
  constexpr bool XLO = DT != TQ_BF16, XLO2 = DT == TQ_F32;
  __shared__ __align__(16) uint16_t xh[TILE][XS];
  __shared__ __align__(16) uint16_t xl[XLO ? TILE : 1][XS];
  __shared__ __align__(16) uint16_t xl2[XLO2 ? TILE : 1][XS];
  __shared__ __align__(16) uint32_t tb[T32 ? 2 : 1][T32 ? 1024 : 1];   // tile32 block values, field masks
  __shared__ int2 s_tab[kQ128Cells];
  __shared__ float s_cent[256];
  __shared__ float s_n[TILE], s_ig[TILE];
  __shared__ float s_c2[4][TILE];
  __shared__ int s_valid[TILE];
  // residual r of the tile in bf16 hi / lo (B operands of the sketch) and
  // per-wave partial |r|^2
  __shared__ __align__(16) uint16_t rh[QJ ? TILE : 1][QJ ? XS : 8];
  __shared__ __align__(16) uint16_t rl[QJ ? TILE : 1][QJ ? XS : 8];
  __shared__ float s_r2[QJ ? 4 : 1][TILE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, hl = lane >> 5;
  const int b = a.bits, L = 1 << b;
  const bool need_c = a.nc != 0;
  const float G = a.G;
  const int cmax = a.ncell - 1;
  for (int i = tid; i < a.ncell; i += 256) s_tab[i] = a.qtab[i];
  for (int i = tid; i < L; i += 256) s_cent[i] = a.cent[i];

  bf16x8 ph[8], pl[8], pm[NP == 3 ? 8 : 1], sh[QJ ? 8 : 1], sl[QJ ? 8 : 1];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    ph[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 0) * 64 + lane]);
    pl[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 1) * 64 + lane]);
    if constexpr (NP == 3) pm[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 2) * 64 + lane]);
    if constexpr (QJ) {
      sh[s] = __builtin_bit_cast(bf16x8, a.sop[((wave * 8 + s) * 3 + 0) * 64 + lane]);
      sl[s] = __builtin_bit_cast(bf16x8, a.sop[((wave * 8 + s) * 3 + 1) * 64 + lane]);
    }
  }
  const bool vec_ok = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;
  const bool row16 = (a.idx_pitch & 15) == 0;
  const int r8 = tid >> 3, c0 = 16 * (tid & 7);

  // tile -> (sequence, block): positions [32 blk, 32 blk + 32) of sequence seq
  auto where = [&](int tile, int& seq, int64_t& blk) {
    seq = tile / a.tiles_per_seq;
    blk = a.first_block + (tile - seq * a.tiles_per_seq);
  };
  auto fetch = [&](Share<DT>& sh, int tile) {
    int seq;
    int64_t blk;
    where(tile, seq, blk);
    const int64_t p = blk * TILE + r8;
    const bool valid = p >= a.tok_off && p < a.tok_off + a.n_tok;
    share_load<DT>(sh, a.x, ((int64_t)seq * a.n_tok + (p - a.tok_off)) * 128 + c0, valid, vec_ok);
  };

  Share<DT> cur;
  int tile = blockIdx.x;
  if (tile < a.n_tiles) fetch(cur, tile);
  __syncthreads();

  for (; tile < a.n_tiles; tile += gridDim.x) {
    int seq;
    int64_t blk;
    where(tile, seq, blk);
    const int64_t abs0 = blk * TILE;
    int64_t oseq, oblk;                                         // output plane and block
    page_block(a.pm, seq, blk, oseq, oblk);
    const int64_t pos0 = oseq * a.seq_stride + oblk * TILE;     // code row of tile row 0
    const bool full = abs0 >= a.tok_off && abs0 + TILE <= a.tok_off + a.n_tok;

    // (a) stage this thread's share; |x| in fp32 from the input values,
    // reduced over the row's 8 threads
    {
      float s2 = 0.f;
      if constexpr (DT == TQ_BF16) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t w4[4] = {cur.w[c].x, cur.w[c].y, cur.w[c].z, cur.w[c].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const bf16x2 v = __builtin_bit_cast(bf16x2, w4[k]);
            s2 = __builtin_amdgcn_fdot2_f32_bf16(v, v, s2, false);
          }
          *reinterpret_cast<uint4*>(&xh[r8][c0 + 8 * c]) = cur.w[c];
        }
      } else {
        float xv[16];
        if constexpr (DT == TQ_F32) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            xv[4 * c] = __uint_as_float(cur.w[c].x); xv[4 * c + 1] = __uint_as_float(cur.w[c].y);
            xv[4 * c + 2] = __uint_as_float(cur.w[c].z); xv[4 * c + 3] = __uint_as_float(cur.w[c].w);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint32_t w4[4] = {cur.w[c].x, cur.w[c].y, cur.w[c].z, cur.w[c].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              xv[8 * c + 2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w4[k] & 0xFFFFu));
              xv[8 * c + 2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w4[k] >> 16));
            }
          }
        }
        uint32_t hw[8], lw[8], mw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          s2 = fmaf(xv[2 * k], xv[2 * k], s2);
          s2 = fmaf(xv[2 * k + 1], xv[2 * k + 1], s2);
          const uint32_t h0 = bf16_bits(xv[2 * k]), h1 = bf16_bits(xv[2 * k + 1]);
          hw[k] = h0 | (h1 << 16);
          const float e0 = xv[2 * k] - bf16_float(h0), e1 = xv[2 * k + 1] - bf16_float(h1);
          const uint32_t l0 = bf16_bits(e0), l1 = bf16_bits(e1);
          lw[k] = l0 | (l1 << 16);
          if constexpr (XLO2)
            mw[k] = bf16_bits(e0 - bf16_float(l0)) | (bf16_bits(e1 - bf16_float(l1)) << 16);
        }
        *reinterpret_cast<uint4*>(&xh[r8][c0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&xh[r8][c0 + 8]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        *reinterpret_cast<uint4*>(&xl[r8][c0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint4*>(&xl[r8][c0 + 8]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
        if constexpr (XLO2) {
          *reinterpret_cast<uint4*>(&xl2[r8][c0]) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
          *reinterpret_cast<uint4*>(&xl2[r8][c0 + 8]) = make_uint4(mw[4], mw[5], mw[6], mw[7]);
        }
      }
      s2 += __shfl_xor(s2, 1);
      s2 += __shfl_xor(s2, 2);
      s2 += __shfl_xor(s2, 4);
      if ((tid & 7) == 0) {
        const int64_t p = abs0 + r8;
        const float n = sqrtf(s2);
        s_n[r8] = n;
        s_ig[r8] = n > 0.f ? G / n : 0.f;
        s_valid[r8] = (p >= a.tok_off && p < a.tok_off + a.n_tok) ? 1 : 0;
      }
    }
    __syncthreads();
    // the next tile's share is in flight while this one is computed
    if (tile + (int)gridDim.x < a.n_tiles) fetch(cur, tile + (int)gridDim.x);

    // (b) rotation: row layout -> D[coordinate][vector], tile32 -> D[vector][coordinate]
    auto prod = [&](f32x16 c, bf16x8 xo, bf16x8 po) { return T32 ? mfma32(xo, po, c) : mfma32(po, xo, c); };
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 xo = *reinterpret_cast<const bf16x8*>(&xh[c32][16 * s + 8 * hl]);
      if constexpr (XLO) {
        const bf16x8 xq = *reinterpret_cast<const bf16x8*>(&xl[c32][16 * s + 8 * hl]);
        if constexpr (XLO2) {
          const bf16x8 xr = *reinterpret_cast<const bf16x8*>(&xl2[c32][16 * s + 8 * hl]);
          acc = prod(acc, xr, ph[s]);
        }
        acc = prod(acc, xq, pl[s]);
        acc = prod(acc, xq, ph[s]);
      }
      if constexpr (NP == 3) acc = prod(acc, xo, pm[s]);
      acc = prod(acc, xo, pl[s]);
      acc = prod(acc, xo, ph[s]);
    }

    // (c) indices; element v of the lane: row layout -> coordinate
    // 32w + 8(v/4) + 4hl + v%4 of vector c32; tile32 -> coordinate 32w + c32
    // of vector 8(v/4) + 4hl + v%4.  key = (y + 1) G.
    int iv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int vec = T32 ? 8 * (v >> 2) + 4 * hl + (v & 3) : c32;
      const float key = fmaf(acc[v], s_ig[vec], G);
      const int c = min((int)key, cmax);
      const int2 e = s_tab[c];
      iv[v] = e.x + (key >= __int_as_float(e.y) ? 1 : 0);
    }
    if (need_c) {
      // norm correction: per-wave partial |y^|^2 of each vector
      float cv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) cv[v] = s_cent[iv[v]];
      if constexpr (!T32) {
        float c2 = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) c2 = fmaf(cv[v], cv[v], c2);
        c2 += __shfl_xor(c2, 32);
        if (hl == 0) s_c2[wave][c32] = c2;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float c2 = cv[v] * cv[v];
          c2 += __shfl_xor(c2, 1);
          c2 += __shfl_xor(c2, 2);
          c2 += __shfl_xor(c2, 4);
          c2 += __shfl_xor(c2, 8);
          c2 += __shfl_xor(c2, 16);
          if (c32 == 0) s_c2[wave][8 * (v >> 2) + 4 * hl + (v & 3)] = c2;
        }
      }
    }

    // (d) pack and store the indices
    if constexpr (!T32) {
      // this wave's 32 coordinates are b words [w*b, w*b + b) of the row;
      // group g of 4 coordinates (4b bits) lives in half g % 2, slot g / 2
      uint32_t gv[4], go[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t g = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) g |= (uint32_t)iv[4 * q + r] << (r * b);
        gv[q] = g;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) go[q] = (uint32_t)__shfl_xor((int)gv[q], 32);
      if (hl == 0 && s_valid[c32]) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx + (pos0 + c32) * a.idx_pitch) + wave * b;
        if (b == 4 && row16) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(gv[0] | (go[0] << 16), gv[1] | (go[1] << 16),
                                                      gv[2] | (go[2] << 16), gv[3] | (go[3] << 16));
        } else {
          uint64_t buf = 0;
          int nb = 0, wo = 0;
#pragma unroll
          for (int g = 0; g < 8; ++g) {
            const uint32_t val = (g & 1) ? go[g >> 1] : gv[g >> 1];
            buf |= (uint64_t)val << nb;
            nb += 4 * b;
            if (nb >= 32) {
              dst[wo++] = (uint32_t)buf;
              buf >>= 32;
              nb -= 32;
            }
          }
        }
      }
    } else {
      // tile32 record r' = 16G + C holds coordinate 16j + C for tokens
      // 4G + e%4 + 16(e/4), e = 0..7, as 8 consecutive b-bit fields (b bytes)
      // of group r'*8 + j; this lane holds the groups G = hl and G = 2 + hl of
      // coordinate 32w + c32.  The block is assembled in LDS (values and, for
      // partial tiles, field masks), then written out with whole words.
      const int C = c32 & 15, j = 2 * wave + (c32 >> 4);
      const uint64_t fm = (uint64_t)((1u << b) - 1u);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int Gq = hl + 2 * qq;
        uint64_t val = 0, msk = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = 4 * (qq + 2 * (e >> 2)) + (e & 3);
          val |= (uint64_t)iv[v] << (e * b);
          if (!full && s_valid[8 * (v >> 2) + 4 * hl + (v & 3)]) msk |= fm << (e * b);
        }
        const int grp = (16 * Gq + C) * 8 + j;
        uint8_t* vb = reinterpret_cast<uint8_t*>(tb[0]) + grp * b;
        uint8_t* mb = reinterpret_cast<uint8_t*>(tb[1]) + grp * b;
        if (b == 4) {
          *reinterpret_cast<uint32_t*>(vb) = (uint32_t)val;
          if (!full) *reinterpret_cast<uint32_t*>(mb) = (uint32_t)msk;
        } else if (b == 8) {
          *reinterpret_cast<uint2*>(vb) = make_uint2((uint32_t)val, (uint32_t)(val >> 32));
          if (!full) *reinterpret_cast<uint2*>(mb) = make_uint2((uint32_t)msk, (uint32_t)(msk >> 32));
        } else if (b == 2) {
          *reinterpret_cast<uint16_t*>(vb) = (uint16_t)val;
          if (!full) *reinterpret_cast<uint16_t*>(mb) = (uint16_t)msk;
        } else {
          for (int k = 0; k < b; ++k) {
            vb[k] = (uint8_t)(val >> (8 * k));
            if (!full) mb[k] = (uint8_t)(msk >> (8 * k));
          }
        }
      }
    }

    // (e) scale: |x|, or |x| / |y^| with norm correction
    if (need_c) __syncthreads();
    if (wave == 0 && hl == 0 && s_valid[c32]) {
      const float n = s_n[c32];
      float sc = n;
      if (need_c) {
        const float nh = sqrtf(((s_c2[0][c32] + s_c2[1][c32]) + s_c2[2][c32]) + s_c2[3][c32]);
        sc = n / nh;
      }
      a.scale[pos0 + c32] = sc;
    }
    // (g) keys with a sketch: residual r = y - (scale / |x|) c[idx] of this
    // lane's 16 coordinates (element v: coordinate 32w + 8(v/4) + 4hl + v%4
    // of vector c32; scale / |x| is 1, or 1 / |c[idx]| with norm correction,
    // also for x = 0, where y = 0), staged for the sketch product
    float qn = 0.f;
    bool qvalid = false;
    if constexpr (QJ) {
      qn = s_n[c32];
      qvalid = s_valid[c32] != 0;
      float ratio = 1.f;           // scale / |x|
      if (need_c) {
        const float nh = sqrtf(((s_c2[0][c32] + s_c2[1][c32]) + s_c2[2][c32]) + s_c2[3][c32]);
        ratio = 1.f / nh;
      }
      const float inv_n = qn > 0.f ? 1.f / qn : 0.f;
      float r2 = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t hh[2], ll[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int v = 4 * g + 2 * h2 + e;
            const float r = acc[v] * inv_n - ratio * s_cent[iv[v]];
            r2 = fmaf(r, r, r2);
            hh[e] = bf16_bits(r);
            ll[e] = bf16_bits(r - bf16_float(hh[e]));
          }
          hw[h2] = hh[0] | (hh[1] << 16);
          lw[h2] = ll[0] | (ll[1] << 16);
        }
        const int col = 32 * wave + 8 * g + 4 * hl;
        *reinterpret_cast<uint2*>(&rh[c32][col]) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2*>(&rl[c32][col]) = make_uint2(lw[0], lw[1]);
      }
      r2 += __shfl_xor(r2, 32);
      if (hl == 0) s_r2[wave][c32] = r2;
    }
    __syncthreads();
    if constexpr (QJ) {
      // (h) u = S r: sketch rows 32w .. 32w + 31 of the 32 vectors, then the
      // sign bits (u >= 0) of those rows as word w of each sign row, and the
      // residual norm |x| |r|
      f32x16 au = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 xrh = *reinterpret_cast<const bf16x8*>(&rh[c32][16 * s + 8 * hl]);
        const bf16x8 xrl = *reinterpret_cast<const bf16x8*>(&rl[c32][16 * s + 8 * hl]);
        au = mfma32(sh[s], xrl, au);
        au = mfma32(sl[s], xrh, au);
        au = mfma32(sh[s], xrh, au);
      }
      uint32_t bits = 0u;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        bits |= (au[v] >= 0.f ? 1u : 0u) << (8 * (v >> 2) + 4 * hl + (v & 3));
      bits |= (uint32_t)__shfl_xor((int)bits, 32);
      const int rows = a.m - 32 * wave;     // sketch rows of this word
      if (rows < 32) bits &= rows > 0 ? (1u << rows) - 1u : 0u;
      if (hl == 0 && qvalid && rows > 0)
        a.sign[(((pos0 + c32) * a.sign_pitch) >> 2) + wave] = bits;
      if (wave == 0 && hl == 0 && qvalid)
        a.rnorm[pos0 + c32] = qn * sqrtf(((s_r2[0][c32] + s_r2[1][c32]) + s_r2[2][c32]) + s_r2[3][c32]);
    }

    if constexpr (T32) {
      // (f) the assembled tile32 block: 512*b bytes = 128*b words
      const int words = 128 * b;
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx) + (oseq * (a.seq_stride / TILE) + oblk) * (int64_t)words;
      for (int w = tid; w < words; w += 256) {
        if (full) {
          dst[w] = tb[0][w];
        } else {
          const uint32_t nm = tb[1][w];
          if (nm != 0u) dst[w] = (dst[w] & ~nm) | (tb[0][w] & nm);
        }
      }
      __syncthreads();
    }
  }
}

template <int DT, bool T32, int NP, bool QJ>
int resident_grid(int n_tiles) {
  // workgroups that stay resident at once (per device, computed once)
  static int per_device[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (per_device[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_q128<DT, T32, NP, QJ>, 256, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 2;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    per_device[dev] = per_cu * cus;
  }
  return n_tiles < per_device[dev] ? n_tiles : per_device[dev];
}

template <int DT, bool T32, int NP, bool QJ = false>
void launch_np(const Q128Args& a, hipStream_t st) {
  hipLaunchKernelGGL((k_q128<DT, T32, NP, QJ>), dim3(resident_grid<DT, T32, NP, QJ>(a.n_tiles)), dim3(256), 0,
                     st, a);
}

template <int DT>
hipError_t launch_dt(const Q128Args& a, bool t32, hipStream_t st) {
  const bool two = a.bits <= 4;      // two parts of Pi suffice up to 4 bits
  if (a.m > 0) {
    // keys with a sketch: three parts of Pi (fp32-level y, so that |r| keeps
    // its relative accuracy), row layout
    launch_np<DT, false, 3, true>(a, st);
  } else if (t32) {
    if (two) launch_np<DT, true, 2>(a, st);
    else launch_np<DT, true, 3>(a, st);
  } else {
    if (two) launch_np<DT, false, 2>(a, st);
    else launch_np<DT, false, 3>(a, st);
  }
  return hipGetLastError();
}

}  // namespace

bool quantize128_supported(const tq_codebook* cb, const QuantJob& job) {
  const int64_t first = job.tok_offset / TILE, last = (job.tok_offset + job.n_tok - 1) / TILE;
  const int64_t tiles = (last - first + 1) * job.n_seq;
  const bool sketch_ok = cb->p.qjl_m == 0 ||
                         (cb->p.qjl_m <= 128 && cb->dev.sop && job.out.layout == TQ_LAYOUT_ROW);
  return cb->p.d == 128 && sketch_ok && cb->dev.rop && cb->dev.qtab && cb->dev.qcells >= 1 &&
         tiles < 0x7FFFFFFFLL && job.n_seq < 0x7FFFFFFFLL;
}

hipError_t launch_quantize128(const tq_codebook* cb, const QuantJob& job, hipStream_t stream) {
  Q128Args a{};
  a.x = job.x;
  a.n_tok = job.n_tok;
  a.tok_off = job.tok_offset;
  a.first_block = job.tok_offset / TILE;
  const int64_t last_block = (job.tok_offset + job.n_tok - 1) / TILE;
  a.tiles_per_seq = (int)(last_block - a.first_block + 1);
  a.n_tiles = (int)(a.tiles_per_seq * job.n_seq);
  a.bits = cb->p.bits;
  a.nc = cb->p.norm_correction;
  a.ncell = cb->dev.qcells;
  a.G = cb->dev.qG;
  a.rop = reinterpret_cast<const uint4*>(cb->dev.rop);
  a.cent = cb->dev.cent;
  a.qtab = reinterpret_cast<const int2*>(cb->dev.qtab);
  a.idx = static_cast<uint8_t*>(job.out.idx);
  a.scale = job.out.scale;
  a.idx_pitch = job.out.idx_row_bytes;
  a.seq_stride = job.out.seq_stride;
  a.pm = job.pm;
  a.m = cb->p.qjl_m;
  a.sop = reinterpret_cast<const uint4*>(cb->dev.sop);
  a.sign = static_cast<uint32_t*>(job.out.sign);
  a.rnorm = job.out.rnorm;
  a.sign_pitch = job.out.sign_row_bytes;
  const bool t32 = job.out.layout == TQ_LAYOUT_TILE32;
  ProfileScope prof(TQ_KERNEL_QUANTIZE, stream);
  switch (job.dt) {
    case TQ_F32: return launch_dt<TQ_F32>(a, t32, stream);
    case TQ_BF16: return launch_dt<TQ_BF16>(a, t32, stream);
    default: return launch_dt<TQ_F16>(a, t32, stream);
  }
}

}  // namespace tq
