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
// Keys with a sketch (row layout, k_q128sk) take three parts of Pi, so y and
// the residual r = y - (scale/|x|) c[idx] carry fp32-level error and |r| its
// relative accuracy.  Eight waves: the four rotation waves write their 32
// coordinates of r to LDS as bf16 hi + lo; one pass later sketch wave w
// forms sketch rows 32w .. 32w + 31 of u = S r with hi.hi + hi.lo + lo.hi
// products of S (registers) and r (about 2^-17 of |S_j| |r|, far inside the
// 1e-5 zone of the sign rule), packs their signs into word w of each sign
// row and, in sketch wave 0, writes rnorm = |x| |r|.
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
// within ~3e-7 of y.  The staged table is padded to kQ128Cells entries with
// the last cell, so the truncated key needs no clamp: for finite input |y|
// exceeds 1 by far less than one cell.  |x| comes from the hardware square
// root (within 1 ulp) and G / |x| from the hardware reciprocal.
//
// Pipeline.  The inputs of the next two tiles are in flight in registers
// while the current tile is rotated, indexed and packed; the grid holds as
// many workgroups as stay resident, each looping over tiles.
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

typedef __attribute__((ext_vector_type(2))) float f32x2;

// {hi(y0) | hi(y1) << 16, lo(y0) | lo(y1) << 16}: hi the bf16 rounding (to
// nearest even) of y, lo that of y - hi, two values per conversion
__device__ inline uint2 split_pair(float y0, float y1) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y0, y1}, bf16x2));
  const float r0 = y0 - __uint_as_float(h << 16);
  const float r1 = y1 - __uint_as_float(h & 0xFFFF0000u);
  return make_uint2(h, __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){r0, r1}, bf16x2)));
}

// The b bytes (b <= 8) of one tile32 group, little-endian; the block base is
// 4-byte aligned, so 4-, 2- and 1-byte groups are naturally aligned and
// 8-byte ones are two words.
__device__ inline uint64_t group_load(const uint8_t* p, int b) {
  if (b == 4) return *reinterpret_cast<const uint32_t*>(p);
  if (b == 2) return *reinterpret_cast<const uint16_t*>(p);
  if (b == 1) return *p;
  if (b == 8) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
    return (uint64_t)w[0] | ((uint64_t)w[1] << 32);
  }
  uint64_t v = 0;
  for (int k = 0; k < b; ++k) v |= (uint64_t)p[k] << (8 * k);
  return v;
}

__device__ inline void group_store(uint8_t* p, int b, uint64_t v) {
  if (b == 4) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)v;
  } else if (b == 2) {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)v;
  } else if (b == 1) {
    *p = (uint8_t)v;
  } else if (b == 8) {
    uint32_t* w = reinterpret_cast<uint32_t*>(p);
    w[0] = (uint32_t)v;
    w[1] = (uint32_t)(v >> 32);
  } else {
    for (int k = 0; k < b; ++k) p[k] = (uint8_t)(v >> (8 * k));
  }
}

// A thread's share of a tile: row tid/8, 16 consecutive input elements from
// coordinate 16*(tid%8), as raw 16-byte words.  Every fetch issues the same
// loads (rows outside the written range read a row inside it and are zeroed
// when staged), so the count of loads in flight is the same on every path
// into a tile and a tile's wait does not drain the next tile's loads.
template <int DT>
struct Share {
  static constexpr int NW = DT == TQ_F32 ? 4 : 2;
  uint4 w[NW];
};

template <int DT>
__device__ inline void share_load(Share<DT>& sh, const void* x, int64_t e0, bool vec_ok) {
  constexpr int EB = DT == TQ_F32 ? 4 : 2;
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

// The staged words of a share: zero for a row outside the written range.
template <int DT>
__device__ inline void share_mask(Share<DT>& sh, bool valid) {
  const uint32_t m = valid ? 0xFFFFFFFFu : 0u;   // an AND in place, no branch
#pragma unroll
  for (int c = 0; c < Share<DT>::NW; ++c) {
    sh.w[c].x &= m; sh.w[c].y &= m; sh.w[c].z &= m; sh.w[c].w &= m;
  }
}

// Sum over each group of 8 consecutive lanes, in every lane of the group: DPP
// exchanges within quads (lane ^ 1, lane ^ 2), then between the two quads of
// each half row (mirror within 8 lanes); no LDS round trip.
__device__ inline float sum8(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

// |x| from |x|^2: the hardware square root (within 1 ulp) for normal inputs,
// the correctly rounded library one below 2^-100
__device__ inline float norm_from_sq(float s2) {
  if (__builtin_expect(s2 < 0x1p-100f, 0)) return sqrtf(s2);
  return __builtin_amdgcn_sqrtf(s2);
}

// All vector-memory loads issued so far have landed (vmcnt(0), other counters
// left alone): the loop that follows then never waits on the operand loads.
__device__ inline void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DT, bool T32, int NP>
// two-part variants keep three workgroups per CU
__global__ void __launch_bounds__(256, NP == 2 ? 3 : 1) k_q128(Q128Args a) {
  constexpr bool XLO = DT != TQ_BF16, XLO2 = DT == TQ_F32;
  // NB = 2 (bf16 input): the staged tile and its per-vector data alternate
  // between two buffers, so a tile ends without a barrier (the next tile's
  // staging writes the other buffers);
  // fp16 and fp32 input stage two or three parts of x and keep one buffer
  // and the barrier, which holds their LDS to what three workgroups per CU
  // can share
  constexpr int NB = DT == TQ_BF16 ? 2 : 1;
  __shared__ __align__(16) uint16_t xh[NB][TILE][XS];
  __shared__ __align__(16) uint16_t xl[XLO ? NB : 1][XLO ? TILE : 1][XS];
  __shared__ __align__(16) uint16_t xl2[XLO2 ? NB : 1][XLO2 ? TILE : 1][XS];
  __shared__ int2 s_tab[kQ128Cells];
  __shared__ float s_cent[256];
  __shared__ __align__(16) float s_n[NB][TILE];
  __shared__ __align__(16) float s_ig[NB][TILE];
  __shared__ float s_c2[4][TILE];
  __shared__ int s_valid[NB][TILE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, hl = lane >> 5;
  const int b = a.bits, L = 1 << b;
  const bool need_c = a.nc != 0;
  const float G = a.G;
  const int cmax = a.ncell - 1;
  for (int i = tid; i < kQ128Cells; i += 256) s_tab[i] = a.qtab[i < cmax ? i : cmax];
  for (int i = tid; i < L; i += 256) s_cent[i] = a.cent[i];

  bf16x8 ph[8], pl[8], pm[NP == 3 ? 8 : 1];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    ph[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 0) * 64 + lane]);
    pl[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 1) * 64 + lane]);
    if constexpr (NP == 3) pm[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 2) * 64 + lane]);
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
    where(tile < a.n_tiles ? tile : a.n_tiles - 1, seq, blk);
    int64_t p = blk * TILE + r8;
    p = p < a.tok_off ? a.tok_off : (p >= a.tok_off + a.n_tok ? a.tok_off + a.n_tok - 1 : p);
    share_load<DT>(sh, a.x, ((int64_t)seq * a.n_tok + (p - a.tok_off)) * 128 + c0, vec_ok);
  };

  // two tiles in flight per workgroup: the share of tile + 2 G is fetched
  // into the registers of tile as soon as that tile sits in LDS
  const int G2 = 2 * (int)gridDim.x;
  auto step = [&](Share<DT>& cur, const int tile, const int q) __attribute__((always_inline)) {
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
      // a tile inside the written range stages every row as loaded
      if (!full) share_mask<DT>(cur, abs0 + r8 >= a.tok_off && abs0 + r8 < a.tok_off + a.n_tok);
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
          *reinterpret_cast<uint4*>(&xh[q][r8][c0 + 8 * c]) = cur.w[c];
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
        *reinterpret_cast<uint4*>(&xh[q][r8][c0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&xh[q][r8][c0 + 8]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        *reinterpret_cast<uint4*>(&xl[q][r8][c0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint4*>(&xl[q][r8][c0 + 8]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
        if constexpr (XLO2) {
          *reinterpret_cast<uint4*>(&xl2[q][r8][c0]) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
          *reinterpret_cast<uint4*>(&xl2[q][r8][c0 + 8]) = make_uint4(mw[4], mw[5], mw[6], mw[7]);
        }
      }
      s2 = sum8(s2);
      if ((tid & 7) == 0) {
        const int64_t p = abs0 + r8;
        const float n = norm_from_sq(s2);
        s_n[q][r8] = n;
        s_ig[q][r8] = n > 0.f ? G * __builtin_amdgcn_rcpf(n) : 0.f;
        s_valid[q][r8] = (p >= a.tok_off && p < a.tok_off + a.n_tok) ? 1 : 0;
      }
    }
    __syncthreads();
    // the share of the tile after next goes in flight while this one is computed
    fetch(cur, tile + G2);

    // (b) rotation: row layout -> D[coordinate][vector], tile32 -> D[vector][coordinate]
    auto prod = [&](f32x16 c, bf16x8 xo, bf16x8 po) { return T32 ? mfma32(xo, po, c) : mfma32(po, xo, c); };
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 xo = *reinterpret_cast<const bf16x8*>(&xh[q][c32][16 * s + 8 * hl]);
      if constexpr (XLO) {
        const bf16x8 xq = *reinterpret_cast<const bf16x8*>(&xl[q][c32][16 * s + 8 * hl]);
        if constexpr (XLO2) {
          const bf16x8 xr = *reinterpret_cast<const bf16x8*>(&xl2[q][c32][16 * s + 8 * hl]);
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
      const float key = fmaf(acc[v], s_ig[q][vec], G);
      const int c = (int)key;
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
      for (int q = 0; q < 4; ++q) go[q] = __builtin_amdgcn_permlane32_swap(gv[q], gv[q], false, false)[1];
      if (hl == 0 && s_valid[q][c32]) {
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
      // coordinate 32w + c32.  Every group has one owner, which stores its b
      // bytes straight into the block (merging with the stored fields of
      // positions outside the written range in a partial tile).
      const int C = c32 & 15, j = 2 * wave + (c32 >> 4);
      uint8_t* blk = a.idx + (oseq * (a.seq_stride / TILE) + oblk) * (int64_t)(512 * b);
      const uint64_t fm = (uint64_t)((1u << b) - 1u);
      if (b == 4 && full) {
        // 4-bit codes, whole tile: each group is one aligned word
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          uint32_t v32 = 0u;
#pragma unroll
          for (int e = 0; e < 8; ++e) v32 |= (uint32_t)iv[4 * (qq + 2 * (e >> 2)) + (e & 3)] << (4 * e);
          reinterpret_cast<uint32_t*>(blk)[(16 * (hl + 2 * qq) + C) * 8 + j] = v32;
        }
      } else
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int Gq = hl + 2 * qq;
        uint64_t val = 0, msk = 0;
        if (b <= 4) {
          // the 8 fields fit one word: 32-bit shifts
          uint32_t v32 = 0u;
#pragma unroll
          for (int e = 0; e < 8; ++e) v32 |= (uint32_t)iv[4 * (qq + 2 * (e >> 2)) + (e & 3)] << (e * b);
          val = v32;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) val |= (uint64_t)iv[4 * (qq + 2 * (e >> 2)) + (e & 3)] << (e * b);
        }
        if (!full) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int v = 4 * (qq + 2 * (e >> 2)) + (e & 3);
            if (s_valid[q][8 * (v >> 2) + 4 * hl + (v & 3)]) msk |= fm << (e * b);
          }
        }
        uint8_t* gp = blk + ((16 * Gq + C) * 8 + j) * b;
        if (full) group_store(gp, b, val);
        else if (msk != 0) group_store(gp, b, (group_load(gp, b) & ~msk) | (val & msk));
      }
    }

    // (e) scale: |x|, or |x| / |y^| with norm correction
    if (need_c) __syncthreads();
    if (wave == 0 && hl == 0 && s_valid[q][c32]) {
      const float n = s_n[q][c32];
      float sc = n;
      if (need_c) {
        const float nh = sqrtf(((s_c2[0][c32] + s_c2[1][c32]) + s_c2[2][c32]) + s_c2[3][c32]);
        sc = n / nh;
      }
      a.scale[pos0 + c32] = sc;
    }
    // with one buffer the next tile's staging overwrites what this tile's
    // waves still read
    if (NB == 1) __syncthreads();
  };

  Share<DT> s0, s1;
  int tile = blockIdx.x;
  wait_loads();
  fetch(s0, tile);
  fetch(s1, tile + (int)gridDim.x);
  __syncthreads();
  for (; tile < a.n_tiles; tile += G2) {
    step(s0, tile, 0);
    if (tile + (int)gridDim.x >= a.n_tiles) break;
    step(s1, tile + (int)gridDim.x, NB - 1);
  }
}

// Keys with a sketch: eight waves per workgroup.  Waves 0-3 ("rotation
// waves") do what k_q128 does for a row-layout tile with three parts of Pi
// (stage, rotate, index, pack, scale) and write the residual r of their 32
// coordinates to LDS as bf16 hi + lo; waves 4-7 ("sketch waves") form
// u = S r for the tile before, its sign words and rnorm.  The two halves of
// a tile's work thus overlap on every SIMD (one wave of each per SIMD), and a
// wave holds either the three parts of its slice of Pi or the two of its
// slice of S, in the same registers.  Residuals and per-vector data of a
// tile are double-buffered between the halves; one pass of the loop takes a
// new tile into the rotation waves and the previous one into the sketch waves.
template <int DT>
__global__ void __launch_bounds__(512, 1) k_q128sk(Q128Args a) {
  constexpr bool XLO = DT != TQ_BF16, XLO2 = DT == TQ_F32;
  // one barrier per pass: the staged tile and its scales alternate between
  // two buffers, the per-vector norms and flags (also read by the sketch
  // waves one pass later) between three
  __shared__ __align__(16) uint16_t xh[2][TILE][XS];
  __shared__ __align__(16) uint16_t xl[XLO ? 2 : 1][XLO ? TILE : 1][XS];
  __shared__ __align__(16) uint16_t xl2[XLO2 ? 2 : 1][XLO2 ? TILE : 1][XS];
  __shared__ int2 s_tab[kQ128Cells];
  __shared__ float s_cent[256];
  __shared__ float s_ig[2][TILE];
  __shared__ float s_c2[4][TILE];
  __shared__ float s_n[3][TILE];
  __shared__ int s_valid[3][TILE];
  __shared__ __align__(16) uint16_t rh[2][TILE][XS];
  __shared__ __align__(16) uint16_t rl[2][TILE][XS];
  __shared__ float s_r2[2][4][TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool rot = wave < 4;
  const int wq = wave & 3;                     // slice of Pi (rotation) or of S (sketch)
  const int c32 = lane & 31, hl = lane >> 5;
  const int b = a.bits, L = 1 << b;
  const bool need_c = a.nc != 0;
  const float G = a.G;
  const int cmax = a.ncell - 1;
  for (int i = tid; i < kQ128Cells; i += 512) s_tab[i] = a.qtab[i < cmax ? i : cmax];
  for (int i = tid; i < L; i += 512) s_cent[i] = a.cent[i];

  // rotation waves: op[8 p + s] = part p (hi, lo, lo2) of Pi at k-step s;
  // sketch waves: op[8 p + s] = part p (hi, lo) of S
  bf16x8 op[24];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      if (p == 2 && !rot) break;
      const uint4* src = rot ? a.rop : a.sop;
      op[8 * p + s] = __builtin_bit_cast(bf16x8, src[((wq * 8 + s) * 3 + p) * 64 + lane]);
    }
  }
  const bool vec_ok = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;
  const bool row16 = (a.idx_pitch & 15) == 0;
  const int r8 = (tid & 255) >> 3, c0 = 16 * (tid & 7);

  auto where = [&](int tile, int& seq, int64_t& blk) {
    seq = tile / a.tiles_per_seq;
    blk = a.first_block + (tile - seq * a.tiles_per_seq);
  };
  auto row0 = [&](int tile) {                  // code row of the tile's row 0
    int seq;
    int64_t blk, oseq, oblk;
    where(tile, seq, blk);
    page_block(a.pm, seq, blk, oseq, oblk);
    return oseq * a.seq_stride + oblk * TILE;
  };
  auto fetch = [&](Share<DT>& sh, int tile) {
    int seq;
    int64_t blk;
    where(tile < a.n_tiles ? tile : a.n_tiles - 1, seq, blk);
    int64_t p = blk * TILE + r8;
    p = p < a.tok_off ? a.tok_off : (p >= a.tok_off + a.n_tok ? a.tok_off + a.n_tok - 1 : p);
    share_load<DT>(sh, a.x, ((int64_t)seq * a.n_tok + (p - a.tok_off)) * 128 + c0, vec_ok);
  };

  const int G1 = (int)gridDim.x, G2 = 2 * G1;
  // pass `it`: the rotation waves take `tile` (if < n_tiles) into buffers
  // q = it % 2 and n3 = it % 3, the sketch waves take tile - G1 (if this is
  // not the first pass) from buffers q ^ 1 and (it + 2) % 3
  auto step = [&](Share<DT>& cur, const int tile, const int q, const int it) __attribute__((always_inline)) {
    const bool have = tile < a.n_tiles;
    const bool prev = tile - G1 >= (int)blockIdx.x;
    const int n3 = it % 3, p3 = (it + 2) % 3;
    // (a) stage this thread's share; |x| in fp32, reduced over the row's 8 threads
    if (rot && have) {
      int seq;
      int64_t blk;
      where(tile, seq, blk);
      const int64_t abs0 = blk * TILE;
      if (!(abs0 >= a.tok_off && abs0 + TILE <= a.tok_off + a.n_tok))
        share_mask<DT>(cur, abs0 + r8 >= a.tok_off && abs0 + r8 < a.tok_off + a.n_tok);
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
          *reinterpret_cast<uint4*>(&xh[q][r8][c0 + 8 * c]) = cur.w[c];
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
        *reinterpret_cast<uint4*>(&xh[q][r8][c0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&xh[q][r8][c0 + 8]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        *reinterpret_cast<uint4*>(&xl[q][r8][c0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint4*>(&xl[q][r8][c0 + 8]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
        if constexpr (XLO2) {
          *reinterpret_cast<uint4*>(&xl2[q][r8][c0]) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
          *reinterpret_cast<uint4*>(&xl2[q][r8][c0 + 8]) = make_uint4(mw[4], mw[5], mw[6], mw[7]);
        }
      }
      s2 = sum8(s2);
      if ((tid & 7) == 0) {
        const int64_t p = abs0 + r8;
        const float n = norm_from_sq(s2);
        s_n[n3][r8] = n;
        s_ig[q][r8] = n > 0.f ? G * __builtin_amdgcn_rcpf(n) : 0.f;
        s_valid[n3][r8] = (p >= a.tok_off && p < a.tok_off + a.n_tok) ? 1 : 0;
      }
    }
    __syncthreads();

    // the share of the tile after next goes in flight while this one is
    // computed, on every pass and in all waves, so that every path into a
    // staging waits alike and no share register is copied while its load is
    // in flight (the sketch waves' loads repeat the rotation waves'
    // addresses and hit the cache)
    fetch(cur, tile + G2);
    int iv[16];
    f32x16 acc = {};
    if (rot && have) {
      // (b) rotation: D[coordinate][vector], coordinates 32 wq .. 32 wq + 31;
      // the hi.hi products and the smaller ones go to two accumulators so
      // the two chains interleave
      f32x16 acs = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 xo = *reinterpret_cast<const bf16x8*>(&xh[q][c32][16 * s + 8 * hl]);
        if constexpr (XLO) {
          const bf16x8 xq = *reinterpret_cast<const bf16x8*>(&xl[q][c32][16 * s + 8 * hl]);
          if constexpr (XLO2) {
            const bf16x8 xr = *reinterpret_cast<const bf16x8*>(&xl2[q][c32][16 * s + 8 * hl]);
            acs = mfma32(op[s], xr, acs);
          }
          acs = mfma32(op[8 + s], xq, acs);
          acs = mfma32(op[s], xq, acs);
        }
        acs = mfma32(op[16 + s], xo, acs);
        acs = mfma32(op[8 + s], xo, acs);
        acc = mfma32(op[s], xo, acc);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] += acs[v];
      // (c) indices: element v is coordinate 32 wq + 8(v/4) + 4hl + v%4 of vector c32
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float key = fmaf(acc[v], s_ig[q][c32], G);
        const int c = (int)key;
        const int2 e = s_tab[c];
        iv[v] = e.x + (key >= __int_as_float(e.y) ? 1 : 0);
      }
      if (need_c) {
        float c2 = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float cv = s_cent[iv[v]];
          c2 = fmaf(cv, cv, c2);
        }
        c2 += __shfl_xor(c2, 32);
        if (hl == 0) s_c2[wq][c32] = c2;
      }
    } else if (!rot && prev) {
      // (h) u = S r of the tile before: sketch rows 32 wq .. 32 wq + 31 of
      // its 32 vectors, their sign bits as word wq of each sign row, and
      // rnorm = |x| |r| (sketch wave 0)
      const int pq = q ^ 1;
      f32x16 au = {}, aus = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 xrh = *reinterpret_cast<const bf16x8*>(&rh[pq][c32][16 * s + 8 * hl]);
        const bf16x8 xrl = *reinterpret_cast<const bf16x8*>(&rl[pq][c32][16 * s + 8 * hl]);
        aus = mfma32(op[s], xrl, aus);
        aus = mfma32(op[8 + s], xrh, aus);
        au = mfma32(op[s], xrh, au);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) au[v] += aus[v];
      uint32_t bits = 0u;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        bits |= (au[v] >= 0.f ? 1u : 0u) << (8 * (v >> 2) + 4 * hl + (v & 3));
      bits |= (uint32_t)__shfl_xor((int)bits, 32);
      const int rows = a.m - 32 * wq;          // sketch rows of this word
      if (rows < 32) bits &= rows > 0 ? (1u << rows) - 1u : 0u;
      const bool qvalid = s_valid[p3][c32] != 0;
      const int64_t pos0 = row0(tile - G1);
      if (hl == 0 && qvalid && rows > 0) a.sign[(((pos0 + c32) * a.sign_pitch) >> 2) + wq] = bits;
      if (wq == 0 && hl == 0 && qvalid)
        a.rnorm[pos0 + c32] =
            s_n[p3][c32] * sqrtf(((s_r2[pq][0][c32] + s_r2[pq][1][c32]) + s_r2[pq][2][c32]) + s_r2[pq][3][c32]);
    }
    if (need_c) __syncthreads();

    if (rot && have) {
      const int64_t pos0 = row0(tile);
      // (d) pack and store the indices: this wave's 32 coordinates are b
      // words [wq b, wq b + b) of the row; group g of 4 coordinates (4b bits)
      // lives in half g % 2, slot g / 2
      uint32_t gv[4], go[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        uint32_t g = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) g |= (uint32_t)iv[4 * qq + r] << (r * b);
        gv[qq] = g;
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) go[qq] = (uint32_t)__shfl_xor((int)gv[qq], 32);
      const bool valid = s_valid[n3][c32] != 0;
      if (hl == 0 && valid) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx + (pos0 + c32) * a.idx_pitch) + wq * b;
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
      // (e) scale |x| (or |x| / |y^|) and (g) the residual
      // r = y - (scale / |x|) c[idx] of this lane's 16 coordinates
      const float qn = s_n[n3][c32];
      float ratio = 1.f;                       // scale / |x|
      if (need_c) {
        const float nh = sqrtf(((s_c2[0][c32] + s_c2[1][c32]) + s_c2[2][c32]) + s_c2[3][c32]);
        ratio = 1.f / nh;
        if (wq == 0 && hl == 0 && valid) a.scale[pos0 + c32] = qn / nh;
      } else if (wq == 0 && hl == 0 && valid) {
        a.scale[pos0 + c32] = qn;
      }
      const float inv_n = qn > 0.f ? 1.f / qn : 0.f;
      float r2 = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 hl2[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int v = 4 * g + 2 * h2;
          const float r0 = fmaf(acc[v], inv_n, -ratio * s_cent[iv[v]]);
          const float r1 = fmaf(acc[v + 1], inv_n, -ratio * s_cent[iv[v + 1]]);
          r2 = fmaf(r0, r0, r2);
          r2 = fmaf(r1, r1, r2);
          hl2[h2] = split_pair(r0, r1);
        }
        const int col = 32 * wq + 8 * g + 4 * hl;
        *reinterpret_cast<uint2*>(&rh[q][c32][col]) = make_uint2(hl2[0].x, hl2[1].x);
        *reinterpret_cast<uint2*>(&rl[q][c32][col]) = make_uint2(hl2[0].y, hl2[1].y);
      }
      r2 += __shfl_xor(r2, 32);
      if (hl == 0) s_r2[q][wq][c32] = r2;
    }
    // no barrier here: what the next pass writes before its barrier (the
    // other staging buffers, the next norm slot) is not read by this pass
  };

  Share<DT> s0, s1;
  int tile = blockIdx.x;
  wait_loads();
  fetch(s0, tile);
  fetch(s1, tile + G1);
  __syncthreads();
  for (int it = 0;; it += 2) {
    step(s0, tile, 0, it);
    if (tile >= a.n_tiles) break;
    tile += G1;
    step(s1, tile, 1, it + 1);
    if (tile >= a.n_tiles) break;
    tile += G1;
  }
}

template <void (*K)(Q128Args)>
int resident_grid(int threads, int n_tiles) {
  // workgroups of kernel K that stay resident at once (per device, computed once)
  static int per_device[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (per_device[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, threads, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 2;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    per_device[dev] = per_cu * cus;
  }
  return n_tiles < per_device[dev] ? n_tiles : per_device[dev];
}

template <int DT, bool T32, int NP>
void launch_np(const Q128Args& a, hipStream_t st) {
  hipLaunchKernelGGL((k_q128<DT, T32, NP>), dim3(resident_grid<k_q128<DT, T32, NP>>(256, a.n_tiles)), dim3(256), 0,
                     st, a);
}

template <int DT>
hipError_t launch_dt(const Q128Args& a, bool t32, hipStream_t st) {
  const bool two = a.bits <= 4;      // two parts of Pi suffice up to 4 bits
  if (a.m > 0) {
    // keys with a sketch: three parts of Pi (fp32-level y, so that |r| keeps
    // its relative accuracy), row layout, rotation and sketch waves
    hipLaunchKernelGGL((k_q128sk<DT>), dim3(resident_grid<k_q128sk<DT>>(512, a.n_tiles)), dim3(512), 0, st, a);
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
