// Online quantization for head dimension 128 (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog): "第一阶段" items 1-2 (rotate by
// Pi, normalise, Lloyd-Max index per coordinate) and "如何实现 TurboQuant" item 1
// (quantize on every cache update), for codebooks without a QJL sketch.
//
// One workgroup of four waves owns a tile of 32 consecutive positions of one
// sequence (tile32-aligned in absolute position) and loops over tiles.
//
// Rotation.  Wave w computes coordinates 32w .. 32w + 31 of z = Pi x for the
// 32 vectors with v_mfma_f32_32x32x16_bf16.  Pi is split into three bf16
// parts hi + lo + lo2 kept in registers (8 k-steps x 3 operands); the tile is
// staged in LDS as bf16 parts of x: one for bf16 input (exact), two for fp16
// (exact), three for fp32.  Every product of parts whose orders add up to at
// most 2^-18 is accumulated in fp32 (3, 5 or 6 MFMAs per k-step); the rest is
// below 2^-26 of each product, so y carries fp32-level error only (a two-part
// split leaves 2^-18 and moves 8-bit indices in the 1e-5 boundary zone more
// often than the codes allow).  Keys with a QJL sketch take the fp32-MFMA
// kernel.
// Row layout codes take z^T (rows = coordinates: a lane holds 16 coordinates
// of one vector); tile32 codes take z (rows = vectors: a lane holds one
// coordinate of 16 vectors, which is how a tile32 record is ordered).
//
// Index.  y = z / |x| lies in [-1, 1]; cell floor((y + 1) G) of a uniform grid
// (cells narrower than the closest pair of decision boundaries, built with
// the codebook) holds the number of boundaries below the cell and the one
// inside it, so idx = count + (y >= boundary).  fp32 rounding of the cell can
// only matter when a boundary lies within ~1e-7 of y.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int TILE = 32;
constexpr int XS = 136;   // bf16 row stride of the staged tile (272 bytes: 16-byte lane reads hit distinct banks)

struct Q128Args {
  const void* x;
  int64_t n_tok, tok_off;
  int64_t tiles_per_seq, first_block, n_tiles;
  int bits, nc, ncell;
  float G;
  const uint4* rop;    // Pi operands [4][8][3][64]
  const float* cent;   // [L]
  const int2* qtab;    // [ncell] index cells
  uint8_t* idx;
  float* scale;
  int64_t idx_pitch, seq_stride;
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

// 16 consecutive input elements as fp32 (zeros when !valid)
template <int DT>
__device__ inline void load16(const void* x, int64_t e0, bool valid, bool vec_ok, float (&v)[16]) {
  if (!valid) {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = 0.f;
    return;
  }
  if constexpr (DT == TQ_F32) {
    const float* p = static_cast<const float*>(x) + e0;
    if (vec_ok) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 u = reinterpret_cast<const float4*>(p)[c];
        v[4 * c] = u.x; v[4 * c + 1] = u.y; v[4 * c + 2] = u.z; v[4 * c + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = p[k];
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(x) + e0;
    uint32_t w[8];
    if (vec_ok) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 u = reinterpret_cast<const uint4*>(p)[c];
        w[4 * c] = u.x; w[4 * c + 1] = u.y; w[4 * c + 2] = u.z; w[4 * c + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = (uint32_t)p[2 * k] | ((uint32_t)p[2 * k + 1] << 16);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (DT == TQ_BF16) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      } else {
        v[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xFFFFu));
        v[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
      }
    }
  }
}

__device__ inline int qindex(float y, const int2* tab, float G, int ncell) {
  int c = (int)fmaf(y, G, G);
  c = c < 0 ? 0 : (c > ncell - 1 ? ncell - 1 : c);
  const int2 e = tab[c];
  return e.x + (y >= __int_as_float(e.y) ? 1 : 0);
}

template <int DT, bool T32>
__global__ void __launch_bounds__(256) k_q128(Q128Args a) {
  constexpr bool XLO = DT != TQ_BF16, XLO2 = DT == TQ_F32;
  __shared__ __align__(16) uint16_t xh[TILE][XS];
  __shared__ __align__(16) uint16_t xl[XLO ? TILE : 1][XS];
  __shared__ __align__(16) uint16_t xl2[XLO2 ? TILE : 1][XS];
  __shared__ __align__(16) uint32_t tb[T32 ? 2 : 1][T32 ? 1024 : 1];   // tile32 block values, field masks
  __shared__ int2 s_tab[kQ128Cells];
  __shared__ float s_cent[256];
  __shared__ float s_n[TILE], s_inv[TILE];
  __shared__ float s_c2[4][TILE];
  __shared__ int s_valid[TILE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, hl = lane >> 5;
  const int b = a.bits, L = 1 << b;
  const bool need_c = a.nc != 0;
  for (int i = tid; i < a.ncell; i += 256) s_tab[i] = a.qtab[i];
  for (int i = tid; i < L; i += 256) s_cent[i] = a.cent[i];

  bf16x8 ph[8], pl[8], pm[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    ph[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 0) * 64 + lane]);
    pl[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 1) * 64 + lane]);
    pm[s] = __builtin_bit_cast(bf16x8, a.rop[((wave * 8 + s) * 3 + 2) * 64 + lane]);
  }
  const bool vec_ok = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;
  __syncthreads();

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const int64_t seq = tile / a.tiles_per_seq;
    const int64_t blk = a.first_block + tile % a.tiles_per_seq;
    const int64_t abs0 = blk * TILE;
    const int64_t pos0 = seq * a.seq_stride + abs0;            // code row of tile row 0
    const int64_t src0 = seq * a.n_tok + (abs0 - a.tok_off);  // input row of tile row 0
    const bool full = abs0 >= a.tok_off && abs0 + TILE <= a.tok_off + a.n_tok;

    // (a) stage the tile: thread -> row tid/8, coordinates 16*(tid%8) .. +15;
    // |x| in fp32 from the input values, reduced over the row's 8 threads
    {
      const int r = tid >> 3, c0 = 16 * (tid & 7);
      const int64_t p = abs0 + r;
      const bool valid = p >= a.tok_off && p < a.tok_off + a.n_tok;
      float xv[16];
      load16<DT>(a.x, (src0 + r) * 128 + c0, valid, vec_ok, xv);
      float s2 = 0.f;
      uint32_t hw[8], lw[8], mw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        s2 = fmaf(xv[2 * k], xv[2 * k], s2);
        s2 = fmaf(xv[2 * k + 1], xv[2 * k + 1], s2);
        const uint32_t h0 = bf16_bits(xv[2 * k]), h1 = bf16_bits(xv[2 * k + 1]);
        hw[k] = h0 | (h1 << 16);
        if constexpr (XLO) {
          const float e0 = xv[2 * k] - bf16_float(h0), e1 = xv[2 * k + 1] - bf16_float(h1);
          const uint32_t l0 = bf16_bits(e0), l1 = bf16_bits(e1);
          lw[k] = l0 | (l1 << 16);
          if constexpr (XLO2)
            mw[k] = bf16_bits(e0 - bf16_float(l0)) | (bf16_bits(e1 - bf16_float(l1)) << 16);
        }
      }
      *reinterpret_cast<uint4*>(&xh[r][c0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&xh[r][c0 + 8]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      if constexpr (XLO) {
        *reinterpret_cast<uint4*>(&xl[r][c0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint4*>(&xl[r][c0 + 8]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      }
      if constexpr (XLO2) {
        *reinterpret_cast<uint4*>(&xl2[r][c0]) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
        *reinterpret_cast<uint4*>(&xl2[r][c0 + 8]) = make_uint4(mw[4], mw[5], mw[6], mw[7]);
      }
      s2 += __shfl_xor(s2, 1);
      s2 += __shfl_xor(s2, 2);
      s2 += __shfl_xor(s2, 4);
      if ((tid & 7) == 0) {
        const float n = sqrtf(s2);
        s_n[r] = n;
        s_inv[r] = n > 0.f ? 1.0f / n : 0.f;
        s_valid[r] = valid ? 1 : 0;
      }
    }
    __syncthreads();

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
      acc = prod(acc, xo, pm[s]);
      acc = prod(acc, xo, pl[s]);
      acc = prod(acc, xo, ph[s]);
    }

    // (c) indices; element v of the lane: row layout -> coordinate
    // 32w + 8(v/4) + 4hl + v%4 of vector c32; tile32 -> coordinate 32w + c32
    // of vector 8(v/4) + 4hl + v%4
    float yv[16];
    int iv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int vec = T32 ? 8 * (v >> 2) + 4 * hl + (v & 3) : c32;
      yv[v] = acc[v] * s_inv[vec];
      iv[v] = qindex(yv[v], s_tab, a.G, a.ncell);
    }
    float cv[16];
    if (need_c) {
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
        const int G = hl + 2 * qq;
        uint64_t val = 0, msk = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = 4 * (qq + 2 * (e >> 2)) + (e & 3);
          const int tok = 8 * (v >> 2) + 4 * hl + (v & 3);
          val |= (uint64_t)iv[v] << (e * b);
          if (s_valid[tok]) msk |= fm << (e * b);
        }
        const int grp = (16 * G + C) * 8 + j;
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

    // (e) scale (norm correction: |x| / |y^|)
    if (need_c) __syncthreads();
    if (wave == 0 && hl == 0 && s_valid[c32]) {
      const float n = s_n[c32];
      float sc = n;
      if (a.nc) {
        const float nh = sqrtf(((s_c2[0][c32] + s_c2[1][c32]) + s_c2[2][c32]) + s_c2[3][c32]);
        sc = n / nh;
      }
      a.scale[pos0 + c32] = sc;
    }
    __syncthreads();

    if constexpr (T32) {
      // (f) the assembled tile32 block: 512*b bytes = 128*b words
      const int words = 128 * b;
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx) + (seq * (a.seq_stride / TILE) + blk) * (int64_t)words;
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

template <int DT>
hipError_t launch_dt(const Q128Args& a, bool t32, int grid, hipStream_t st) {
  if (t32) hipLaunchKernelGGL((k_q128<DT, true>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_q128<DT, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool quantize128_supported(const tq_codebook* cb, const QuantJob& job) {
  (void)job;
  return cb->p.d == 128 && cb->p.qjl_m == 0 && cb->dev.rop && cb->dev.qtab && cb->dev.qcells >= 1;
}

hipError_t launch_quantize128(const tq_codebook* cb, const QuantJob& job, hipStream_t stream) {
  Q128Args a{};
  a.x = job.x;
  a.n_tok = job.n_tok;
  a.tok_off = job.tok_offset;
  a.first_block = job.tok_offset / TILE;
  const int64_t last_block = (job.tok_offset + job.n_tok - 1) / TILE;
  a.tiles_per_seq = last_block - a.first_block + 1;
  a.n_tiles = a.tiles_per_seq * job.n_seq;
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
  const int grid = (int)(a.n_tiles < 2048 ? a.n_tiles : 2048);
  const bool t32 = job.out.layout == TQ_LAYOUT_TILE32;
  ProfileScope prof(TQ_KERNEL_QUANTIZE, stream);
  switch (job.dt) {
    case TQ_F32: return launch_dt<TQ_F32>(a, t32, grid, stream);
    case TQ_BF16: return launch_dt<TQ_BF16>(a, t32, grid, stream);
    default: return launch_dt<TQ_F16>(a, t32, grid, stream);
  }
}

}  // namespace tq
