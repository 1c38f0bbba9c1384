// Query prologue of the d = 128 decode attention (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog), "如何实现 TurboQuant" item 1:
// the query is rotated once; "第二阶段" supplies the sketch of the rotated
// query that the QJL correction needs.
//
// Workgroup (part, row), part 0..3: coordinates 32 part .. 32 part + 31 of
// q~ = Pi_K q' and rows 32 part .. + 31 of t = sqrt(pi/2)/m (S_K Pi_K) q' for
// the row's 8 query slots (q' = sm_scale log2(e) q), written as bf16 hi / lo
// B operands of the split kernel's MFMAs.  Only the part's 32 columns of the
// two matrices are staged (32 KB, one batch of coalesced 16-byte loads).
// The body serves its own 256-thread launch (k_prologue) and rides along in
// the append launch of a fused decode step (k_quantize_small, 512 threads):
// threads with active == false only take part in the barriers.
#pragma once

#include "tq_internal.hpp"

namespace tq {
namespace prologue {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int D = 128;                 // head dimension of this kernel family
constexpr int QOP_Q = 8 * 64 * 4;      // Q operand dwords: 8 MFMAs x 64 lanes x 4
constexpr int QOP_T = 4 * 64 * 4;      // T operand dwords
constexpr int QOP_DWORDS = QOP_Q + QOP_T + 64;   // + QJL offsets [4 parts][16 columns]
constexpr int kSignShift = 64;    // the sketch-query operand carries 2^-kSignShift

__device__ inline uint32_t bf16_rne_bits(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline void run(const PArgs& a, const int part, const int row, const bool active) {
  __shared__ __align__(16) float mat[D][32];
  __shared__ __align__(16) float mat2[D][32];
  __shared__ __align__(16) float qs[8][D];
  __shared__ float qt[8][32];
  __shared__ float tt[8][32];
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;          // b * Hkv + h
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int tid = threadIdx.x;
  const bool sk = a.m > 0 && 32 * part < a.mp;
  // all matrix loads first (one round trip), then the query elements:
  // 16-byte chunk c = tid + 256 j is row c / 8, columns 32 part + 4 (c % 8)
  if (active) {
  f32x4 r1[4], r2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    const int k = c >> 3, i4 = 32 * part + 4 * (c & 7);
    r1[j] = *reinterpret_cast<const f32x4*>(a.rotKT + (int64_t)k * D + i4);
    r2[j] = sk ? *reinterpret_cast<const f32x4*>(a.sprotKT + (int64_t)k * a.mp + i4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + 256 * j;
    const int slot = e >> 7, i = e & (D - 1);
    const bool live = qg * 8 + slot < a.g;
    const int64_t off = ((int64_t)b * a.Hq + h * a.g + qg * 8 + (live ? slot : 0)) * D + i;
    float v;
    if (a.qdt == TQ_F32) v = static_cast<const float*>(a.q)[off];
    else if (a.qdt == TQ_BF16) v = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.q)[off] << 16);
    else v = (float)static_cast<const _Float16*>(a.q)[off];
    qs[slot][i] = live ? v * a.qscale : 0.f;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    *reinterpret_cast<f32x4*>(&mat[c >> 3][4 * (c & 7)]) = r1[j];
    *reinterpret_cast<f32x4*>(&mat2[c >> 3][4 * (c & 7)]) = r2[j];
  }
  }
  __syncthreads();
  if (active) {
    const int i = tid & 31, c = tid >> 5;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll 4
    for (int k = 0; k < D; k += 4) {
      const f32x4 qv = *reinterpret_cast<const f32x4*>(&qs[c][k]);
#pragma unroll
      for (int u = 0; u < 4; ++u) s1 = fmaf(mat[k + u][i], qv[u], s1);
      if (sk) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s2 = fmaf(mat2[k + u][i], qv[u], s2);
      }
    }
    qt[c][i] = s1;
    tt[c][i] = s2;
  }
  __syncthreads();
  if (!active) return;
  uint32_t* dst = a.qop + (int64_t)row * QOP_DWORDS;
  // Q operand [u][lane][p]: MFMA u, lane group g4 covers dims 32*g4 + 4u .. +3;
  // dwords p = 0,1 -> dims (4u, 4u+1) (hi then lo slot of the key operand),
  // p = 2,3 -> dims (4u+2, 4u+3).  Columns 0-7 hold hi, 8-15 lo.  This
  // workgroup writes lane group g4 = part: f -> (u, col, p).
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int f = tid + 256 * r;
    const int p = f & 3, col = (f >> 2) & 15, u = f >> 6;
    const int cl = col & 7, lo = col >> 3;
    const int dim = 4 * u + 2 * (p >> 1);
    uint32_t hv[2];
    for (int h2 = 0; h2 < 2; ++h2) {
      const float v = qt[cl][dim + h2];
      const uint32_t hi = bf16_rne_bits(v);
      hv[h2] = lo ? bf16_rne_bits(v - __uint_as_float(hi << 16)) : hi;
    }
    dst[(u * 64 + 16 * part + col) * 4 + p] = hv[0] | (hv[1] << 16);
  }
  // T operand [cc][lane][p]: dword p of MFMA cc faces sign dword K = 4cc + p
  // of lane group g4, whose low / high halves hold sign bits jl / jh at bf16
  // bit P; the entry is t of sketch row 32*g4 + j times 2^(128 - 2^(P-7)) and
  // 2^-kSignShift (exact power-of-two scalings).
  if (a.m > 0) {
    const int p = tid & 3, col = (tid >> 2) & 15, cc = tid >> 6;
    const int cl = col & 7, lo = col >> 3;
    const int K = 4 * cc + p;
    const int P = (K < 8) ? 14 - K : 22 - K;
    const int ex = 128 - (1 << (P - 7)) - kSignShift;
    uint32_t hv[2];
    for (int h2 = 0; h2 < 2; ++h2) {
      const int j = h2 ? 30 - K : (K == 15 ? 31 : 14 - K);
      const float v = ldexpf(tt[cl][j], ex);
      const uint32_t hi = bf16_rne_bits(v);
      hv[h2] = lo ? bf16_rne_bits(v - __uint_as_float(hi << 16)) : hi;
    }
    dst[QOP_Q + (cc * 64 + 16 * part + col) * 4 + p] = hv[0] | (hv[1] << 16);
  }
  // QJL accumulator offsets, this part's share: -sum over its 32 sketch rows
  // of (hi + lo) of t, in the scale of the sign products (2^-kSignShift), for
  // the hi columns; the lo columns start at 0
  if (tid < 16) {
    float s = 0.f;
    if (tid < 8) {
      for (int j = 0; j < 32; ++j) {
        const float v = tt[tid][j];
        const float fh = __uint_as_float(bf16_rne_bits(v) << 16);
        s += fh + __uint_as_float(bf16_rne_bits(v - fh) << 16);
      }
    }
    reinterpret_cast<float*>(dst)[QOP_Q + QOP_T + 16 * part + tid] = tid < 8 ? -ldexpf(s, -kSignShift) : 0.f;
  }
}

}  // namespace prologue
}  // namespace tq
