// Vectors back from their codes (gfx950).
//
// Page "6倍KV缓存压缩零精度损失：谷歌TurboQuant技术如何提升智能体运行效率",
// 三、工程实现 item 1 (a compress / decompress pair), with the arithmetic of page
// "什么是TurboQuant？…" 工作原理 > 第一阶段 items 1-2 and 第二阶段：QJL 残差校正
// written out in the original domain:
//   x_hat = Pi^T (scale c[idx]) + rnorm Pi^T sqrt(pi/2)/m S^T (2 sign - 1).
//
// d = 128, qjl_m <= 128 (k_dq128).  A workgroup of four waves owns a tile of
// 32 positions of one sequence (tile32-aligned in absolute position) and
// loops over tiles.  Wave w forms output coordinates 32w .. 32w + 31 of the
// tile's vectors as D[coordinate][vector] with v_mfma_f32_32x32x16_bf16:
//   A  = rows 32w.. of Pi^T in bf16 hi + lo (registers, loaded once),
//   B  = c[idx] of the 32 vectors in bf16 hi + lo (pair-table lookups),
//   hi.hi + hi.lo + lo.hi per k-step (the dropped lo.lo is ~2^-18);
//   A' = rows 32w.. of sqrt(pi/2)/m (S Pi)^T in hi + lo, column j pre-scaled
//        by 2^(127 - 2^(j % 8)),
//   B' = the sign bits left where they lie as bf16 {0, 2^(2^e - 127)}, e = j % 8,
//   so every product is exact in the scaling and, with the column sums cs,
//   sum_j A'[k][j] (2 sign_j - 1) = 2 (A' B')[k] - cs[k].
// The waves share no data (each reads the tile's codes itself), so the loop
// has no barrier.
//
// Other shapes (k_dq_generic): one workgroup per 8 vectors; the weighted
// centroids scale c[idx] and the signs 2 sign - 1 go to LDS, and thread k
// forms coordinate k of the 8 outputs in fp32 from Pi (row-major, read down
// column k) and sqrt(pi/2)/m S Pi (row-major).
#include <algorithm>

#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int TILE = 32;

struct DQArgs {
  const uint8_t* idx;
  const uint32_t* sign;
  const float* scale;
  const float* rnorm;
  int64_t idx_pitch, sign_pitch, seq_stride;
  int64_t n_tok, tok_off, first_block;
  int tiles_per_seq, n_tiles;
  int d, dp, m, mp, bits, sw;    // sw: sign words of a row that carry bits (ceil(m / 32))
  const uint4* dqop;             // Pi^T operands [4][8][3][64]
  const uint4* dqs;              // scaled (S Pi)^T operands [4][8][3][64]
  const float* dqcs;             // column sums [128]
  const uint32_t* tab;           // pair table (bits <= 4) or single-code table
  const float* cent;             // [L] (generic kernel)
  const float* rot;              // [dp][dp] Pi row-major (generic kernel)
  const float* sprot;            // [mp][dp] sqrt(pi/2)/m S Pi row-major (generic kernel)
  void* out;
  int odt;
  int layout;
};

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline uint32_t rne16(float v, int odt) {
  if (odt == TQ_BF16) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
  }
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

// bits [bit, bit + n) of a little-endian word array held in registers
// (n <= 32, bit and the array length compile-time)
template <int NW>
__device__ inline uint32_t reg_bits(const uint32_t (&w)[NW], int bit, int n) {
  const int i = bit >> 5, s = bit & 31;
  uint32_t v = w[i] >> s;
  if (s + n > 32 && i + 1 < NW) v = __builtin_amdgcn_alignbit(w[i + 1], w[i], s);
  return n >= 32 ? v : (v & ((1u << n) - 1u));
}

template <int B, bool T32, bool QJL>
__global__ void __launch_bounds__(256) k_dq128(DQArgs a) {
  constexpr bool PAIR = B <= 4;
  constexpr int NWD = 4 * B;                  // idx words of a row (d = 128)
  constexpr int BLKW = 128 * B;               // words of a tile32 block (d = 128)
  __shared__ __align__(8) uint32_t s_tab[PAIR ? (2 << (2 * B)) : (1 << B)];
  __shared__ uint32_t s_blk[T32 ? 4 : 1][T32 ? BLKW : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, hl = lane >> 5;
  constexpr int TABW = PAIR ? (2 << (2 * B)) : (1 << B);
  for (int i = tid; i < TABW; i += 256) s_tab[i] = a.tab[i];

  bf16x8 ph[8], pl[8], qh[QJL ? 8 : 1], ql[QJL ? 8 : 1];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    ph[s] = __builtin_bit_cast(bf16x8, a.dqop[((wave * 8 + s) * 3 + 0) * 64 + lane]);
    pl[s] = __builtin_bit_cast(bf16x8, a.dqop[((wave * 8 + s) * 3 + 1) * 64 + lane]);
    if constexpr (QJL) {
      qh[s] = __builtin_bit_cast(bf16x8, a.dqs[((wave * 8 + s) * 3 + 0) * 64 + lane]);
      ql[s] = __builtin_bit_cast(bf16x8, a.dqs[((wave * 8 + s) * 3 + 1) * 64 + lane]);
    }
  }
  // element v of the lane's accumulator: coordinate 32w + 8(v/4) + 4hl + v%4
  float cs[QJL ? 16 : 1];
  if constexpr (QJL) {
#pragma unroll
    for (int v = 0; v < 16; ++v) cs[v] = a.dqcs[32 * wave + 8 * (v >> 2) + 4 * hl + (v & 3)];
  }
  __syncthreads();

  // Loads of one tile for this lane: its vector's code row (row layout) or
  // its share of the tile32 block, scale, rnorm and sign words.  The next
  // tile's loads are issued before the current tile is computed; past the
  // last tile they repeat it, so every pass issues the same loads.
  struct Ld {
    uint32_t w[T32 ? BLKW / 64 : NWD];
    uint32_t sg[QJL ? 4 : 1];
    float sc, rn;
  };
  auto load = [&](Ld& L, int tile) __attribute__((always_inline)) {
    tile = tile < a.n_tiles ? tile : a.n_tiles - 1;
    const int seq = tile / a.tiles_per_seq;
    const int64_t blk = a.first_block + (tile - (int64_t)seq * a.tiles_per_seq);
    const int64_t p = blk * TILE + c32;
    const int64_t pc = p < a.tok_off ? a.tok_off : (p >= a.tok_off + a.n_tok ? a.tok_off + a.n_tok - 1 : p);
    const int64_t row = (int64_t)seq * a.seq_stride + pc;
    L.sc = a.scale[row];
    L.rn = 0.f;
    if constexpr (QJL) {
      L.rn = a.rnorm[row];
      const uint32_t* sr = a.sign + ((row * a.sign_pitch) >> 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) L.sg[i] = sr[i < a.sw ? i : 0];
    }
    if constexpr (!T32) {
      const uint32_t* ir = reinterpret_cast<const uint32_t*>(a.idx + row * a.idx_pitch);
#pragma unroll
      for (int i = 0; i < NWD; ++i) L.w[i] = ir[i];
    } else {
      const uint32_t* bsrc = reinterpret_cast<const uint32_t*>(a.idx) +
                             ((int64_t)seq * (a.seq_stride / TILE) + blk) * (int64_t)BLKW;
#pragma unroll
      for (int i = 0; i < BLKW / 64; ++i) L.w[i] = bsrc[lane + 64 * i];
    }
  };
  Ld cur, nxt;
  load(cur, blockIdx.x);

  for (int tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    load(nxt, tile + (int)gridDim.x);
    const int seq = tile / a.tiles_per_seq;
    const int64_t blk = a.first_block + (tile - (int64_t)seq * a.tiles_per_seq);
    const int64_t p = blk * TILE + c32;
    const bool valid = p >= a.tok_off && p < a.tok_off + a.n_tok;
    const float sc = cur.sc, rn = cur.rn;
    uint32_t sg[4] = {0u, 0u, 0u, 0u};
    if constexpr (QJL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sg[i] = i < a.sw ? cur.sg[i] : 0u;
    }
    uint32_t w[T32 ? 1 : NWD];
    if constexpr (!T32) {
#pragma unroll
      for (int i = 0; i < NWD; ++i) w[i] = cur.w[i];
    } else {
      // the tile's block into this wave's LDS slot; the gathers below are
      // reads of the same wave after its own writes (LDS order within a wave)
#pragma unroll
      for (int i = 0; i < BLKW / 64; ++i) s_blk[wave][lane + 64 * i] = cur.w[i];
    }
    // tile32 slot of this lane's token within the block
    const int tt = c32, G = (tt & 15) >> 2, e = (tt & 3) + 4 * (tt >> 4);

    // two accumulator chains (even / odd k-steps) so that consecutive MFMAs
    // do not wait on each other's results
    f32x16 acc = {}, acc2 = {}, accq = {}, accq2 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // codes of coordinates 16s + 8hl + c, c = 0..7: pair q = (2q, 2q + 1)
      uint32_t bh[4], bl[4];
      if constexpr (!T32 && PAIR) {
        // the 8 codes are one 8B-bit field of the row (<= 32 bits); the pair
        // index of codes 2q, 2q + 1 is its bits [2Bq, 2Bq + 2B)
        const uint32_t f0 = reg_bits<NWD>(w, (16 * s) * B, 8 * B), f1 = reg_bits<NWD>(w, (16 * s + 8) * B, 8 * B);
        const uint32_t f = hl ? f1 : f0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t pe = (f >> (2 * B * q)) & ((1u << (2 * B)) - 1u);
          const uint2 t = *reinterpret_cast<const uint2*>(&s_tab[2 * pe]);
          bh[q] = t.x;
          bl[q] = t.y;
        }
      } else {
        uint32_t code[8];
        if constexpr (!T32) {
          // 8B bits (> 32): the low and high halves of the field, then codes
          const uint32_t l0 = reg_bits<NWD>(w, (16 * s) * B, 32), l1 = reg_bits<NWD>(w, (16 * s + 8) * B, 32);
          const uint32_t h0 = reg_bits<NWD>(w, (16 * s) * B + 32, 8 * B - 32);
          const uint32_t h1 = reg_bits<NWD>(w, (16 * s + 8) * B + 32, 8 * B - 32);
          const uint64_t f = hl ? ((uint64_t)h1 << 32 | l1) : ((uint64_t)h0 << 32 | l0);
#pragma unroll
          for (int c = 0; c < 8; ++c) code[c] = (uint32_t)(f >> (B * c)) & ((1u << B) - 1u);
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int r = 16 * G + 8 * hl + c;
            const int bit = ((r * 8 + s) * 8 + e) * B;
            const int wi = bit >> 5, sh = bit & 31;
            uint32_t v = s_blk[wave][wi] >> sh;
            if constexpr (32 % B != 0) {
              if (sh + B > 32) v = __builtin_amdgcn_alignbit(s_blk[wave][wi + 1], s_blk[wave][wi], sh);
            }
            code[c] = v & ((1u << B) - 1u);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (PAIR) {
            const uint32_t pe = code[2 * q] | (code[2 * q + 1] << B);
            const uint2 t = *reinterpret_cast<const uint2*>(&s_tab[2 * pe]);
            bh[q] = t.x;
            bl[q] = t.y;
          } else {
            const uint32_t t0 = s_tab[code[2 * q]], t1 = s_tab[code[2 * q + 1]];
            bh[q] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
            bl[q] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
          }
        }
      }
      const bf16x8 Bh = __builtin_bit_cast(bf16x8, (u32x4){bh[0], bh[1], bh[2], bh[3]});
      const bf16x8 Bl = __builtin_bit_cast(bf16x8, (u32x4){bl[0], bl[1], bl[2], bl[3]});
      f32x16& ac = (s & 1) ? acc2 : acc;
      ac = mfma32(ph[s], Bh, ac);
      ac = mfma32(ph[s], Bl, ac);
      ac = mfma32(pl[s], Bh, ac);
      if constexpr (QJL) {
        // sketch rows 16s + 8hl + e' (e' = 0..7): byte 2s + hl of the sign row
        const uint32_t sb = (sg[s >> 1] >> (8 * (2 * (s & 1) + hl))) & 0xFFu;
        const uint32_t x7 = (sb | (sb << 16)) << 7;
        const bf16x8 Bq = __builtin_bit_cast(
            bf16x8, (u32x4){x7 & 0x01000080u, x7 & 0x04000200u, x7 & 0x10000800u, x7 & 0x40002000u});
        f32x16& aq = (s & 1) ? accq2 : accq;
        aq = mfma32(qh[s], Bq, aq);
        aq = mfma32(ql[s], Bq, aq);
      }
    }

    if (valid) {
      const int64_t orow = (int64_t)seq * a.n_tok + (p - a.tok_off);
      float x[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[v] = sc * (acc[v] + acc2[v]);
        if constexpr (QJL) x[v] = fmaf(rn, 2.f * (accq[v] + accq2[v]) - cs[v], x[v]);
      }
      // element 4g + r: coordinate 32w + 8g + 4hl + r
      const int64_t o0 = orow * 128 + 32 * wave + 4 * hl;
      if (a.odt == TQ_F32) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o0 + 8 * g) =
              make_float4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]);
      } else if (a.odt == TQ_BF16) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o0 + 8 * g) =
              make_uint2(rne16(x[4 * g], TQ_BF16) | (rne16(x[4 * g + 1], TQ_BF16) << 16),
                         rne16(x[4 * g + 2], TQ_BF16) | (rne16(x[4 * g + 3], TQ_BF16) << 16));
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o0 + 8 * g) =
              make_uint2(rne16(x[4 * g], TQ_F16) | (rne16(x[4 * g + 1], TQ_F16) << 16),
                         rne16(x[4 * g + 2], TQ_F16) | (rne16(x[4 * g + 3], TQ_F16) << 16));
      }
    }
    cur = nxt;
  }
}

// ------------------------------------------------------------ any shape

constexpr int GV = 8;   // vectors per workgroup pass

__global__ void __launch_bounds__(256) k_dq_generic(DQArgs a) {
  __shared__ float s_w[GV][256];
  __shared__ float s_pm[GV][256];
  __shared__ float s_rn[GV];
  const int tid = threadIdx.x;
  const int64_t nvec = a.n_tok * (int64_t)(a.n_tiles);   // n_tiles holds n_seq here
  const int B = a.bits, ndb = (a.d + 15) / 16;
  const int64_t groups = (nvec + GV - 1) / GV;
  for (int64_t gi = blockIdx.x; gi < groups; gi += gridDim.x) {
    // weighted centroids, signs and residual norms of the group's vectors
    for (int e = tid; e < GV * a.dp; e += 256) {
      const int v = e / a.dp, i = e - v * a.dp;
      const int64_t gv = gi * GV + v;
      float wv = 0.f;
      if (gv < nvec && i < a.d) {
        const int64_t seq = gv / a.n_tok, t = gv - seq * a.n_tok;
        const int64_t pos = a.tok_off + t, row = seq * a.seq_stride + pos;
        int64_t bit;
        const uint8_t* base;
        if (a.layout == TQ_LAYOUT_ROW) {
          base = a.idx + row * a.idx_pitch;
          bit = (int64_t)i * B;
        } else {
          const int64_t blk = pos / TILE;
          const int tt = (int)(pos & 31);
          const int G = (tt & 15) >> 2, es = (tt & 3) + 4 * (tt >> 4);
          const int r = 16 * G + (i & 15), j = i >> 4;
          base = a.idx + (seq * (a.seq_stride / TILE) + blk) * (int64_t)(64 * 8 * ndb * B / 8);
          bit = ((int64_t)(r * ndb + j) * 8 + es) * B;
        }
        const uint32_t lo = base[bit >> 3], hi = (bit & 7) + B > 8 ? base[(bit >> 3) + 1] : 0u;
        const uint32_t code = ((lo | (hi << 8)) >> (bit & 7)) & ((1u << B) - 1u);
        wv = a.scale[row] * a.cent[code];
      }
      s_w[v][i] = wv;
    }
    if (a.m > 0) {
      for (int e = tid; e < GV * a.mp; e += 256) {
        const int v = e / a.mp, j = e - v * a.mp;
        const int64_t gv = gi * GV + v;
        float pm = 0.f;
        if (gv < nvec && j < a.m) {
          const int64_t seq = gv / a.n_tok, t = gv - seq * a.n_tok;
          const int64_t row = seq * a.seq_stride + a.tok_off + t;
          const uint32_t wd = a.sign[((row * a.sign_pitch) >> 2) + (j >> 5)];
          pm = ((wd >> (j & 31)) & 1u) ? 1.f : -1.f;
        }
        s_pm[v][j] = pm;
      }
      if (tid < GV) {
        const int64_t gv = gi * GV + tid;
        float rn = 0.f;
        if (gv < nvec) {
          const int64_t seq = gv / a.n_tok, t = gv - seq * a.n_tok;
          rn = a.rnorm[seq * a.seq_stride + a.tok_off + t];
        }
        s_rn[tid] = rn;
      }
    }
    __syncthreads();
    const int k = tid;
    if (k < a.d) {
      float x[GV];
#pragma unroll
      for (int v = 0; v < GV; ++v) x[v] = 0.f;
      for (int i = 0; i < a.d; ++i) {
        const float r = a.rot[(int64_t)i * a.dp + k];
#pragma unroll
        for (int v = 0; v < GV; ++v) x[v] = fmaf(r, s_w[v][i], x[v]);
      }
      if (a.m > 0) {
        float z[GV];
#pragma unroll
        for (int v = 0; v < GV; ++v) z[v] = 0.f;
        for (int j = 0; j < a.m; ++j) {
          const float r = a.sprot[(int64_t)j * a.dp + k];
#pragma unroll
          for (int v = 0; v < GV; ++v) z[v] = fmaf(r, s_pm[v][j], z[v]);
        }
#pragma unroll
        for (int v = 0; v < GV; ++v) x[v] = fmaf(s_rn[v], z[v], x[v]);
      }
#pragma unroll
      for (int v = 0; v < GV; ++v) {
        const int64_t gv = gi * GV + v;
        if (gv >= nvec) break;
        const int64_t o = gv * a.d + k;
        if (a.odt == TQ_F32) static_cast<float*>(a.out)[o] = x[v];
        else static_cast<uint16_t*>(a.out)[o] = (uint16_t)rne16(x[v], a.odt);
      }
    }
    __syncthreads();
  }
}

// workgroups of a k_dq128 instantiation that stay resident per CU (cached)
template <int B, bool T32, bool QJL>
int resident_one() {
  static int per_device[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (per_device[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_dq128<B, T32, QJL>, 256, 0) != hipSuccess || n < 1) n = 1;
    per_device[dev] = n;
  }
  return per_device[dev];
}

template <int B>
int resident_b(bool t32, bool qjl) {
  if (t32) return qjl ? resident_one<B, true, true>() : resident_one<B, true, false>();
  return qjl ? resident_one<B, false, true>() : resident_one<B, false, false>();
}

int resident_per_cu(int bits, bool t32, bool qjl) {
  switch (bits) {
    case 1: return resident_b<1>(t32, qjl);
    case 2: return resident_b<2>(t32, qjl);
    case 3: return resident_b<3>(t32, qjl);
    case 4: return resident_b<4>(t32, qjl);
    case 5: return resident_b<5>(t32, qjl);
    case 6: return resident_b<6>(t32, qjl);
    case 7: return resident_b<7>(t32, qjl);
    default: return resident_b<8>(t32, qjl);
  }
}

template <int B, bool T32>
void launch_b_t(const DQArgs& a, bool qjl, int grid, hipStream_t st) {
  if (qjl) hipLaunchKernelGGL((k_dq128<B, T32, true>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_dq128<B, T32, false>), dim3(grid), dim3(256), 0, st, a);
}

template <int B>
void launch_b(const DQArgs& a, bool t32, bool qjl, int grid, hipStream_t st) {
  if (t32) launch_b_t<B, true>(a, qjl, grid, st);
  else launch_b_t<B, false>(a, qjl, grid, st);
}

int device_cus() {
  static int per_device[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (per_device[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    per_device[dev] = cus;
  }
  return per_device[dev];
}

}  // namespace

bool dequantize128_supported(const tq_codebook* cb) {
  return cb->p.d == 128 && cb->p.qjl_m <= 128 && cb->dev.dqop &&
         (cb->p.qjl_m == 0 || (cb->dev.dqs && cb->dev.dqcs));
}

hipError_t launch_dequantize(const tq_codebook* cb, const DequantJob& job, hipStream_t stream) {
  DQArgs a{};
  const tq_codes& c = job.codes;
  a.idx = static_cast<const uint8_t*>(c.idx);
  a.sign = static_cast<const uint32_t*>(c.sign);
  a.scale = c.scale;
  a.rnorm = c.rnorm;
  a.idx_pitch = c.idx_row_bytes;
  a.sign_pitch = c.sign_row_bytes;
  a.seq_stride = c.seq_stride;
  a.n_tok = job.n_tok;
  a.tok_off = job.tok_offset;
  a.d = cb->p.d; a.dp = cb->dp; a.m = cb->p.qjl_m; a.mp = cb->mp; a.bits = cb->p.bits;
  a.sw = (cb->p.qjl_m + 31) / 32;
  a.dqop = reinterpret_cast<const uint4*>(cb->dev.dqop);
  a.dqs = reinterpret_cast<const uint4*>(cb->dev.dqs);
  a.dqcs = cb->dev.dqcs;
  a.tab = cb->dev.pair_tab;
  a.cent = cb->dev.cent;
  a.rot = cb->dev.rot;
  a.sprot = cb->dev.sprot;
  a.out = job.out;
  a.odt = job.dt;
  a.layout = c.layout;
  ProfileScope prof(TQ_KERNEL_DEQUANTIZE, stream);
  if (dequantize128_supported(cb)) {
    a.first_block = job.tok_offset / TILE;
    const int64_t last_block = (job.tok_offset + job.n_tok - 1) / TILE;
    a.tiles_per_seq = (int)(last_block - a.first_block + 1);
    a.n_tiles = (int)(a.tiles_per_seq * job.n_seq);
    const bool t32 = c.layout == TQ_LAYOUT_TILE32, qjl = cb->p.qjl_m > 0;
    const int grid = (int)std::min<int64_t>(a.n_tiles, (int64_t)resident_per_cu(cb->p.bits, t32, qjl) * device_cus());
    switch (cb->p.bits) {
      case 1: launch_b<1>(a, t32, qjl, grid, stream); break;
      case 2: launch_b<2>(a, t32, qjl, grid, stream); break;
      case 3: launch_b<3>(a, t32, qjl, grid, stream); break;
      case 4: launch_b<4>(a, t32, qjl, grid, stream); break;
      case 5: launch_b<5>(a, t32, qjl, grid, stream); break;
      case 6: launch_b<6>(a, t32, qjl, grid, stream); break;
      case 7: launch_b<7>(a, t32, qjl, grid, stream); break;
      default: launch_b<8>(a, t32, qjl, grid, stream); break;
    }
  } else {
    a.n_tiles = (int)job.n_seq;       // the generic kernel takes n_seq here
    const int64_t groups = (job.n_seq * job.n_tok + GV - 1) / GV;
    const int grid = (int)std::min<int64_t>(groups, 8LL * device_cus());
    hipLaunchKernelGGL(k_dq_generic, dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tq
