// Online quantization kernel (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog): "第一阶段" items 1-2 (rotate by
// Pi, normalise, Lloyd-Max index per coordinate), "第二阶段：QJL 残差校正"
// (one sign bit per sketch row of the residual), "如何实现 TurboQuant" item 1
// (quantize on every cache update).
//
// One workgroup owns a tile of 32 consecutive vector positions of one
// sequence (tile32-aligned in absolute position) and loops over tiles
// (persistent grid).  Waves 0..dp/32-1 each keep a 32-row slice of Pi in
// registers as the B operand of v_mfma_f32_32x32x2f32 and compute a 32x32
// block of Z = X Pi^T; with QJL, waves dp/32.. keep a 32-row slice of S and
// compute U = R S^T the same way, and each 64-lane ballot of U >= 0 is two
// finished 32-bit sign words.
#include "decode_prologue.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int TILE = 32;

struct QArgs {
  const void* x;
  int64_t n_tok, tok_off;
  int64_t tiles_per_seq, first_block, n_tiles;
  int d, bits, m, nc, layout;
  const float* cent;
  const float* bnd;
  const float* rot;   // [dp][dp]
  const float* qjl;   // [mp][dp]
  uint8_t* idx;
  uint32_t* sign;
  float* scale;
  float* rnorm;
  int64_t idx_pitch, sign_pitch, seq_stride;
  PageMap pm;         // where a sequence's blocks are written (identity unless paged)
};

template <int DT>
__device__ inline float load_elem(const void* p, int64_t i) {
  if constexpr (DT == TQ_F32) {
    return static_cast<const float*>(p)[i];
  } else if constexpr (DT == TQ_BF16) {
    uint32_t u = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(u << 16);
  } else {
    return (float)static_cast<const _Float16*>(p)[i];
  }
}

// WIDE = false (dp <= 128): one wave per 32-column block of Pi (and of S),
// whose B operand stays in registers.  WIDE = true (dp up to 256): four waves
// loop over the column blocks and stream the B operand from L2 (each row of
// Pi / S is read by every tile; 16 loads per wave are in flight).
template <int DP, int DT, bool WIDE>
__global__ void __launch_bounds__(WIDE ? 256 : 512) k_quantize(QArgs a) {
  constexpr int KS = DP / 2;      // k-steps of the 32x32x2 MFMA
  constexpr int RW = DP / 32;     // rotation column blocks
  __shared__ float xs[TILE][DP + 1];   // X, then the residual R
  __shared__ float ys[TILE][DP + 1];   // Y = Pi x / |x|
  __shared__ uint8_t ids[TILE][DP];
  __shared__ float s_cent[256];
  __shared__ float s_bnd[256];
  __shared__ float s_n[TILE], s_inv[TILE];
  __shared__ int s_valid[TILE];

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int nwaves = nthr >> 6;
  const int L = 1 << a.bits;
  const int mp = (a.m + 31) & ~31;
  const int QW = a.m > 0 ? mp / 32 : 0;      // QJL column blocks
  for (int i = tid; i < L; i += nthr) s_cent[i] = a.cent[i];
  for (int i = tid; i < L - 1; i += nthr) s_bnd[i] = a.bnd[i];

  // register B operands (WIDE = false): B[k][j] = M[j][k], lane holds k = 2kk + lane/32
  float bop[WIDE ? 1 : KS];
  const bool rot_wave = !WIDE && wave < RW;
  const bool qjl_wave = !WIDE && a.m > 0 && wave >= RW && wave < RW + QW;
  if constexpr (!WIDE) {
    if (rot_wave) {
      const float* src = a.rot + (int64_t)(32 * wave + (lane & 31)) * DP + (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) bop[kk] = src[2 * kk];
    } else if (qjl_wave) {
      const float* src = a.qjl + (int64_t)(32 * (wave - RW) + (lane & 31)) * DP + (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) bop[kk] = src[2 * kk];
    }
  }
  __syncthreads();

  // 32x32 block of X M^T (rows = tile rows, columns 32*cb..) with M = Pi or S
  auto gemm_block = [&](const float (*in)[DP + 1], const float* M, int cb) {
    f32x16 acc = {};
    const float* src = M + (int64_t)(32 * cb + (lane & 31)) * DP + (lane >> 5);
#pragma unroll 16
    for (int kk = 0; kk < KS; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(in[lane & 31][2 * kk + (lane >> 5)], src[2 * kk],
                                                 acc, 0, 0, 0);
    return acc;
  };

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const int64_t seq = tile / a.tiles_per_seq;
    const int64_t blk = a.first_block + tile % a.tiles_per_seq;
    const int64_t abs0 = blk * TILE;
    int64_t oseq, oblk;                                   // output plane and block
    page_block(a.pm, seq, blk, oseq, oblk);
    const int64_t pos0 = oseq * a.seq_stride + oblk * TILE;   // code row of tile row 0
    const int64_t src0 = seq * a.n_tok + (abs0 - a.tok_off);  // input row of tile row 0

    // (a) load X (fp32) -- rows outside [tok_off, tok_off + n_tok) are zero
    if (tid < TILE) {
      const int64_t p = abs0 + tid;
      s_valid[tid] = (p >= a.tok_off && p < a.tok_off + a.n_tok) ? 1 : 0;
    }
    const bool full_tile = abs0 >= a.tok_off && abs0 + TILE <= a.tok_off + a.n_tok;
    if (full_tile && a.d == DP && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0) {
      // the tile's 32 rows are contiguous in the input: 16-byte loads
      constexpr int EPV = DT == TQ_F32 ? 4 : 8;          // elements per 16 bytes
      const char* base = static_cast<const char*>(a.x) + src0 * DP * (DT == TQ_F32 ? 4 : 2);
      for (int c = tid; c < TILE * DP / EPV; c += nthr) {
        const uint4 u = reinterpret_cast<const uint4*>(base)[c];
        const int e0 = c * EPV, r = e0 / DP, i0 = e0 % DP;
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        if constexpr (DT == TQ_F32) {
#pragma unroll
          for (int k = 0; k < 4; ++k) xs[r][i0 + k] = __uint_as_float(w[k]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if constexpr (DT == TQ_BF16) {
              xs[r][i0 + 2 * k] = __uint_as_float(w[k] << 16);
              xs[r][i0 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
            } else {
              xs[r][i0 + 2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xFFFFu));
              xs[r][i0 + 2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
            }
          }
        }
      }
    } else {
      for (int e = tid; e < TILE * DP; e += nthr) {
        const int r = e / DP, i = e % DP;
        const int64_t p = abs0 + r;
        float v = 0.f;
        if (i < a.d && p >= a.tok_off && p < a.tok_off + a.n_tok)
          v = load_elem<DT>(a.x, (src0 + r) * a.d + i);
        xs[r][i] = v;
      }
    }
    __syncthreads();

    // (b) norms, 8 lanes per row
    if (tid < 256) {
      const int r = tid >> 3, part = tid & 7;
      float s = 0.f;
      for (int i = part; i < DP; i += 8) s += xs[r][i] * xs[r][i];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      if (part == 0) {
        const float n = sqrtf(s);
        s_n[r] = n;
        s_inv[r] = n > 0.f ? 1.0f / n : 0.f;
      }
    }
    __syncthreads();

    // (c) rotation Z = X Pi^T on fp32 MFMA; (d) y = z / n and
    // idx = #{k : y >= t_k} (binary search on sorted t)
    auto finish_rot = [&](const f32x16& acc, int cb) {
      const int col = 32 * cb + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const float y = acc[v] * s_inv[row];
        int idx = 0;
        for (int step = L >> 1; step >= 1; step >>= 1)
          if (y >= s_bnd[idx + step - 1]) idx += step;
        ys[row][col] = y;
        ids[row][col] = (uint8_t)idx;
      }
    };
    if constexpr (WIDE) {
      for (int cb = wave; cb < RW; cb += nwaves) finish_rot(gemm_block(xs, a.rot, cb), cb);
    } else if (rot_wave) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[lane & 31][2 * kk + (lane >> 5)], bop[kk],
                                                   acc, 0, 0, 0);
      finish_rot(acc, wave);
    }
    __syncthreads();

    // (e) scale (norm correction) and QJL residual, 8 lanes per row
    if (tid < 256) {
      const int r = tid >> 3, part = tid & 7;
      float c2 = 0.f;
      for (int i = part; i < a.d; i += 8) {
        const float c = s_cent[ids[r][i]];
        c2 += c * c;
      }
      c2 += __shfl_xor(c2, 1);
      c2 += __shfl_xor(c2, 2);
      c2 += __shfl_xor(c2, 4);
      const float n = s_n[r];
      const float nh = sqrtf(c2);
      const float sc = a.nc ? n / nh : n;
      float rho2 = 0.f;
      if (a.m > 0) {
        const float f = a.nc ? 1.0f / nh : 1.0f;
        for (int i = part; i < DP; i += 8) {
          float rr = 0.f;
          if (i < a.d) rr = ys[r][i] - s_cent[ids[r][i]] * f;
          xs[r][i] = rr;
          rho2 += rr * rr;
        }
        rho2 += __shfl_xor(rho2, 1);
        rho2 += __shfl_xor(rho2, 2);
        rho2 += __shfl_xor(rho2, 4);
      }
      if (part == 0 && s_valid[r]) {
        a.scale[pos0 + r] = sc;
        if (a.m > 0) a.rnorm[pos0 + r] = n * sqrtf(rho2);
      }
    }
    __syncthreads();

    // (f) QJL signs: U = R S^T, one ballot = two 32-bit sign words
    auto finish_qjl = [&](const f32x16& u, int wj) {
      const int nbits = a.m - 32 * wj;               // valid bits in this word
      const uint32_t keep = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const unsigned long long msk = __ballot(u[v] >= 0.f);
        const int row_lo = 8 * (v >> 2) + (v & 3);
        const int row_hi = row_lo + 4;
        if (lane == 0) {
          if (s_valid[row_lo])
            a.sign[((pos0 + row_lo) * a.sign_pitch >> 2) + wj] = (uint32_t)msk & keep;
          if (s_valid[row_hi])
            a.sign[((pos0 + row_hi) * a.sign_pitch >> 2) + wj] = (uint32_t)(msk >> 32) & keep;
        }
      }
    };
    if constexpr (WIDE) {
      for (int cb = wave; cb < QW; cb += nwaves) finish_qjl(gemm_block(xs, a.qjl, cb), cb);
    } else if (qjl_wave) {
      f32x16 u = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        u = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[lane & 31][2 * kk + (lane >> 5)], bop[kk], u,
                                                 0, 0, 0);
      finish_qjl(u, wave - RW);
    }

    // (g) pack indices
    const int b = a.bits;
    if (a.layout == TQ_LAYOUT_ROW) {
      const int W = b * DP / 32;                     // words per row
      for (int e = tid; e < TILE * W; e += nthr) {
        const int r = e / W, w = e % W;
        if (!s_valid[r]) continue;
        const int bit0 = 32 * w;
        const int i0 = bit0 / b;
        int i1 = (bit0 + 31) / b;
        if (i1 > a.d - 1) i1 = a.d - 1;
        uint64_t accw = 0;
        for (int i = i0; i <= i1; ++i)
          accw |= (uint64_t)ids[r][i] << (i * b - bit0 + 32);
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx + (pos0 + r) * a.idx_pitch);
        dst[w] = (uint32_t)(accw >> 32);
      }
    } else {
      // tile32: the block's bit stream is 64 records x ndb groups x 8 fields;
      // field q = (r*ndb + j)*8 + e of record r = 16*G + C holds coordinate
      // 16*j + C of token 4*G + e%4 + 16*(e/4)
      bool full = true;
      for (int r = 0; r < TILE; ++r) full = full && s_valid[r];
      const int ndb = (a.d + 15) / 16;
      const int words = 16 * ndb * b;                 // 64*ndb*b bytes
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx) +
                      (oseq * (a.seq_stride / TILE) + oblk) * (int64_t)words;
      for (int w = tid; w < words; w += nthr) {
        const int bit0 = 32 * w;
        const int q0 = bit0 / b;
        const int q1 = (bit0 + 31) / b;
        uint64_t val = 0, msk = 0;
        // walk the fields q0..q1: field q = (r*ndb + j)*8 + e, one division per word
        int e = q0 & 7, j = (q0 >> 3) % ndb, r = (q0 >> 3) / ndb;
        for (int q = q0; q <= q1; ++q) {
          const int i = 16 * j + (r & 15);
          const int t = 4 * (r >> 4) + (e & 3) + 16 * (e >> 2);
          const int sh = q * b - bit0 + 32;
          if (s_valid[t]) {
            if (i < a.d) val |= (uint64_t)ids[t][i] << sh;
            msk |= (uint64_t)((1u << b) - 1u) << sh;
          }
          if (++e == 8) {
            e = 0;
            if (++j == ndb) { j = 0; ++r; }
          }
        }
        const uint32_t nv = (uint32_t)(val >> 32), nm = (uint32_t)(msk >> 32);
        if (full) {
          dst[w] = nv;
        } else if (nm != 0u) {
          dst[w] = (dst[w] & ~nm) | (nv & nm);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- appends
//
// Few vectors (decode-time appends): one workgroup per vector; y = Pi x / |x|
// and u = S r are matrix-vector products over the transposed matrices
// (coalesced rows).  tile32 fields of different vectors can share a 32-bit
// word, so they are updated with an atomic AND (clear) and an atomic OR (set).

struct SmallJob {
  const void* x;
  int64_t n_tok, tok_off;
  int d, bits, m, nc, layout, dp, mp;
  const float* cent;
  const float* bnd;
  const float* rotT;  // [dp][dp], rotT[k][i] = Pi[i][k]
  const float* qjlT;  // [dp][mp], qjlT[i][j] = S[j][i]
  uint8_t* idx;
  uint32_t* sign;
  float* scale;
  float* rnorm;
  int64_t idx_pitch, sign_pitch, seq_stride;
  PageMap pm;
};

struct SmallArgs {
  SmallJob job[2];
  int64_t nvec;      // vectors per job (n_seq * n_tok)
  int njobs;         // job rows of the grid; a further row runs the decode prologue
  PArgs pro;         // decode query prologue of pro_rows rows (4 workgroups each)
  int64_t pro_rows;
};

__device__ inline float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int DT, int NI>
__global__ void __launch_bounds__(4 * NI) k_quantize_small(SmallArgs sa) {
  // One workgroup of 4*NI threads per vector (NI = 128 or 256 >= dp, mp):
  // thread (i, kq) = (tid % NI, tid / NI) forms the partial product of output
  // coordinate i over the input coordinates NI/4 kq .. NI/4 (kq + 1) - 1, so
  // every matrix load of a thread is independent and issued together; the
  // four partials are summed in LDS in a fixed order.  With NI = 128 the
  // thread's rotation and sketch entries, the boundaries and the centroids
  // are all requested before the vector itself, so the vector costs one
  // memory round trip in total.
  constexpr int NT = 4 * NI, KQ = NI / 4, NW = NI / 64;
  constexpr bool PRE = NI == 128;
  if ((int)blockIdx.y >= sa.njobs) {
    // the fused decode step: workgroup (4 row + part) of this grid row forms
    // the query operands of decode row `row` (its first 256 threads work,
    // the others only meet its barriers)
    if ((int64_t)(blockIdx.x >> 2) >= sa.pro_rows) return;
    prologue::run(sa.pro, (int)(blockIdx.x & 3), (int)(blockIdx.x >> 2), threadIdx.x < 256);
    return;
  }
  if ((int64_t)blockIdx.x >= sa.nvec) return;   // the grid is as wide as the prologue's
  const SmallJob& a = sa.job[blockIdx.y];
  __shared__ float xs[NI];
  __shared__ float part[4][NI];
  __shared__ float rs[NI];
  __shared__ uint8_t ids[NI];
  __shared__ float red[2][NW];
  __shared__ float s_bnd[256], s_cent[256];
  const int64_t vec = blockIdx.x;                 // seq * n_tok + t
  const int64_t seq = vec / a.n_tok, t = vec % a.n_tok;
  const int64_t pos = a.tok_off + t;              // position in the sequence
  int64_t oseq, oblk;                             // output plane and block of the position
  page_block(a.pm, seq, pos >> 5, oseq, oblk);
  const int64_t row = oseq * a.seq_stride + oblk * 32 + (pos & 31);
  const int tid = threadIdx.x;
  const int i = tid & (NI - 1), kq = tid / NI, l = tid & 63, w = tid >> 6;
  const int L = 1 << a.bits;
  float rv[PRE ? KQ : 1], qv[PRE ? KQ : 1];
  if constexpr (PRE) {
    const bool sk = a.m > 0;
    const float* qsrc = sk ? a.qjlT : a.rotT;
    const int qstr = sk ? a.mp : a.dp;
    const int ir = i < a.dp ? i : a.dp - 1, iq = i < qstr ? i : qstr - 1;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const int k = KQ * kq + kk;
      const int kc = k < a.d ? k : a.d - 1;
      rv[kk] = a.rotT[kc * a.dp + ir];
      qv[kk] = qsrc[kc * qstr + iq];
    }
  }
  const float bv = tid < L - 1 ? a.bnd[tid] : 0.f;
  const float cv = tid < L ? a.cent[tid] : 0.f;
  if (tid < NI) xs[tid] = (tid < a.d) ? load_elem<DT>(a.x, vec * a.d + tid) : 0.f;
  if (tid < 256) { s_bnd[tid] = bv; s_cent[tid] = cv; }
  __syncthreads();
  float n2 = 0.f;
#pragma unroll
  for (int j = 0; j < NW; ++j) n2 += xs[l + 64 * j] * xs[l + 64 * j];
  const float n = sqrtf(wave_sum(n2));
  const float inv = n > 0.f ? 1.0f / n : 0.f;
  {
    float z = 0.f;
    if (i < a.dp) {
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) {
        const int k = KQ * kq + kk;
        const int kc = k < a.d ? k : a.d - 1;     // xs[k] = 0 beyond d
        if constexpr (PRE) z += rv[kk] * xs[k];
        else z += a.rotT[kc * a.dp + i] * xs[k];
      }
    }
    part[kq][i] = z;
  }
  __syncthreads();
  float y = 0.f, c = 0.f;
  if (tid < NI) {
    y = (((part[0][i] + part[1][i]) + part[2][i]) + part[3][i]) * inv;
    int q = 0;
    for (int step = L >> 1; step >= 1; step >>= 1)
      if (y >= s_bnd[q + step - 1]) q += step;
    c = (i < a.d) ? s_cent[q] : 0.f;
    if (i < a.d) ids[i] = (uint8_t)q;
    const float s2 = wave_sum(c * c);
    if (l == 0) red[0][w] = s2;
  }
  __syncthreads();
  float nh2 = 0.f;
#pragma unroll
  for (int j = 0; j < NW; ++j) nh2 += red[0][j];
  const float nh = sqrtf(nh2);
  const float sc = a.nc ? n / nh : n;
  if (a.m > 0) {
    if (tid < NI) {
      const float f = a.nc ? 1.0f / nh : 1.0f;
      const float r = (i < a.d) ? y - c * f : 0.f;
      rs[i] = r;
      const float s2 = wave_sum(r * r);
      if (l == 0) red[1][w] = s2;
    }
    __syncthreads();
    {
      float u = 0.f;
      if (i < a.m) {
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk) {
          const int k = KQ * kq + kk;
          const int kc = k < a.d ? k : a.d - 1;   // rs[k] = 0 beyond d
          if constexpr (PRE) u += qv[kk] * rs[k];
          else u += a.qjlT[kc * a.mp + i] * rs[k];
        }
      }
      part[kq][i] = u;
    }
    __syncthreads();
    if (tid < NI) {
      const float u = ((part[0][i] + part[1][i]) + part[2][i]) + part[3][i];
      const unsigned long long bb = __ballot(u >= 0.f);
      uint32_t* srow = a.sign + ((row * a.sign_pitch) >> 2);
      const int words = (a.m + 31) / 32;
      const int wd = 2 * w + l;                     // word of this wave's coordinates
      if (l < 2 && wd < words) {
        uint32_t wv = (uint32_t)(bb >> (32 * l));
        const int nbits = a.m - 32 * wd;
        if (nbits < 32) wv &= (1u << nbits) - 1u;
        srow[wd] = wv;
      }
      if (tid == 0) {
        float r2 = 0.f;
        for (int j = 0; j < NW; ++j) r2 += red[1][j];
        a.rnorm[row] = n * sqrtf(r2);
      }
    }
  }
  if (tid == 0) a.scale[row] = sc;
  __syncthreads();
  const int b = a.bits;
  if (a.layout == TQ_LAYOUT_ROW) {
    const int W = b * a.dp / 32;
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx + row * a.idx_pitch);
    for (int wd = tid; wd < W; wd += NT) {
      const int bit0 = 32 * wd;
      const int j0 = bit0 / b;
      int j1 = (bit0 + 31) / b;
      if (j1 > a.d - 1) j1 = a.d - 1;
      uint64_t acc = 0;
      for (int j = j0; j <= j1; ++j) acc |= (uint64_t)ids[j] << (j * b - bit0 + 32);
      dst[wd] = (uint32_t)(acc >> 32);
    }
  } else {
    const int ndb = (a.d + 15) / 16;
    const int words = 16 * ndb * b;
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx) + (oseq * (a.seq_stride / 32) + oblk) * (int64_t)words;
    const int tt = (int)(pos & 31);
    const int G = (tt & 15) >> 2, e = (tt & 3) + 4 * (tt >> 4);
    if (tid < a.d) {
      const int r = 16 * G + (tid & 15), j = tid >> 4;
      const int bit = ((r * ndb + j) * 8 + e) * b;
      const uint64_t v = (uint64_t)ids[tid] << (bit & 31);
      const uint64_t mk = (uint64_t)((1u << b) - 1u) << (bit & 31);
      const int wd = bit >> 5;
      atomicAnd(dst + wd, ~(uint32_t)mk);
      atomicOr(dst + wd, (uint32_t)v);
      if ((mk >> 32) != 0) {
        atomicAnd(dst + wd + 1, ~(uint32_t)(mk >> 32));
        atomicOr(dst + wd + 1, (uint32_t)(v >> 32));
      }
    }
  }
}

template <int DP, bool WIDE>
hipError_t launch_dp(const QArgs& a, int dt, int nthr, int grid, hipStream_t st) {
  switch (dt) {
    case TQ_F32: hipLaunchKernelGGL((k_quantize<DP, TQ_F32, WIDE>), dim3(grid), dim3(nthr), 0, st, a); break;
    case TQ_BF16: hipLaunchKernelGGL((k_quantize<DP, TQ_BF16, WIDE>), dim3(grid), dim3(nthr), 0, st, a); break;
    default: hipLaunchKernelGGL((k_quantize<DP, TQ_F16, WIDE>), dim3(grid), dim3(nthr), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

static SmallJob make_small_job(const tq_codebook* cb, const QuantJob& job) {
  SmallJob s{};
  s.x = job.x;
  s.n_tok = job.n_tok;
  s.tok_off = job.tok_offset;
  s.d = cb->p.d; s.bits = cb->p.bits; s.m = cb->p.qjl_m; s.nc = cb->p.norm_correction;
  s.layout = job.out.layout; s.dp = cb->dp; s.mp = cb->mp;
  s.cent = cb->dev.cent; s.bnd = cb->dev.bnd; s.rotT = cb->dev.rotT; s.qjlT = cb->dev.qjlT;
  s.idx = static_cast<uint8_t*>(job.out.idx);
  s.sign = static_cast<uint32_t*>(job.out.sign);
  s.scale = job.out.scale; s.rnorm = job.out.rnorm;
  s.idx_pitch = job.out.idx_row_bytes; s.sign_pitch = job.out.sign_row_bytes;
  s.seq_stride = job.out.seq_stride;
  s.pm = job.pm;
  return s;
}

hipError_t launch_quantize_small(const tq_codebook* const* cbs, const QuantJob* jobs, int njobs,
                                 hipStream_t stream, const PArgs* pro, int64_t pro_rows) {
  SmallArgs sa{};
  for (int t = 0; t < njobs; ++t) sa.job[t] = make_small_job(cbs[t], jobs[t]);
  const int64_t nvec = jobs[0].n_seq * jobs[0].n_tok;
  sa.nvec = nvec;
  sa.njobs = njobs;
  if (pro) {
    sa.pro = *pro;
    sa.pro_rows = pro_rows;
  }
  const int64_t gx = pro && 4 * pro_rows > nvec ? 4 * pro_rows : nvec;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)(njobs + (pro ? 1 : 0)));
  ProfileScope prof(TQ_KERNEL_QUANTIZE, stream);
  bool wide = false;
  for (int t = 0; t < njobs; ++t) wide = wide || cbs[t]->dp > 128 || cbs[t]->mp > 128;
  if (!wide) {
    switch (jobs[0].dt) {
      case TQ_F32: hipLaunchKernelGGL((k_quantize_small<TQ_F32, 128>), grid, dim3(512), 0, stream, sa); break;
      case TQ_BF16: hipLaunchKernelGGL((k_quantize_small<TQ_BF16, 128>), grid, dim3(512), 0, stream, sa); break;
      default: hipLaunchKernelGGL((k_quantize_small<TQ_F16, 128>), grid, dim3(512), 0, stream, sa); break;
    }
  } else {
    switch (jobs[0].dt) {
      case TQ_F32: hipLaunchKernelGGL((k_quantize_small<TQ_F32, 256>), grid, dim3(1024), 0, stream, sa); break;
      case TQ_BF16: hipLaunchKernelGGL((k_quantize_small<TQ_BF16, 256>), grid, dim3(1024), 0, stream, sa); break;
      default: hipLaunchKernelGGL((k_quantize_small<TQ_F16, 256>), grid, dim3(1024), 0, stream, sa); break;
    }
  }
  return hipGetLastError();
}

bool quantize_supported(const tq_codebook* cb) {
  return cb->dp <= 256 && (cb->p.qjl_m == 0 || cb->mp <= 256);
}

hipError_t launch_quantize(const tq_codebook* cb, const QuantJob& job, hipStream_t stream) {
  if (quantize128_supported(cb, job)) return launch_quantize128(cb, job, stream);
  QArgs a{};
  a.x = job.x;
  a.n_tok = job.n_tok;
  a.tok_off = job.tok_offset;
  a.first_block = job.tok_offset / TILE;
  const int64_t last_block = (job.tok_offset + job.n_tok - 1) / TILE;
  a.tiles_per_seq = last_block - a.first_block + 1;
  a.n_tiles = a.tiles_per_seq * job.n_seq;
  a.d = cb->p.d;
  a.bits = cb->p.bits;
  a.m = cb->p.qjl_m;
  a.nc = cb->p.norm_correction;
  a.layout = job.out.layout;
  a.cent = cb->dev.cent;
  a.bnd = cb->dev.bnd;
  a.rot = cb->dev.rot;
  a.qjl = cb->dev.qjl;
  a.idx = static_cast<uint8_t*>(job.out.idx);
  a.sign = static_cast<uint32_t*>(job.out.sign);
  a.scale = job.out.scale;
  a.rnorm = job.out.rnorm;
  a.idx_pitch = job.out.idx_row_bytes;
  a.sign_pitch = job.out.sign_row_bytes;
  a.seq_stride = job.out.seq_stride;
  a.pm = job.pm;
  ProfileScope prof(TQ_KERNEL_QUANTIZE, stream);
  if (cb->dp <= 128 && (cb->p.qjl_m == 0 || cb->mp <= 128)) {
    const int waves_needed = cb->dp / 32 + (cb->p.qjl_m > 0 ? cb->mp / 32 : 0);
    const int nw = waves_needed < 4 ? 4 : waves_needed;
    const int nthr = 64 * nw;
    const int grid = (int)(a.n_tiles < 2048 ? a.n_tiles : 2048);
    switch (cb->dp) {
      case 32: return launch_dp<32, false>(a, job.dt, nthr, grid, stream);
      case 64: return launch_dp<64, false>(a, job.dt, nthr, grid, stream);
      case 96: return launch_dp<96, false>(a, job.dt, nthr, grid, stream);
      default: return launch_dp<128, false>(a, job.dt, nthr, grid, stream);
    }
  }
  // d in (128, 256] or a sketch of more than 128 rows: four waves stream Pi
  // and S from L2 (DP is the row stride of both matrices, = dp)
  const int grid = (int)(a.n_tiles < 1024 ? a.n_tiles : 1024);
  switch (cb->dp) {
    case 32: return launch_dp<32, true>(a, job.dt, 256, grid, stream);
    case 64: return launch_dp<64, true>(a, job.dt, 256, grid, stream);
    case 96: return launch_dp<96, true>(a, job.dt, 256, grid, stream);
    case 128: return launch_dp<128, true>(a, job.dt, 256, grid, stream);
    case 160: return launch_dp<160, true>(a, job.dt, 256, grid, stream);
    case 192: return launch_dp<192, true>(a, job.dt, 256, grid, stream);
    case 224: return launch_dp<224, true>(a, job.dt, 256, grid, stream);
    default: return launch_dp<256, true>(a, job.dt, 256, grid, stream);
  }
}

}  // namespace tq
