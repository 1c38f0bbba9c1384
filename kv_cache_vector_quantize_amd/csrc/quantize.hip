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

// tile32 element q of a block (q-th b-bit field of its bit stream) ->
// (coordinate i, token t): q = (r*ndb + j)*8 + e, record r = 16*G + C holds
// coordinate 16*j + C for the tokens 4*G + e%4 + 16*(e/4).
__device__ inline void tile32_element(int q, int ndb, int& i, int& t) {
  const int e = q & 7, rj = q >> 3;
  const int j = rj % ndb, r = rj / ndb;
  i = 16 * j + (r & 15);
  t = 4 * (r >> 4) + (e & 3) + 16 * (e >> 2);
}

template <int DP, int DT>
__global__ void __launch_bounds__(512) k_quantize(QArgs a) {
  constexpr int KS = DP / 2;      // k-steps of the 32x32x2 MFMA
  constexpr int RW = DP / 32;     // rotation waves
  __shared__ float xs[TILE][DP + 1];   // X, then Y, then the residual R
  __shared__ uint8_t ids[TILE][DP];
  __shared__ float s_cent[256];
  __shared__ float s_bnd[256];
  __shared__ float s_n[TILE], s_inv[TILE];
  __shared__ int s_valid[TILE];

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int L = 1 << a.bits;
  const int mp = (a.m + 31) & ~31;
  for (int i = tid; i < L; i += nthr) s_cent[i] = a.cent[i];
  for (int i = tid; i < L - 1; i += nthr) s_bnd[i] = a.bnd[i];

  // B operands in registers: B[k][j] = M[j][k], lane holds k = 2kk + lane/32
  float bop[KS];
  const bool rot_wave = wave < RW;
  const bool qjl_wave = a.m > 0 && wave >= RW && wave < RW + mp / 32;
  if (rot_wave) {
    const float* src = a.rot + (int64_t)(32 * wave + (lane & 31)) * DP + (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) bop[kk] = src[2 * kk];
  } else if (qjl_wave) {
    const float* src = a.qjl + (int64_t)(32 * (wave - RW) + (lane & 31)) * DP + (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) bop[kk] = src[2 * kk];
  }
  __syncthreads();

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const int64_t seq = tile / a.tiles_per_seq;
    const int64_t blk = a.first_block + tile % a.tiles_per_seq;
    const int64_t abs0 = blk * TILE;
    const int64_t pos0 = seq * a.seq_stride + abs0;      // code row of tile row 0
    const int64_t src0 = seq * a.n_tok + (abs0 - a.tok_off);  // input row of tile row 0

    // (a) load X (fp32) -- rows outside [tok_off, tok_off + n_tok) are zero
    if (tid < TILE) {
      const int64_t p = abs0 + tid;
      s_valid[tid] = (p >= a.tok_off && p < a.tok_off + a.n_tok) ? 1 : 0;
    }
    for (int e = tid; e < TILE * DP; e += nthr) {
      const int r = e / DP, i = e % DP;
      const int64_t p = abs0 + r;
      float v = 0.f;
      if (i < a.d && p >= a.tok_off && p < a.tok_off + a.n_tok)
        v = load_elem<DT>(a.x, (src0 + r) * a.d + i);
      xs[r][i] = v;
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

    // (c) rotation Z = X Pi^T on fp32 MFMA
    f32x16 acc = {};
    if (rot_wave) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[lane & 31][2 * kk + (lane >> 5)], bop[kk],
                                                   acc, 0, 0, 0);
    }
    __syncthreads();

    // (d) y = z / n and idx = #{k : y >= t_k} (binary search on sorted t)
    if (rot_wave) {
      const int col = 32 * wave + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const float y = acc[v] * s_inv[row];
        int idx = 0;
        for (int step = L >> 1; step >= 1; step >>= 1)
          if (y >= s_bnd[idx + step - 1]) idx += step;
        xs[row][col] = y;
        ids[row][col] = (uint8_t)idx;
      }
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
          if (i < a.d) rr = xs[r][i] - s_cent[ids[r][i]] * f;
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
    if (qjl_wave) {
      f32x16 u = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        u = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[lane & 31][2 * kk + (lane >> 5)], bop[kk], u,
                                                 0, 0, 0);
      const int wj = wave - RW;                      // sign word index
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
      // tile32: the block's bit stream is 64 records x ndb groups x 8 fields
      bool full = true;
      for (int r = 0; r < TILE; ++r) full = full && s_valid[r];
      const int ndb = (a.d + 15) / 16;
      const int words = 16 * ndb * b;                 // 64*ndb*b bytes
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx) +
                      (seq * (a.seq_stride / TILE) + blk) * (int64_t)words;
      for (int w = tid; w < words; w += nthr) {
        const int bit0 = 32 * w;
        const int q0 = bit0 / b;
        const int q1 = (bit0 + 31) / b;
        uint64_t val = 0, msk = 0;
        for (int q = q0; q <= q1; ++q) {
          int i, t;
          tile32_element(q, ndb, i, t);
          const int sh = q * b - bit0 + 32;
          if (s_valid[t]) {
            if (i < a.d) val |= (uint64_t)ids[t][i] << sh;
            msk |= (uint64_t)((1u << b) - 1u) << sh;
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

template <int DP>
hipError_t launch_dp(const QArgs& a, int dt, int nthr, int grid, hipStream_t st) {
  switch (dt) {
    case TQ_F32: hipLaunchKernelGGL((k_quantize<DP, TQ_F32>), dim3(grid), dim3(nthr), 0, st, a); break;
    case TQ_BF16: hipLaunchKernelGGL((k_quantize<DP, TQ_BF16>), dim3(grid), dim3(nthr), 0, st, a); break;
    default: hipLaunchKernelGGL((k_quantize<DP, TQ_F16>), dim3(grid), dim3(nthr), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

bool quantize_supported(const tq_codebook* cb) {
  return cb->dp <= 128 && (cb->p.qjl_m == 0 || cb->mp <= 128);
}

hipError_t launch_quantize(const tq_codebook* cb, const QuantJob& job, hipStream_t stream) {
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
  const int waves_needed = cb->dp / 32 + (cb->p.qjl_m > 0 ? cb->mp / 32 : 0);
  const int nw = waves_needed < 4 ? 4 : waves_needed;
  const int nthr = 64 * nw;
  int64_t grid = a.n_tiles < 2048 ? a.n_tiles : 2048;
  ProfileScope prof(TQ_KERNEL_QUANTIZE, stream);
  switch (cb->dp) {
    case 32: return launch_dp<32>(a, job.dt, nthr, (int)grid, stream);
    case 64: return launch_dp<64>(a, job.dt, nthr, (int)grid, stream);
    case 96: return launch_dp<96>(a, job.dt, nthr, (int)grid, stream);
    default: return launch_dp<128>(a, job.dt, nthr, (int)grid, stream);
  }
}

}  // namespace tq
