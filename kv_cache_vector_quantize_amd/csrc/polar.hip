// PolarQuant encoding: quantize and dequantize (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog), "TurboQuant 工作原理" >
// "第一阶段：随机旋转 + PolarQuant 压缩" item 2: the rotated, normalised vector
// is carried to polar form by pairing dimensions recursively (the radius
// keeps the magnitude, the angles the direction) and each angle is coded by
// a Lloyd-Max quantizer for its known law; "第二阶段：QJL 残差校正" sketches
// the residual as for the scalar encoding.
//
// Quantize: a workgroup owns 32 consecutive positions of one sequence
// (persistent grid over such tiles).  The rotation Z = X Pi^T runs on fp32
// MFMA (v_mfma_f32_32x32x2f32, one wave per 32 columns with its slice of Pi
// in registers); y = z / |x| is staged in LDS and the polar levels are
// walked in place: level 1 takes the coordinate pairs, each higher level the
// radii of the level below (two LDS radius buffers, one barrier per level);
// every angle is coded against its level's boundaries (binary search, a tie
// goes up).  With a sketch, each coordinate of y_hat is the product of the
// cos / sin of its path's centroid angles, r = y - y_hat is staged, and
// U = R S^T runs on fp32 MFMA as the rotation; 64-lane ballots of U >= 0
// give the sign words.  Codes are packed per 32-bit word of the row's
// level-major bit stream.
//
// Dequantize: the same tile; y_hat from the codes, then
// x_hat = scale y_hat Pi + rnorm (2 sigma - 1) (sqrt(pi/2)/m S Pi) as row
// vectors, on fp32 MFMA with Pi and the folded sketch streamed from L2.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int TILE = 32;
constexpr int kPolarThreads = 512;
constexpr int kMaxTrig = 2 * 256 * kPolarMaxLevels;   // (cos, sin) of every centroid
constexpr int kMaxBnd = 255 * kPolarMaxLevels;

struct PolarTables {
  int d, levels, b1, br, field_bits;
  int cent_off[kPolarMaxLevels + 2];
  int bnd_off[kPolarMaxLevels + 2];
  const float* trig;   // (cos, sin) of each centroid, level-major
  const float* bnd;    // boundaries, level-major
};

struct PQArgs {
  const void* x;
  int64_t n_tok, tok_off;
  int64_t tiles_per_seq, first_block, n_tiles;
  int m;
  PolarTables t;
  const float* rot;   // [dp][dp] row-major Pi
  const float* qjl;   // [mp][dp] row-major S
  uint8_t* idx;
  uint32_t* sign;
  float* scale;
  float* rnorm;
  int64_t idx_pitch, sign_pitch, seq_stride;
  PageMap pm;
};

template <int DT>
__device__ inline float load_elem(const void* p, int64_t i) {
  if constexpr (DT == TQ_F32) {
    return static_cast<const float*>(p)[i];
  } else if constexpr (DT == TQ_BF16) {
    return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
  } else {
    return (float)static_cast<const _Float16*>(p)[i];
  }
}

// first code slot of level lv (slots are level-major: d/2 level-1 angles,
// then d/4 level-2 angles, ...)
__device__ inline int level_slot0(int d, int lv) { return d - (d >> (lv - 1)); }

// y_hat[j] of one vector: product over the levels of the cos (lower child)
// or sin (upper child) of the centroid angle on j's path
__device__ inline float polar_coord(const PolarTables& t, const float* s_trig, const uint8_t* ids, int j) {
  float v = 1.f;
  for (int lv = 1; lv <= t.levels; ++lv) {
    const int node = j >> lv;
    const int c = ids[level_slot0(t.d, lv) + node];
    v *= s_trig[2 * (t.cent_off[lv] + c) + ((j >> (lv - 1)) & 1)];
  }
  return v;
}

template <int DP, int DT>
__global__ void __launch_bounds__(kPolarThreads) k_polar_quantize(PQArgs a) {
  constexpr int KS = DP / 2;
  constexpr int RW = DP / 32;
  __shared__ float xs[TILE][DP + 1];          // X, then the residual R
  __shared__ float ys[TILE][DP + 1];          // Y = Pi x / |x|
  __shared__ float rad[2][TILE][DP / 2 + 1];  // radii of the current and next level
  __shared__ uint8_t ids[TILE][DP];           // code slots (d - 1 used)
  __shared__ float s_trig[kMaxTrig];
  __shared__ float s_bnd[kMaxBnd];
  __shared__ float s_n[TILE], s_inv[TILE];
  __shared__ int s_valid[TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int d = a.t.d;
  const int mp = (a.m + 31) & ~31;
  const int QW = a.m > 0 ? mp / 32 : 0;
  const int ntrig = 2 * a.t.cent_off[a.t.levels + 1], nbnd = a.t.bnd_off[a.t.levels + 1];
  for (int i = tid; i < ntrig; i += kPolarThreads) s_trig[i] = a.t.trig[i];
  for (int i = tid; i < nbnd; i += kPolarThreads) s_bnd[i] = a.t.bnd[i];

  // B operands in registers: B[k][j] = M[j][k], lane holds k = 2kk + lane/32
  float bop[KS];
  const bool rot_wave = wave < RW;
  const bool qjl_wave = a.m > 0 && wave >= RW && wave < RW + QW;
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
    int64_t oseq, oblk;
    page_block(a.pm, seq, blk, oseq, oblk);
    const int64_t pos0 = oseq * a.seq_stride + oblk * TILE;
    const int64_t src0 = seq * a.n_tok + (abs0 - a.tok_off);

    // (a) X in fp32; rows outside [tok_off, tok_off + n_tok) and padding
    // coordinates are zero
    if (tid < TILE) {
      const int64_t p = abs0 + tid;
      s_valid[tid] = (p >= a.tok_off && p < a.tok_off + a.n_tok) ? 1 : 0;
    }
    for (int e = tid; e < TILE * DP; e += kPolarThreads) {
      const int r = e / DP, i = e % DP;
      const int64_t p = abs0 + r;
      float v = 0.f;
      if (i < d && p >= a.tok_off && p < a.tok_off + a.n_tok) v = load_elem<DT>(a.x, (src0 + r) * d + i);
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

    // (c) Y = X Pi^T / |x| (a zero vector gives y = +0 exactly)
    if (rot_wave) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[lane & 31][2 * kk + (lane >> 5)], bop[kk], acc, 0, 0, 0);
      const int col = 32 * wave + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        ys[row][col] = s_n[row] > 0.f ? acc[v] * s_inv[row] : 0.f;
      }
    }
    __syncthreads();

    // (d) polar levels: level 1 on coordinate pairs, level l on the radii of
    // level l - 1; each angle is coded against its level's boundaries
    for (int lv = 1; lv <= a.t.levels; ++lv) {
      const int nf = d >> lv;
      const int bits = lv == 1 ? a.t.b1 : a.t.br;
      const float* tb = s_bnd + a.t.bnd_off[lv];
      const int slot0 = level_slot0(d, lv);
      float (*src)[DP / 2 + 1] = rad[(lv + 1) & 1];
      float (*dst)[DP / 2 + 1] = rad[lv & 1];
      for (int e = tid; e < TILE * nf; e += kPolarThreads) {
        const int r = e / nf, i = e % nf;
        float u, w;
        if (lv == 1) { u = ys[r][2 * i]; w = ys[r][2 * i + 1]; }
        else { u = src[r][2 * i]; w = src[r][2 * i + 1]; }
        const float ang = atan2f(w, u);
        dst[r][i] = sqrtf(fmaf(u, u, w * w));
        int c = 0;
        for (int step = 1 << (bits - 1); step >= 1; step >>= 1)
          if (ang >= tb[c + step - 1]) c += step;
        ids[r][slot0 + i] = (uint8_t)c;
      }
      __syncthreads();
    }

    // (e) scale = |x|; with a sketch, r = y - y_hat (y_hat from the codes)
    // and rnorm = |x| |r|, 8 lanes per row
    if (tid < 256) {
      const int r = tid >> 3, part = tid & 7;
      float rho2 = 0.f;
      if (a.m > 0) {
        for (int j = part; j < DP; j += 8) {
          float rr = 0.f;
          if (j < d) rr = ys[r][j] - polar_coord(a.t, s_trig, ids[r], j);
          xs[r][j] = rr;
          rho2 += rr * rr;
        }
        rho2 += __shfl_xor(rho2, 1);
        rho2 += __shfl_xor(rho2, 2);
        rho2 += __shfl_xor(rho2, 4);
      }
      if (part == 0 && s_valid[r]) {
        a.scale[pos0 + r] = s_n[r];
        if (a.m > 0) a.rnorm[pos0 + r] = s_n[r] * sqrtf(rho2);
      }
    }
    __syncthreads();

    // (f) sign words from U = R S^T: one ballot = two finished words
    if (qjl_wave) {
      f32x16 u = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        u = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[lane & 31][2 * kk + (lane >> 5)], bop[kk], u, 0, 0, 0);
      const int wj = wave - RW;
      const int nbits = a.m - 32 * wj;
      const uint32_t keep = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const unsigned long long msk = __ballot(u[v] >= 0.f);
        const int row_lo = 8 * (v >> 2) + (v & 3);
        const int row_hi = row_lo + 4;
        if (lane == 0) {
          if (s_valid[row_lo]) a.sign[((pos0 + row_lo) * a.sign_pitch >> 2) + wj] = (uint32_t)msk & keep;
          if (s_valid[row_hi]) a.sign[((pos0 + row_hi) * a.sign_pitch >> 2) + wj] = (uint32_t)(msk >> 32) & keep;
        }
      }
    }

    // (g) pack: word w of a row holds bits [32 w, 32 w + 32) of the stream
    {
      const int W = (a.t.field_bits + 31) / 32;
      const int h = d >> 1, b1 = a.t.b1, br = a.t.br, B1T = h * b1;
      for (int e = tid; e < TILE * W; e += kPolarThreads) {
        const int r = e / W, w = e % W;
        if (!s_valid[r]) continue;
        const int lo = 32 * w, hi = lo + 31;
        uint64_t acc = 0;
        if (lo < B1T) {
          const int s1 = min(h - 1, hi / b1);
          for (int s = lo / b1; s <= s1; ++s) acc |= (uint64_t)ids[r][s] << (s * b1 - lo + 32);
        }
        if (hi >= B1T && d > 2) {
          const int f0 = lo > B1T ? (lo - B1T) / br : 0;
          const int f1 = min(d - 2 - h, (hi - B1T) / br);
          for (int f = f0; f <= f1; ++f) acc |= (uint64_t)ids[r][h + f] << (B1T + f * br - lo + 32);
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.idx + (pos0 + r) * a.idx_pitch);
        dst[w] = (uint32_t)(acc >> 32);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- dequantize

struct PDArgs {
  const uint8_t* idx;
  const uint32_t* sign;
  const float* scale;
  const float* rnorm;
  int64_t idx_pitch, sign_pitch, seq_stride;
  int64_t n_tok, tok_off, n_seq, n_tiles, tiles_per_seq;
  int m, mp, dp;
  PolarTables t;
  const float* rot;     // [dp][dp] Pi
  const float* sprot;   // [mp][dp] sqrt(pi/2)/m S Pi
  void* out;
  int out_dt;
};

// Tiles of 32 positions of [tok_off, tok_off + n_tok) (not aligned to the
// code blocks: rows of a tile are consecutive requested positions).
template <int DP>
__global__ void __launch_bounds__(256) k_polar_dequantize(PDArgs a) {
  constexpr int KS = DP / 2;
  __shared__ float yh[TILE][DP + 1];      // scale * y_hat
  __shared__ float sg[TILE][128 + 1];     // rnorm * (2 sigma - 1), zero past m (m <= 128)
  __shared__ uint8_t ids[TILE][DP];
  __shared__ float s_trig[kMaxTrig];
  __shared__ float s_out[TILE][DP + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int d = a.t.d;
  const int ntrig = 2 * a.t.cent_off[a.t.levels + 1];
  for (int i = tid; i < ntrig; i += 256) s_trig[i] = a.t.trig[i];
  __syncthreads();
  const int W = (a.t.field_bits + 31) / 32;
  const int h = d >> 1, b1 = a.t.b1, br = a.t.br, B1T = h * b1;
  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const int64_t seq = tile / a.tiles_per_seq;
    const int64_t t0 = (tile % a.tiles_per_seq) * TILE;       // first requested position of the tile
    const int rows = (int)min((int64_t)TILE, a.n_tok - t0);
    // unpack code slots
    for (int e = tid; e < TILE * (d - 1); e += 256) {
      const int r = e / (d - 1), s = e % (d - 1);
      int c = 0;
      if (r < rows) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(
            a.idx + (seq * a.seq_stride + a.tok_off + t0 + r) * a.idx_pitch);
        const int bit = s < h ? s * b1 : B1T + (s - h) * br;
        const int bw = s < h ? b1 : br;
        const int wd = bit >> 5, sh = bit & 31;
        uint32_t v = row[wd] >> sh;
        if (sh + bw > 32 && wd + 1 < W) v |= row[wd + 1] << (32 - sh);
        c = (int)(v & ((1u << bw) - 1u));
      }
      ids[r][s] = (uint8_t)c;
    }
    __syncthreads();
    for (int e = tid; e < TILE * DP; e += 256) {
      const int r = e / DP, j = e % DP;
      float v = 0.f;
      if (r < rows && j < d)
        v = a.scale[seq * a.seq_stride + a.tok_off + t0 + r] * polar_coord(a.t, s_trig, ids[r], j);
      yh[r][j] = v;
    }
    for (int e = tid; e < TILE * a.mp; e += 256) {
      const int r = e / a.mp, j = e % a.mp;
      float sv = 0.f;
      if (r < rows && j < a.m) {
        const int64_t row = seq * a.seq_stride + a.tok_off + t0 + r;
        const uint32_t w = a.sign[(row * a.sign_pitch >> 2) + (j >> 5)];
        sv = ((w >> (j & 31)) & 1u) ? a.rnorm[row] : -a.rnorm[row];
      }
      sg[r][j] = sv;
    }
    __syncthreads();
    // X_hat = Yh Pi + Sg (c S Pi): wave w owns output columns 32 w .. 32 w + 31
    for (int cb = wave; cb < DP / 32; cb += 4) {
      f32x16 acc = {};
      const int col = 32 * cb + (lane & 31);
      for (int kk = 0; kk < KS; ++kk) {
        const int k = 2 * kk + (lane >> 5);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(yh[lane & 31][k], a.rot[(int64_t)k * a.dp + col], acc, 0, 0, 0);
      }
      if (a.m > 0) {
        for (int kk = 0; kk < a.mp / 2; ++kk) {
          const int k = 2 * kk + (lane >> 5);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sg[lane & 31][k], a.sprot[(int64_t)k * a.dp + col], acc, 0, 0,
                                                     0);
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) s_out[8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)][col] = acc[v];
    }
    __syncthreads();
    for (int e = tid; e < rows * d; e += 256) {
      const int r = e / d, j = e % d;
      const int64_t o = (seq * a.n_tok + t0 + r) * d + j;
      const float v = s_out[r][j];
      if (a.out_dt == TQ_F32) static_cast<float*>(a.out)[o] = v;
      else if (a.out_dt == TQ_BF16) {
        uint32_t u = __float_as_uint(v);
        u += 0x7FFFu + ((u >> 16) & 1u);
        static_cast<uint16_t*>(a.out)[o] = (uint16_t)(u >> 16);
      } else {
        static_cast<_Float16*>(a.out)[o] = (_Float16)v;
      }
    }
    __syncthreads();
  }
}

PolarTables tables_of(const tq_codebook* cb) {
  PolarTables t{};
  t.d = cb->p.d;
  t.levels = cb->pq.levels;
  t.b1 = cb->pq.b1;
  t.br = cb->pq.br;
  t.field_bits = cb->pq.field_bits;
  for (int i = 0; i < kPolarMaxLevels + 2; ++i) {
    t.cent_off[i] = cb->pq.cent_off[i];
    t.bnd_off[i] = cb->pq.bnd_off[i];
  }
  t.trig = cb->dev.ptrig;
  t.bnd = cb->dev.pbnd;
  return t;
}

template <int DP>
hipError_t launch_pq_dt(const PQArgs& a, tq_dtype dt, int grid, hipStream_t st) {
  switch (dt) {
    case TQ_F32: hipLaunchKernelGGL((k_polar_quantize<DP, TQ_F32>), dim3(grid), dim3(kPolarThreads), 0, st, a); break;
    case TQ_BF16: hipLaunchKernelGGL((k_polar_quantize<DP, TQ_BF16>), dim3(grid), dim3(kPolarThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((k_polar_quantize<DP, TQ_F16>), dim3(grid), dim3(kPolarThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

bool polar_quantize_supported(const tq_codebook* cb) {
  const int d = cb->p.d;
  return cb->pq.polar && d >= 4 && d <= 128 && (d & (d - 1)) == 0 && cb->p.qjl_m <= 128 &&
         cb->pq.levels <= kPolarMaxLevels;
}

hipError_t launch_polar_quantize(const tq_codebook* cb, const QuantJob& job, hipStream_t stream) {
  PQArgs a{};
  a.x = job.x;
  a.n_tok = job.n_tok;
  a.tok_off = job.tok_offset;
  a.first_block = job.tok_offset / TILE;
  const int64_t last_block = (job.tok_offset + job.n_tok - 1) / TILE;
  a.tiles_per_seq = last_block - a.first_block + 1;
  a.n_tiles = a.tiles_per_seq * job.n_seq;
  a.m = cb->p.qjl_m;
  a.t = tables_of(cb);
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
  const int grid = (int)(a.n_tiles < 2048 ? a.n_tiles : 2048);
  ProfileScope prof(TQ_KERNEL_QUANTIZE, stream);
  switch (cb->dp) {
    case 32: return launch_pq_dt<32>(a, job.dt, grid, stream);
    case 64: return launch_pq_dt<64>(a, job.dt, grid, stream);
    default: return launch_pq_dt<128>(a, job.dt, grid, stream);
  }
}

hipError_t launch_polar_dequantize(const tq_codebook* cb, const DequantJob& job, hipStream_t stream) {
  PDArgs a{};
  a.idx = static_cast<const uint8_t*>(job.codes.idx);
  a.sign = static_cast<const uint32_t*>(job.codes.sign);
  a.scale = job.codes.scale;
  a.rnorm = job.codes.rnorm;
  a.idx_pitch = job.codes.idx_row_bytes;
  a.sign_pitch = job.codes.sign_row_bytes;
  a.seq_stride = job.codes.seq_stride;
  a.n_tok = job.n_tok;
  a.tok_off = job.tok_offset;
  a.n_seq = job.n_seq;
  a.tiles_per_seq = (job.n_tok + TILE - 1) / TILE;
  a.n_tiles = a.tiles_per_seq * job.n_seq;
  a.m = cb->p.qjl_m;
  a.mp = cb->mp;
  a.dp = cb->dp;
  a.t = tables_of(cb);
  a.rot = cb->dev.rot;
  a.sprot = cb->dev.sprot;
  a.out = job.out;
  a.out_dt = job.dt;
  const int grid = (int)(a.n_tiles < 2048 ? a.n_tiles : 2048);
  ProfileScope prof(TQ_KERNEL_DEQUANTIZE, stream);
  switch (cb->dp) {
    case 32: hipLaunchKernelGGL((k_polar_dequantize<32>), dim3(grid), dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((k_polar_dequantize<64>), dim3(grid), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((k_polar_dequantize<128>), dim3(grid), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace tq
