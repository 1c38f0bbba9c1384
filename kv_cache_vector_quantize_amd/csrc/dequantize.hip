// Vectors back from their codes (gfx950).
//
// Page "6倍KV缓存压缩零精度损失：谷歌TurboQuant技术如何提升智能体运行效率",
// 三、工程实现 item 1 (a compress / decompress pair), with the arithmetic of page
// "什么是TurboQuant？…" 工作原理 > 第一阶段 items 1-2 and 第二阶段：QJL 残差校正
// written out in the original domain:
//   x_hat = Pi^T (scale c[idx]) + rnorm Pi^T sqrt(pi/2)/m S^T (2 sign - 1).
//
// d = 128, qjl_m <= 128 (k_dq128).  A workgroup of four waves loops over
// tiles of 32 positions of one sequence (tile32-aligned in absolute
// position).  Wave w forms output coordinates 32w .. 32w + 31 of the tile's
// vectors as D[coordinate][vector] with v_mfma_f32_32x32x16_bf16:
//   A  = rows 32w.. of Pi^T in bf16 hi + lo (registers, loaded once),
//   B  = c[idx] of the 32 vectors in bf16 hi + lo,
//   hi.hi + hi.lo + lo.hi per k-step (the dropped lo.lo is ~2^-18);
//   A' = rows 32w.. of sqrt(pi/2)/m (S Pi)^T in hi + lo, column j pre-scaled
//        by 2^(127 - 2^(j % 8)),
//   B' = the sign bits left where they lie as bf16 {0, 2^(2^e - 127)}, e = j % 8,
//   so every product is exact in the scaling and, with the column sums cs,
//   sum_j A'[k][j] (2 sign_j - 1) = 2 (A' B')[k] - cs[k].
// The contraction index is permuted: k-step s, lane half h, element j is
// input coordinate (or sketch row) 64h + 8s + j, so a lane's codes for two
// consecutive steps are one contiguous run of its row.  B is the same for
// the four waves: wave w builds steps 2w and 2w + 1 (pair-table lookups)
// into an LDS stage of the next tile while the current tile's stage feeds
// the MFMAs, one barrier per tile.
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
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int TILE = 32;

struct DQArgs {
  const uint8_t* idx;
  const uint32_t* sign;
  const float* scale;
  const float* rnorm;
  int64_t idx_pitch, sign_pitch, seq_stride;
  int64_t n_tok, tok_off, first_block;
  int tiles_per_seq, n_tiles;
  int n_seqs, step_q, step_r;    // k_dq128: sequences; grid stride / tiles_per_seq and its remainder
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

// Workgroup barrier that orders LDS only: the waves' global stores need not
// complete before it (a plain __syncthreads() waits for them).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// LDS of one k_dq128 workgroup: two staged tiles of B operands, two staged
// tile32 blocks, each wave's output block (32 vectors x 32 coordinates,
// rows padded) and the centroid table held as COPIES interleaved copies
// (entry e of copy c at byte e * ENT * COPIES + c * ENT; lane l reads copy
// l % COPIES) so that random reads of one pass spread over the banks.  The
// copy count keeps a workgroup within 53 KB (three per CU) for 16-bit
// output and 80 KB (two per CU) for fp32 output.
template <int B, bool T32, bool O32>
struct DqLds {
  static constexpr bool PAIR = B <= 4;
  static constexpr int ESH = PAIR ? 3 : 2;                    // log2 bytes per entry
  static constexpr int TABB = (PAIR ? (1 << (2 * B)) : (1 << B)) << ESH;
  static constexpr int STAGE = 2 * 8 * 2 * 64 * 16;
  // A tile32 block holds four token groups of 32 B dwords each; staged, each
  // group is followed by one pad dword so that the four groups (read together
  // by the lanes of one instruction) start in different banks.
  static constexpr int BLKW = 128 * B;                        // dwords of a tile32 block
  static constexpr int BLKP = BLKW + 8;                       // + group pads, + a straddling read
  static constexpr int BLK = T32 ? 2 * BLKP * 4 : 0;
  static constexpr int OROW = O32 ? 36 : 20;                  // dwords per staged output row
  static constexpr int OST = 4 * 32 * OROW * 4;
  static constexpr int AVAIL = (O32 ? 80 : 53) * 1024 - STAGE - BLK - OST;
  static constexpr int CSH = TABB * 32 <= AVAIL ? 5 : TABB * 16 <= AVAIL ? 4 : TABB * 8 <= AVAIL ? 3
                           : TABB * 4 <= AVAIL ? 2 : TABB * 2 <= AVAIL ? 1 : 0;
  static constexpr int COPIES = 1 << CSH;
};

template <int B, bool T32, bool QJL, bool O32>
__global__ void __launch_bounds__(256) k_dq128(DQArgs a) {
  using L = DqLds<B, T32, O32>;
  constexpr bool PAIR = L::PAIR;
  constexpr int NLD = (B + 1) / 2;                  // row layout: dwords holding a lane's 16 codes
  constexpr int NBL = (L::BLKW + 255) / 256;        // tile32: dwords a thread stages per block
  __shared__ __align__(16) uint4 s_B[2][8][2][64];  // [stage][k-step][hi, lo][lane]
  __shared__ __align__(16) char s_tab[L::TABB * L::COPIES];
  __shared__ __align__(16) uint32_t s_blk[T32 ? 2 : 1][T32 ? L::BLKP : 4];
  __shared__ __align__(16) uint32_t s_o[4][32 * L::OROW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, hl = lane >> 5;
  {
    constexpr int EW = 1 << (L::ESH - 2);           // dwords per entry
    uint32_t* dst = reinterpret_cast<uint32_t*>(s_tab);
    for (int i = tid; i < L::TABB * L::COPIES / 4; i += 256)
      dst[i] = a.tab[(i >> (L::ESH - 2 + L::CSH)) * EW + (i & (EW - 1))];
  }
  const uint32_t laneoff = (uint32_t)(lane & (L::COPIES - 1)) << L::ESH;

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

  // Tile t of this workgroup's sequence t0, t0 + S, ... as (sequence, tile
  // within the sequence), advanced by S without a division; tiles past the
  // last repeat it, so every pass issues the same loads.
  struct Tk {
    int seq, r;
  };
  auto advance = [&](Tk& k) __attribute__((always_inline)) {
    k.seq += a.step_q;
    k.r += a.step_r;
    if (k.r >= a.tiles_per_seq) {
      k.r -= a.tiles_per_seq;
      ++k.seq;
    }
  };
  auto locate = [&](Tk k, int& seq, int64_t& blk) __attribute__((always_inline)) {
    const bool past = k.seq >= a.n_seqs;
    seq = past ? a.n_seqs - 1 : k.seq;
    blk = a.first_block + (past ? a.tiles_per_seq - 1 : k.r);
  };
  auto row_of = [&](int seq, int64_t blk) __attribute__((always_inline)) {
    const int64_t p = blk * TILE + c32;
    const int64_t pc = p < a.tok_off ? a.tok_off : (p >= a.tok_off + a.n_tok ? a.tok_off + a.n_tok - 1 : p);
    return (int64_t)seq * a.seq_stride + pc;
  };
  // per-lane scalars of a tile: scale, residual norm, sign bytes 8hl .. 8hl + 7
  struct Sc {
    float sc, rn;
    uint32_t sg[2];
  };
  auto load_sc = [&](Sc& S, Tk k) __attribute__((always_inline)) {
    int seq;
    int64_t blk;
    locate(k, seq, blk);
    const int64_t row = row_of(seq, blk);
    S.sc = a.scale[row];
    S.rn = 0.f;
    S.sg[0] = S.sg[1] = 0u;
    if constexpr (QJL) {
      S.rn = a.rnorm[row];
      const uint32_t* sr = a.sign + ((row * a.sign_pitch) >> 2);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int wi = 2 * hl + i;
        const uint32_t v = sr[wi < a.sw ? wi : 0];
        S.sg[i] = wi < a.sw ? v : 0u;
      }
    }
  };
  // raw codes of a tile: row layout, this lane's coordinates 64hl + 16w ..
  // + 15 (bits from (64hl + 16w) B, dword aligned down); tile32, this
  // thread's share of the block
  struct Raw {
    uint32_t w[T32 ? NBL : NLD];
  };
  auto load_raw = [&](Raw& R, Tk k) __attribute__((always_inline)) {
    int seq;
    int64_t blk;
    locate(k, seq, blk);
    if constexpr (!T32) {
      const uint32_t* ir = reinterpret_cast<const uint32_t*>(a.idx + row_of(seq, blk) * a.idx_pitch);
      const int d0 = ((64 * hl + 16 * wave) * B) >> 5;
#pragma unroll
      for (int i = 0; i < NLD; ++i) R.w[i] = ir[d0 + i];
    } else {
      const uint32_t* bsrc = reinterpret_cast<const uint32_t*>(a.idx) +
                             ((int64_t)seq * (a.seq_stride / TILE) + blk) * (int64_t)L::BLKW;
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        const int k = tid + 256 * i;
        R.w[i] = bsrc[k < L::BLKW ? k : L::BLKW - 1];
      }
    }
  };
  auto stage_raw = [&](const Raw& R, int sb) __attribute__((always_inline)) {
    if constexpr (T32) {
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        const int k0 = tid + 256 * i, k = k0 < L::BLKW ? k0 : L::BLKW - 1;
        s_blk[sb][k + k / (32 * B)] = R.w[i];
      }
    }
  };
  // hi and lo dwords of codes (c0, c1): {hi(c0) | hi(c1) << 16, lo(c0) | lo(c1) << 16}
  auto lookup2 = [&](uint32_t c0, uint32_t c1) __attribute__((always_inline)) {
    if constexpr (PAIR) {
      const uint32_t pe = c0 | (c1 << B);
      return *reinterpret_cast<const uint2*>(s_tab + ((pe << (L::ESH + L::CSH)) | laneoff));
    } else {
      const uint32_t t0 = *reinterpret_cast<const uint32_t*>(s_tab + ((c0 << (L::ESH + L::CSH)) | laneoff));
      const uint32_t t1 = *reinterpret_cast<const uint32_t*>(s_tab + ((c1 << (L::ESH + L::CSH)) | laneoff));
      return make_uint2(__builtin_amdgcn_perm(t1, t0, 0x05040100u), __builtin_amdgcn_perm(t1, t0, 0x07060302u));
    }
  };
  // B operands of k-steps 2w, 2w + 1 of one tile into stage sbuf
  auto build = [&](const Raw& R, int rb, int sbuf) __attribute__((always_inline)) {
    constexpr uint32_t MASK = (1u << B) - 1u;
    uint32_t code[2][8];
    if constexpr (!T32) {
      // the lane's 16 B bits start 16 bits into its first dword for odd B
      // on odd waves; shift them down to bit 0
      uint32_t v[NLD];
      if constexpr (B % 2 == 1) {
        const uint32_t sh = (uint32_t)(wave & 1) * 16u;
#pragma unroll
        for (int i = 0; i + 1 < NLD; ++i) v[i] = __builtin_amdgcn_alignbit(R.w[i + 1], R.w[i], sh);
        v[NLD - 1] = R.w[NLD - 1] >> sh;
      } else {
#pragma unroll
        for (int i = 0; i < NLD; ++i) v[i] = R.w[i];
      }
#pragma unroll
      for (int ls = 0; ls < 2; ++ls)
#pragma unroll
        for (int j = 0; j < 8; ++j) code[ls][j] = reg_bits<NLD>(v, (8 * ls + j) * B, B);
    } else {
      // token tt of the tile sits in record group G = (tt % 16) / 4, slot
      // es = tt % 4 + 4 (tt / 16); coordinate i = 64hl + 8s + j is record
      // r = 16G + 8(s % 2) + j, coordinate group jj = 4hl + s / 2, at bit
      // ((8 r + jj) 8 + es) B of the block, i.e. in token group G's staged
      // segment (which starts at dword 32 B G + G)
      const uint32_t* blk = s_blk[rb];
      const int G = (c32 & 15) >> 2, es = (c32 & 3) + 4 * (c32 >> 4), jj = 4 * hl + wave;
      const int lb = (1024 * G + 8 * jj + es) * B;
      const uint32_t* bp = blk + (lb >> 5) + G;
      const uint32_t sh = (uint32_t)(lb & 31);
#pragma unroll
      for (int ls = 0; ls < 2; ++ls)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int o = 16 * B * ls + 2 * B * j;
          uint32_t v = bp[o];
          if constexpr (32 % B != 0) v = __builtin_amdgcn_alignbit(bp[o + 1], v, sh);
          else v >>= sh;
          code[ls][j] = v & MASK;
        }
    }
#pragma unroll
    for (int ls = 0; ls < 2; ++ls) {
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint2 t = lookup2(code[ls][2 * q], code[ls][2 * q + 1]);
        bh[q] = t.x;
        bl[q] = t.y;
      }
      s_B[sbuf][2 * wave + ls][0][lane] = make_uint4(bh[0], bh[1], bh[2], bh[3]);
      s_B[sbuf][2 * wave + ls][1][lane] = make_uint4(bl[0], bl[1], bl[2], bl[3]);
    }
  };

  // Output of one tile.  The wave's block (its 32 coordinates of the 32
  // vectors, lane-interleaved as the MFMA leaves it) goes through the wave's
  // own LDS rows, so that each store instruction writes whole 64-byte (16-bit)
  // or 128-byte (fp32) runs of vector rows.  Stores go through a buffer
  // resource based at the tile's first position: rows outside [tok_off,
  // tok_off + n_tok) store to an offset past the resource's range, which the
  // hardware drops, so every pass issues the same stores.
  auto store_tile = [&](const f32x16& acc, const f32x16& accq, const Sc& S, int seq, int64_t blk)
                        __attribute__((always_inline)) {
    constexpr int esz = O32 ? 4 : 2;
    char* base = static_cast<char*>(a.out) + ((int64_t)seq * a.n_tok + blk * TILE - a.tok_off) * 128 * esz;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, TILE * 128 * esz, 0x00020000);
    const int64_t p0 = blk * TILE;
    uint32_t* so = s_o[wave];
    float x[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[v] = S.sc * acc[v];
      if constexpr (QJL) x[v] = fmaf(S.rn, 2.f * accq[v] - cs[v], x[v]);
    }
    // element 4g + r: coordinate 32w + 8g + 4hl + r of vector c32
    if constexpr (O32) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint4*>(so + c32 * L::OROW + 8 * g + 4 * hl) =
            make_uint4(__float_as_uint(x[4 * g]), __float_as_uint(x[4 * g + 1]), __float_as_uint(x[4 * g + 2]),
                       __float_as_uint(x[4 * g + 3]));
      // store i: vector 8i + lane / 8, coordinates 4 (lane % 8) .. + 3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 8 * i + (lane >> 3), q = lane & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(so + k * L::OROW + 4 * q);
        const bool valid = p0 + k >= a.tok_off && p0 + k < a.tok_off + a.n_tok;
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){v.x, v.y, v.z, v.w}, rs,
                                               valid ? (k * 128 + 32 * wave + 4 * q) * 4 : 0x7FFFFFF0, 0, 0);
      }
    } else {
      uint32_t h[8];
      if (a.odt == TQ_BF16) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[2 * i], x[2 * i + 1]}, bf16x2));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[2 * i], x[2 * i + 1]}, f16x2));
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(so + c32 * L::OROW + 4 * g + 2 * hl) = make_uint2(h[2 * g], h[2 * g + 1]);
      // store i: vector 16i + lane / 4, coordinates 8 (lane % 4) .. + 7
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = 16 * i + (lane >> 2), q = lane & 3;
        const uint4 v = *reinterpret_cast<const uint4*>(so + k * L::OROW + 4 * q);
        const bool valid = p0 + k >= a.tok_off && p0 + k < a.tok_off + a.n_tok;
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){v.x, v.y, v.z, v.w}, rs,
                                               valid ? (k * 128 + 32 * wave + 8 * q) * 2 : 0x7FFFFFF0, 0, 0);
      }
    }
  };

  // One tile: raw codes two tiles ahead into rl, scalars one ahead into sn;
  // the next tile's B stage from rb (row) or the staged block; the MFMAs on
  // this tile's stage; the stores.  Two calls per trip alternate the
  // register sets, so no register is copied while its load is in flight.
  Tk k0, k1, k2;
  k0.seq = (int)blockIdx.x / a.tiles_per_seq;
  k0.r = (int)blockIdx.x - k0.seq * a.tiles_per_seq;
  k1 = k0;
  advance(k1);
  k2 = k1;
  advance(k2);
  auto body = [&](int it, Raw& rl, const Raw& rb, const Sc& sc, Sc& sn) __attribute__((always_inline)) {
    const int buf = it & 1;
    load_raw(rl, k2);
    load_sc(sn, k1);
    lds_barrier();     // stage buf complete; stage buf ^ 1 and block buf ^ 1 free / ready
    build(rb, buf ^ 1, buf ^ 1);

    __builtin_amdgcn_s_setprio(1);
    f32x16 acc = {}, accq = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 Bh = __builtin_bit_cast(bf16x8, s_B[buf][s][0][lane]);
      const bf16x8 Bl = __builtin_bit_cast(bf16x8, s_B[buf][s][1][lane]);
      acc = mfma32(ph[s], Bh, acc);
      acc = mfma32(ph[s], Bl, acc);
      acc = mfma32(pl[s], Bh, acc);
      if constexpr (QJL) {
        // sketch rows 64hl + 8s + e': byte s of the lane's eight sign bytes
        const uint32_t sb = (sc.sg[s >> 2] >> (8 * (s & 3))) & 0xFFu;
        const uint32_t x7 = (sb | (sb << 16)) << 7;
        const bf16x8 Bq = __builtin_bit_cast(
            bf16x8, (u32x4){x7 & 0x01000080u, x7 & 0x04000200u, x7 & 0x10000800u, x7 & 0x40002000u});
        accq = mfma32(qh[s], Bq, accq);
        accq = mfma32(ql[s], Bq, accq);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    int seq;
    int64_t blk;
    locate(k0, seq, blk);
    store_tile(acc, accq, sc, seq, blk);
    // the block two tiles ahead into the block stage read at the last build
    stage_raw(rl, buf);
    k0 = k1;
    k1 = k2;
    advance(k2);
  };

  const int n_it = (a.n_tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  Raw ra, rb;
  Sc sa, sb;
  load_raw(rb, k0);
  load_raw(ra, k1);
  load_sc(sa, k0);
  stage_raw(rb, 0);
  stage_raw(ra, 1);
  __syncthreads();   // tables, staged blocks
  build(rb, 0, 0);
  // Nothing outstanding on entry: the counted waits in the loop are then set
  // by its back edge alone (a tile's loads followed by the stores) rather
  // than by the prologue's operand loads.
  __builtin_amdgcn_s_waitcnt(0);
  for (int it = 0; it < n_it; it += 2) {
    body(it, rb, ra, sa, sb);
    if (it + 1 >= n_it) break;
    body(it + 1, ra, rb, sb, sa);
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
template <int B, bool T32, bool QJL, bool O32>
int resident_one() {
  static int per_device[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (per_device[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_dq128<B, T32, QJL, O32>, 256, 0) != hipSuccess || n < 1)
      n = 1;
    per_device[dev] = n;
  }
  return per_device[dev];
}

// launch (grid = 0: return the resident workgroups per CU instead)
template <int B, bool T32, bool QJL, bool O32>
int run_one(const DQArgs& a, int grid, hipStream_t st) {
  if (grid == 0) return resident_one<B, T32, QJL, O32>();
  hipLaunchKernelGGL((k_dq128<B, T32, QJL, O32>), dim3(grid), dim3(256), 0, st, a);
  return 0;
}

template <int B>
int run_b(const DQArgs& a, bool t32, bool qjl, bool o32, int grid, hipStream_t st) {
  if (t32) {
    if (qjl) return o32 ? run_one<B, true, true, true>(a, grid, st) : run_one<B, true, true, false>(a, grid, st);
    return o32 ? run_one<B, true, false, true>(a, grid, st) : run_one<B, true, false, false>(a, grid, st);
  }
  if (qjl) return o32 ? run_one<B, false, true, true>(a, grid, st) : run_one<B, false, true, false>(a, grid, st);
  return o32 ? run_one<B, false, false, true>(a, grid, st) : run_one<B, false, false, false>(a, grid, st);
}

int run_dq128(const DQArgs& a, int bits, bool t32, bool qjl, bool o32, int grid, hipStream_t st) {
  switch (bits) {
    case 1: return run_b<1>(a, t32, qjl, o32, grid, st);
    case 2: return run_b<2>(a, t32, qjl, o32, grid, st);
    case 3: return run_b<3>(a, t32, qjl, o32, grid, st);
    case 4: return run_b<4>(a, t32, qjl, o32, grid, st);
    case 5: return run_b<5>(a, t32, qjl, o32, grid, st);
    case 6: return run_b<6>(a, t32, qjl, o32, grid, st);
    case 7: return run_b<7>(a, t32, qjl, o32, grid, st);
    default: return run_b<8>(a, t32, qjl, o32, grid, st);
  }
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
    const bool t32 = c.layout == TQ_LAYOUT_TILE32, qjl = cb->p.qjl_m > 0, o32 = job.dt == TQ_F32;
    const int res = run_dq128(a, cb->p.bits, t32, qjl, o32, 0, stream);
    const int grid = (int)std::min<int64_t>(a.n_tiles, (int64_t)res * device_cus());
    a.n_seqs = (int)job.n_seq;
    a.step_q = grid / a.tiles_per_seq;
    a.step_r = grid % a.tiles_per_seq;
    run_dq128(a, cb->p.bits, t32, qjl, o32, grid, stream);
  } else {
    a.n_tiles = (int)job.n_seq;       // the generic kernel takes n_seq here
    const int64_t groups = (job.n_seq * job.n_tok + GV - 1) / GV;
    const int grid = (int)std::min<int64_t>(groups, 8LL * device_cus());
    hipLaunchKernelGGL(k_dq_generic, dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tq
