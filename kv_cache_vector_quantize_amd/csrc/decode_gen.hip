// Decode attention from packed codes for the shapes the d = 128 kernels of
// decode.hip do not take: any head dimension 3 <= d <= 256, scalar key and
// value codes of 1..8 bits, sketches of up to 256 rows.
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog), "如何实现 TurboQuant" item 1
// and "专业提示": the query is rotated once and the attention dot products are
// taken from the stored indices; "第二阶段" supplies the QJL correction.  The
// computation, the split of the context and the partial records are those of
// decode.hip, and so is the use of v_mfma_f32_16x16x32_bf16 with bf16 hi/lo
// operands; only the operand layouts are general:
//  1. k_gprologue, one workgroup per row (batch, KV head, <= 8 query heads):
//     q~ = Pi_K q' and t = sqrt(pi/2)/m S_K Pi_K q' in fp32 (q' = sm_scale
//     log2(e) q), written as B operands: the query operand of MFMA u holds,
//     in lane group g4, coordinates g4 dp/4 + 4u .. + 3 of the 8 queries (hi
//     parts in columns 0-7, lo parts in 8-15, each value twice, facing the hi
//     and lo of a centroid); the sketch operand of MFMA c holds sketch rows
//     32c + 8 g4 .. + 7 (hi / lo columns).
//  2. k_gsplit<BK, BIG, WV>, 8 waves per workgroup (BIG: d > 128, up to 16
//     query MFMAs and output blocks; WV: value codes over 4 bits, whose
//     tile32 share per lane is twice as large), each wave a chunk of the row in
//     32-token tiles of two 16-token blocks.  Key logits: a lane holds the
//     key bits of its token's coordinates g4 dp/4 .. (g4 + 1) dp/4 - 1 in
//     registers (BK is a template parameter, so the fields of MFMA u sit at
//     constant offsets), each field indexes an LDS table of bf16 hi | lo;
//     the sketch term: each byte of sign bits indexes a table of eight bf16
//     +-1.  Online softmax in base 2.  Weights x values: the tile32 block is
//     staged in the wave's LDS slot; a lane cuts the eight value fields of
//     its coordinate and token slots from two 32-bit windows.  The waves'
//     partials merge in LDS; one record per workgroup and query slot.
//  3. k_gcombine, one workgroup per (row, query slot): log-sum-exp merge of
//     the workgroup records in a fixed order, then out = Pi_V^T o~ / l.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kGWaves = 8;                    // waves per split workgroup
constexpr int kGMaxD = 256;                   // largest head dimension
constexpr int kGMaxM = 256;                   // largest sketch
constexpr int kGNu = kGMaxD / 16;             // query MFMAs per block at most
constexpr int kGNs = kGMaxM / 32;             // sketch MFMAs per block at most
constexpr int kGTab = 256;                    // centroid table entries (8 bits)
constexpr int kGBlkMax = 64 * 16 * 8;         // tile32 block bytes at d = 256, 8 bits
constexpr int kGSlot = kGBlkMax + 16;         // a wave's value slot (+ slack for the last window)
constexpr int kGMerge = kGWaves * 8 * kGMaxD * 4;         // partials of all waves
constexpr int kGLds = kGWaves * kGSlot > kGMerge ? kGWaves * kGSlot : kGMerge;
constexpr int kGMaxWg = 1024;                 // workgroup records per row
// operand dwords per row: query [dp/16][64 lanes][4], then sketch [8][64][4]
constexpr int kGQop = kGNu * 256, kGTop = kGNs * 256;
__host__ __device__ inline int64_t grow_dwords(int dp) { return (int64_t)(dp / 16) * 256 + kGTop; }

__device__ inline uint32_t bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// ------------------------------------------------------------ 1. prologue

struct GPArgs {
  const void* q;
  int qdt;
  int Hq, Hkv, g, qgroups;
  int d, dp, m, mp;
  float qscale;            // sm_scale * log2(e)
  const float* rotT;       // [dp][dp], rotT[k][i] = Pi_K[i][k], zero-padded
  const float* sprotT;     // [dp][mp], sqrt(pi/2)/m (S_K Pi_K)[j][k] at [k][j], or null
  uint32_t* qop;           // [rows][grow_dwords(dp)]
};

__global__ void __launch_bounds__(256) k_gprologue(GPArgs a) {
  __shared__ float qs[8][kGMaxD];
  __shared__ float qt[8][kGMaxD + 1];
  __shared__ float tt[8][kGMaxM + 1];
  const int row = blockIdx.x;
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int tid = threadIdx.x;
  for (int e = tid; e < 8 * kGMaxD; e += 256) {
    const int c = e / kGMaxD, k = e % kGMaxD;
    const int jq = qg * 8 + c;
    float v = 0.f;
    if (k < a.d && jq < a.g) {
      const int64_t off = ((int64_t)b * a.Hq + (int64_t)h * a.g + jq) * a.d + k;
      if (a.qdt == TQ_F32) v = static_cast<const float*>(a.q)[off];
      else if (a.qdt == TQ_BF16) v = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.q)[off] << 16);
      else v = (float)static_cast<const _Float16*>(a.q)[off];
      v *= a.qscale;
    }
    qs[c][k] = v;
  }
  __syncthreads();
  if (tid < a.dp) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < a.d; ++k) {
      const float r = a.rotT[(int64_t)k * a.dp + tid];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(r, qs[c][k], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) qt[c][tid] = tid < a.d ? acc[c] : 0.f;
  }
  if (tid < a.mp) {
    float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (a.m > 0) {
      for (int k = 0; k < a.d; ++k) {
        const float r = a.sprotT[(int64_t)k * a.mp + tid];
#pragma unroll
        for (int c = 0; c < 8; ++c) tv[c] = fmaf(r, qs[c][k], tv[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) tt[c][tid] = tid < a.m ? tv[c] : 0.f;
  }
  __syncthreads();
  uint32_t* dst = a.qop + (int64_t)row * grow_dwords(a.dp);
  // query operand: MFMA u, lane (col, g4), dword p = coordinate
  // g4 dp/4 + 4u + p, the hi (col < 8) or lo (col >= 8) part twice
  const int nu = a.dp / 16, q4 = a.dp / 4;
  for (int e = tid; e < nu * 256; e += 256) {
    const int u = e >> 8, lane = (e >> 2) & 63, p = e & 3;
    const int col = lane & 15, g4 = lane >> 4;
    const float x = qt[col & 7][g4 * q4 + 4 * u + p];
    const uint32_t hi = bf16_rne(x);
    const uint32_t v = col < 8 ? hi : bf16_rne(x - __uint_as_float(hi << 16));
    dst[e] = v | (v << 16);
  }
  // sketch operand: MFMA c, lane (col, g4), dword p = sketch rows
  // 32c + 8 g4 + 2p and + 1, hi or lo parts
  const int ns = a.mp / 32;
  for (int e = tid; e < ns * 256; e += 256) {
    const int c = e >> 8, lane = (e >> 2) & 63, p = e & 3;
    const int col = lane & 15, g4 = lane >> 4;
    const int j = 32 * c + 8 * g4 + 2 * p;
    uint32_t v[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float x = tt[col & 7][j + k];
      const uint32_t hi = bf16_rne(x);
      v[k] = col < 8 ? hi : bf16_rne(x - __uint_as_float(hi << 16));
    }
    dst[nu * 256 + e] = v[0] | (v[1] << 16);
  }
}

// ------------------------------------------------------------ 2. split

struct GSArgs {
  const uint32_t* qop;
  const char* kidx;
  const char* ksign;       // null without a sketch
  const float* kscale;
  const float* krnorm;
  int64_t k_pitch, ks_pitch, k_stride;
  const char* vidx;
  const float* vscale;
  int64_t v_stride;
  const float* kcent;      // [2^bk]
  const float* vcent;      // [2^bv]
  int lk, lv;
  const int32_t* seq_lens;
  int64_t n_ctx;
  int Hq, Hkv, g, qgroups;
  int d, dp, m, bv, g16;
  int blk_bytes;           // tile32 block bytes: 64 * g16 * bv
  int chunk, n_parts, n_wg;
  float* part_o;           // [rows][n_wg][8][dp]
  float* part_ml;          // [rows][n_wg][8][2]
  float* logits;           // [B][Hq][n_ctx] or null
  const int32_t* table;    // paged pools, as in decode.hip
  int64_t max_pages, n_pages;
  int psh;
};

// Bits [off, off + w) of the little-endian words wd (compile-time offsets).
template <int NW>
__device__ inline uint32_t kfield(const uint32_t (&wd)[NW], int off, int w) {
  const int i = off >> 5, s = off & 31;
  uint32_t v;
  if (s + w <= 32 || i + 1 >= NW) v = wd[i] >> s;
  else v = __builtin_amdgcn_alignbit(wd[i + 1], wd[i], s);
  return v & ((1u << w) - 1u);
}

// BIG: d > 128 (up to 16 query MFMAs and coordinate blocks); otherwise d <= 128
// (up to 8), which leaves the registers to load each tile one tile ahead.
template <int BK, bool BIG, bool WV>
__global__ void __launch_bounds__(64 * kGWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) k_gsplit(GSArgs a) {
  constexpr int NU = BIG ? kGNu : kGNu / 2;   // query MFMAs per block / coordinate blocks, at most
  constexpr int KW = NU * BK / 8;             // key dwords of a lane's coordinate slice (dp/4 fields)
  __shared__ __align__(16) uint32_t s_kt[kGTab];     // bf16 hi | lo << 16 of key centroid e
  __shared__ __align__(16) uint32_t s_vt[kGTab];     // the same for value centroids
  // codes of <= 4 bits: entry a | b << bits holds the table entries of a and b
  // (two coordinates of a key, two token slots of a value)
  __shared__ __align__(16) uint2 s_kp[BK <= 4 ? 256 : 1];
  __shared__ __align__(16) uint2 s_vp[256];
  __shared__ __align__(16) u32x4 s_sgn[256];         // byte -> eight bf16 +-1
  __shared__ __align__(16) uint32_t s_op[kGQop + kGTop];   // query operands, sketch operands at kGQop
  __shared__ __align__(16) char s_work[kGLds];
  __shared__ __align__(16) float s_sc[kGWaves][96];  // per wave: kscale[32], rnorm[32], vscale[32]
  __shared__ float s_M[kGWaves][8], s_l[kGWaves][8];
  const int tid = threadIdx.x;
  auto hilo = [](const float* cent, int n, int e) {   // bf16 hi | lo << 16 of centroid e (0 past n)
    const float c = e < n ? cent[e] : 0.f;
    const uint32_t hi = bf16_rne(c);
    return hi | (bf16_rne(c - __uint_as_float(hi << 16)) << 16);
  };
  for (int i = tid; i < kGTab; i += 64 * kGWaves) {
    s_kt[i] = hilo(a.kcent, a.lk, i);
    s_vt[i] = hilo(a.vcent, a.lv, i);
    if constexpr (BK <= 4) {
      if (i < (1 << (2 * BK)))
        s_kp[i] = make_uint2(hilo(a.kcent, a.lk, i & ((1 << BK) - 1)), hilo(a.kcent, a.lk, i >> BK));
    }
    if (a.bv <= 4 && i < (1 << (2 * a.bv)))
      s_vp[i] = make_uint2(hilo(a.vcent, a.lv, i & ((1 << a.bv) - 1)), hilo(a.vcent, a.lv, i >> a.bv));
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = (((i >> (2 * p)) & 1) ? 0x3F80u : 0xBF80u) | ((((i >> (2 * p + 1)) & 1) ? 0x3F80u : 0xBF80u) << 16);
    s_sgn[i] = u32x4{w[0], w[1], w[2], w[3]};
  }
  {
    const int nu = a.dp / 16, ns = (a.m + 31) / 32;
    const uint32_t* src = a.qop + (int64_t)blockIdx.y * grow_dwords(a.dp);
    for (int i = tid; i < nu * 256; i += 64 * kGWaves) s_op[i] = src[i];
    for (int i = tid; i < ns * 256; i += 64 * kGWaves) s_op[kGQop + i] = src[nu * 256 + i];
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int part = blockIdx.x * kGWaves + wave;
  const int row = blockIdx.y;
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const bool paged = a.table != nullptr;
  const int64_t seq = paged ? h : bh;
  int64_t n_valid = a.n_ctx;
  if (a.seq_lens) {
    const int64_t lb = a.seq_lens[b];
    n_valid = lb < 0 ? 0 : (lb < a.n_ctx ? lb : a.n_ctx);
  }
  const int64_t t_begin = (int64_t)part * a.chunk;
  int64_t t_end = t_begin + a.chunk;
  if (t_end > n_valid) t_end = n_valid;
  if (part >= a.n_parts) t_end = t_begin;

  const int nu = a.dp / 16, ns = (a.m + 31) / 32, ndb = a.dp / 16;
  // this lane's key slice: coordinates g4 dp/4 .. + dp/4 - 1 start at bit
  // sb of the row; nkw dwords from dword kd0 hold it, shifted down by ksh
  const int sb = g4 * (a.dp / 4) * BK;
  const int kd0 = sb >> 5, ksh = sb & 31;
  const int nkw = (ksh + (a.dp / 4) * BK + 31) >> 5;
  const char* kbase = a.kidx + seq * a.k_stride * a.k_pitch;
  const char* sbase = ns ? a.ksign + seq * a.k_stride * a.ks_pitch : nullptr;
  const int64_t vblk0 = seq * (a.v_stride >> 5);
  char* s_v = s_work + wave * kGSlot;
  const uint32_t* s_v32 = reinterpret_cast<const uint32_t*>(s_v);
  float* stage = &s_sc[wave][0];
  // value fields of coordinate 16 db + c16: token slots e = 0..7 (tokens
  // 4 g4 + e % 4 + 16 (e / 4)) are 8 consecutive fields from bit
  // vp0 + 8 bv db of the block
  const int vp0 = (16 * g4 + c16) * a.g16 * 8 * a.bv;

  auto phys = [&](int64_t pos) -> int64_t {
    if (!paged) return pos;
    int64_t lp = pos >> a.psh;
    lp = lp < a.max_pages ? lp : a.max_pages - 1;
    int64_t pg = a.table[(int64_t)b * a.max_pages + lp];
    pg = pg < 0 ? 0 : (pg >= a.n_pages ? a.n_pages - 1 : pg);
    return (pg << a.psh) | (pos & ((1LL << a.psh) - 1));
  };

  float M = -INFINITY, l = 0.f;
  f32x4 acc_o[NU];
#pragma unroll
  for (int db = 0; db < NU; ++db) acc_o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Raw data of one tile: key slices and sign words of tokens c16 and
  // 16 + c16, the token scalars of lane % 32, the lane's share of the tile32
  // block.  The next tile's loads go in flight while the current one is
  // computed (past the last tile they repeat it, so the count of loads in
  // flight is the same on every pass): as soon as the current one's are
  // consumed, except with 16 output accumulators and key codes over 4 bits or
  // value codes over 4 bits (registers): then after the key and sketch
  // products, when the current key words are dead.
  // 16-byte words of a tile32 block per lane: g16 bv / 16 (WV: value codes
  // of more than 4 bits)
  constexpr int VB = WV ? NU / 2 : NU / 4;
  constexpr bool kEarly = !BIG || (!WV && BK <= 4);
  struct Raw {
    uint32_t kw[2][KW + 1];
    uint32_t sw[2][kGNs];
    float ks, kr, vs;
    u32x4 vb[VB];
  };
  const int nvb = a.blk_bytes >> 4;
  const int kp32 = (int)a.k_pitch, sp32 = (int)a.ks_pitch;     // <= 256 and 32 bytes
  auto load = [&](Raw& R, const int64_t t0) {
    const int lim = t_end - t0 < 32 ? (int)(t_end - t0) : 32;
    const int64_t pt0 = phys(t0);       // the tile's 32 positions lie in one page
    // the tile's first row (uniform), then 32-bit lane offsets
    const char* kt = kbase + pt0 * a.k_pitch + 4 * kd0;
    const char* st = ns ? sbase + pt0 * a.ks_pitch : nullptr;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int tk = 16 * blk + c16 < lim ? 16 * blk + c16 : lim - 1;
      const uint32_t* kr = reinterpret_cast<const uint32_t*>(kt + (uint32_t)(tk * kp32));
#pragma unroll
      for (int i = 0; i <= KW; ++i) R.kw[blk][i] = i < nkw ? kr[i] : 0u;
      const uint32_t* sr = ns ? reinterpret_cast<const uint32_t*>(st + (uint32_t)(tk * sp32)) : nullptr;
#pragma unroll
      for (int c = 0; c < kGNs; ++c) R.sw[blk][c] = c < ns ? sr[c] : 0u;
    }
    const int tk = (lane & 31) < lim ? (lane & 31) : lim - 1;
    const int64_t r = seq * a.k_stride + pt0;
    R.ks = a.kscale[r + tk];
    R.kr = ns ? a.krnorm[r + tk] : 0.f;
    R.vs = a.vscale[seq * a.v_stride + pt0 + tk];
    const u32x4* src = reinterpret_cast<const u32x4*>(a.vidx + (vblk0 + (pt0 >> 5)) * (int64_t)a.blk_bytes);
#pragma unroll
    for (int j = 0; j < VB; ++j) R.vb[j] = lane + 64 * j < nvb ? src[lane + 64 * j] : u32x4{0u, 0u, 0u, 0u};
  };

  const int64_t ntile = t_end > t_begin ? (t_end - t_begin + 31) / 32 : 0;
  const int64_t t_last = t_begin + 32 * (ntile - 1);
  Raw R;
  if (ntile > 0) load(R, t_begin);
  for (int64_t it = 0; it < ntile; ++it) {
    const int64_t t0 = t_begin + 32 * it;
    const int64_t t_next = t0 + 32 < t_last ? t0 + 32 : t_last;
    const int lim = t_end - t0 < 32 ? (int)(t_end - t0) : 32;
    // ---- consume the tile: scalars and the value block into the wave's
    // LDS slots, key slices shifted to bit 0, sign words
    stage[lane] = lane < 32 ? R.ks : R.kr;
    if (lane < 32) stage[64 + lane] = R.vs;
    {
      u32x4* dv = reinterpret_cast<u32x4*>(s_v);
#pragma unroll
      for (int j = 0; j < VB; ++j)
        if (lane + 64 * j < nvb) dv[lane + 64 * j] = R.vb[j];
    }
    uint32_t kw[2][KW + 1], sw[2][kGNs];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < KW; ++i) kw[blk][i] = __builtin_amdgcn_alignbit(R.kw[blk][i + 1], R.kw[blk][i], ksh);
      kw[blk][KW] = 0u;
#pragma unroll
      for (int c = 0; c < kGNs; ++c) sw[blk][c] = R.sw[blk][c];
    }
    if constexpr (kEarly) load(R, t_next);

    __builtin_amdgcn_s_setprio(1);
    // ---- S^T = K^ Q~^T (16 tokens x 16 columns per block)
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 accq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // (fully unrolled with guards, so every register array index is a constant)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u < nu) {
        const u32x4 qb = *reinterpret_cast<const u32x4*>(&s_op[(u * 64 + lane) * 4]);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          u32x4 ka;
          if constexpr (BK <= 4) {
            const uint2 e0 = s_kp[kfield<KW + 1>(kw[blk], 4 * u * BK, 2 * BK)];
            const uint2 e1 = s_kp[kfield<KW + 1>(kw[blk], (4 * u + 2) * BK, 2 * BK)];
            ka = u32x4{e0.x, e0.y, e1.x, e1.y};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) ka[e] = s_kt[kfield<KW + 1>(kw[blk], (4 * u + e) * BK, BK)];
          }
          acc[blk] = mfma(ka, qb, acc[blk]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kGNs; ++c) {
      if (c < ns) {
        const u32x4 tb = *reinterpret_cast<const u32x4*>(&s_op[kGQop + (c * 64 + lane) * 4]);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          accq[blk] = mfma(s_sgn[(sw[blk][c] >> (8 * g4)) & 0xFFu], tb, accq[blk]);
      }
    }
    if constexpr (!kEarly) load(R, t_next);
    // logits (base 2): the scales per column, then hi + lo columns
    float lg[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const f32x4 ks = *reinterpret_cast<const f32x4*>(stage + 16 * blk + 4 * g4);
      const f32x4 kr = *reinterpret_cast<const f32x4*>(stage + 32 + 16 * blk + 4 * g4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float u = ks[r] * acc[blk][r];
        if (ns) u = fmaf(kr[r], accq[blk][r], u);
        lg[blk][r] = u + dpp_ror8(u);
      }
    }
    if (lim < 32) {                     // the tile's tokens past the end of the range
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * blk + 4 * g4 + r >= lim) lg[blk][r] = -INFINITY;
    }
    if (a.logits && c16 < 8 && qg * 8 + c16 < a.g) {
      float* dst = a.logits + ((int64_t)b * a.Hq + (int64_t)h * a.g + qg * 8 + c16) * a.n_ctx + t0;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tt = 16 * blk + 4 * g4 + r;
          if (tt < lim) dst[tt] = lg[blk][r] * kLn2;
        }
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- online softmax (base 2); a column's maximum over the tile's tokens
    float tm = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                     fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    if (tm > M) {                       // the tile holds a valid token, so tm > -inf
      const float al = __builtin_amdgcn_exp2f(M - tm);    // 0 while M = -inf
      l *= al;
#pragma unroll
      for (int db = 0; db < NU; ++db) acc_o[db] *= al;
      M = tm;
    }
    const f32x4 vs0 = *reinterpret_cast<const f32x4*>(stage + 64 + 4 * g4);
    const f32x4 vs1 = *reinterpret_cast<const f32x4*>(stage + 80 + 4 * g4);
    // weights of the lane's token slots e (tokens 4 g4 + e % 4 + 16 (e / 4)),
    // each twice: the bf16-truncated weight in columns < 8, the truncated
    // remainder in the others (about 2^-16 of the weight left out).  Tokens
    // past the range have p = 0 and the finite scale of a token in it.
    const float sel_lo = c16 >= 8 ? 1.f : 0.f;
    u32x4 pop[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(lg[blk][r] - M);   // 0 for -inf
        l += p;
        const float w = p * (blk == 0 ? vs0[r] : vs1[r]);
        const float x = fmaf(-sel_lo, __uint_as_float(__float_as_uint(w) & 0xFFFF0000u), w);
        pop[blk][r] = __builtin_amdgcn_perm(__float_as_uint(x), __float_as_uint(x), 0x03020302u);
      }
    __builtin_amdgcn_s_setprio(1);
    // ---- O^T += V^ P^T, coordinates 16 db + c16
#pragma unroll
    for (int db = 0; db < NU; ++db) {
      if (db >= ndb) continue;
      const int p0 = vp0 + 8 * a.bv * db;
      const uint32_t w0 = __builtin_amdgcn_alignbit(s_v32[(p0 >> 5) + 1], s_v32[p0 >> 5], p0 & 31);
      u32x4 va0, va1;
      if constexpr (!WV) {
        // all 8 fields in one window, read as pairs
        const int b2 = 2 * a.bv;
        const uint2 e0 = s_vp[__builtin_amdgcn_ubfe(w0, 0, b2)], e1 = s_vp[__builtin_amdgcn_ubfe(w0, b2, b2)];
        const uint2 e2 = s_vp[__builtin_amdgcn_ubfe(w0, 2 * b2, b2)], e3 = s_vp[__builtin_amdgcn_ubfe(w0, 3 * b2, b2)];
        va0 = u32x4{e0.x, e0.y, e1.x, e1.y};
        va1 = u32x4{e2.x, e2.y, e3.x, e3.y};
      } else {
        const int p1 = p0 + 4 * a.bv;
        const uint32_t w1 = __builtin_amdgcn_alignbit(s_v32[(p1 >> 5) + 1], s_v32[p1 >> 5], p1 & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          va0[e] = s_vt[__builtin_amdgcn_ubfe(w0, e * a.bv, a.bv)];
          va1[e] = s_vt[__builtin_amdgcn_ubfe(w1, e * a.bv, a.bv)];
        }
      }
      acc_o[db] = mfma(va0, pop[0], acc_o[db]);
      acc_o[db] = mfma(va1, pop[1], acc_o[db]);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // positions of this wave's range that no tile covered (beyond len_b)
  if (a.logits && part < a.n_parts) {
    int64_t to = t_begin + a.chunk;
    if (to > a.n_ctx) to = a.n_ctx;
    const int64_t from = t_end > t_begin ? t_end : t_begin;
    const int nq = a.g - qg * 8 < 8 ? a.g - qg * 8 : 8;
    for (int c = 0; c < nq; ++c) {
      float* dst = a.logits + ((int64_t)b * a.Hq + (int64_t)h * a.g + qg * 8 + c) * a.n_ctx;
      for (int64_t t = from + lane; t < to; t += 64) dst[t] = -INFINITY;
    }
  }

  // ---- wave partials -> LDS, then one record per workgroup (fixed order)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();
  float (*s_o)[8][kGMaxD] = reinterpret_cast<float (*)[8][kGMaxD]>(s_work);
#pragma unroll
  for (int db = 0; db < NU; ++db) {
    if (db >= ndb) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float o = acc_o[db][r] + dpp_ror8(acc_o[db][r]);
      const int i = 16 * db + 4 * g4 + r;
      if (c16 < 8) s_o[wave][c16][i] = i < a.d ? o : 0.f;
    }
  }
  if (lane < 8) {
    s_M[wave][lane] = M;
    s_l[wave][lane] = l;
  }
  __syncthreads();
  const int64_t rec0 = ((int64_t)row * a.n_wg + blockIdx.x) * 8;
  for (int e = tid; e < 8 * a.dp; e += 64 * kGWaves) {
    const int c = e / a.dp, i = e % a.dp;
    float Mx = s_M[0][c];
#pragma unroll
    for (int wv = 1; wv < kGWaves; ++wv) Mx = fmaxf(Mx, s_M[wv][c]);
    float ov = 0.f, ls = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < kGWaves; ++wv) {
        if (s_M[wv][c] == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f(s_M[wv][c] - Mx);
        ov += sc * s_o[wv][c][i];
        ls += sc * s_l[wv][c];
      }
    }
    a.part_o[(rec0 + c) * a.dp + i] = ov;
    if (i == 0) {
      a.part_ml[(rec0 + c) * 2 + 0] = Mx;
      a.part_ml[(rec0 + c) * 2 + 1] = ls;
    }
  }
}

// ------------------------------------------------------------ 3. combine

struct GCArgs {
  const float* part_o;
  const float* part_ml;
  const float* rotV;       // [dp][dp] row-major Pi_V, zero-padded
  int Hq, Hkv, g, qgroups, n_wg;
  int d, dp;
  float* out;              // [B][Hq][d]
};

__global__ void __launch_bounds__(256) k_gcombine(GCArgs a) {
  __shared__ float scl[kGMaxWg];
  __shared__ float ov[kGMaxD];
  __shared__ float red[2][4];
  const int c = blockIdx.x, row = blockIdx.y;
  const int qg = row % a.qgroups;
  const int jq = qg * 8 + c;
  if (jq >= a.g) return;                       // uniform over the workgroup
  const int bh = row / a.qgroups;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t base = (int64_t)row * a.n_wg * 8 + c;   // record of workgroup p: base + 8 p
  float Mx = -INFINITY;
  for (int p = tid; p < a.n_wg; p += 256) Mx = fmaxf(Mx, a.part_ml[(base + 8 * p) * 2]);
  Mx = wave_max(Mx);
  if (lane == 0) red[0][wv] = Mx;
  __syncthreads();
  Mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float ls = 0.f;
  for (int p = tid; p < a.n_wg; p += 256) {
    const float Mp = a.part_ml[(base + 8 * p) * 2];
    const float lp = a.part_ml[(base + 8 * p) * 2 + 1];
    const float f = (Mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mp - Mx);
    scl[p] = f;
    ls += f * lp;
  }
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) ls += __shfl_xor(ls, k);
  if (lane == 0) red[1][wv] = ls;
  __syncthreads();
  if (tid < a.dp) {
    float acc = 0.f;
    for (int p = 0; p < a.n_wg; ++p) acc = fmaf(scl[p], a.part_o[(base + 8 * p) * a.dp + tid], acc);
    const float l = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
    ov[tid] = acc * (l > 0.f ? 1.0f / l : 0.f);
  }
  __syncthreads();
  if (tid < a.d) {
    float r = 0.f;
    for (int i = 0; i < a.d; ++i) r = fmaf(a.rotV[(int64_t)i * a.dp + tid], ov[i], r);
    a.out[((int64_t)b * a.Hq + (int64_t)h * a.g + jq) * a.d + tid] = r;
  }
}

template <int BK>
void launch_gsplit(const GSArgs& a, dim3 grid, hipStream_t st) {
  const bool wv = a.bv > 4;
  if (a.dp > 128) {
    if (wv) hipLaunchKernelGGL((k_gsplit<BK, true, true>), grid, dim3(64 * kGWaves), 0, st, a);
    else hipLaunchKernelGGL((k_gsplit<BK, true, false>), grid, dim3(64 * kGWaves), 0, st, a);
  } else {
    if (wv) hipLaunchKernelGGL((k_gsplit<BK, false, true>), grid, dim3(64 * kGWaves), 0, st, a);
    else hipLaunchKernelGGL((k_gsplit<BK, false, false>), grid, dim3(64 * kGWaves), 0, st, a);
  }
}

}  // namespace

bool decode_generic_supported(const tq_codebook* kcb, const tq_codebook* vcb) {
  if (kcb->pq.polar || vcb->pq.polar) return false;
  const int d = kcb->p.d;
  return d == vcb->p.d && d >= 1 && d <= kGMaxD && kcb->p.qjl_m <= kGMaxM && kcb->p.bits >= 1 &&
         kcb->p.bits <= 8 && vcb->p.bits >= 1 && vcb->p.bits <= 8;
}

int64_t decode_generic_row_bytes(int d) { return grow_dwords(pad32(d)) * 4; }

hipError_t launch_decode_generic(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, tq_dtype qdt,
                                 const DecodePlan& plan, const tq_codes& k, const tq_codes& v,
                                 const int32_t* seq_lens, float sm_scale, float* out, float* logits, void* ws,
                                 hipStream_t stream, const PageMap& pm) {
  char* w = static_cast<char*>(ws);
  uint32_t* qop = reinterpret_cast<uint32_t*>(w + plan.off_qop);
  float* part_o = reinterpret_cast<float*>(w + plan.off_part_o);
  float* part_ml = reinterpret_cast<float*>(w + plan.off_part_ml);
  if (plan.rows == 0) return hipSuccess;
  if (plan.n_wg > kGMaxWg) return hipErrorInvalidValue;
  const int d = kcb->p.d, dp = pad32(d);

  GPArgs pa{};
  pa.q = q; pa.qdt = qdt;
  pa.Hq = (int)plan.Hq; pa.Hkv = (int)plan.Hkv; pa.g = plan.g; pa.qgroups = plan.qgroups;
  pa.d = d; pa.dp = dp; pa.m = kcb->p.qjl_m; pa.mp = kcb->mp;
  pa.qscale = sm_scale * kLog2e;
  pa.rotT = kcb->dev.rotT;
  pa.sprotT = kcb->dev.sprotT;
  pa.qop = qop;
  hipLaunchKernelGGL(k_gprologue, dim3((unsigned)plan.rows), dim3(256), 0, stream, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (plan.n_parts > 0) {
    GSArgs sa{};
    sa.qop = qop;
    sa.kidx = static_cast<const char*>(k.idx);
    sa.ksign = static_cast<const char*>(k.sign);
    sa.kscale = k.scale;
    sa.krnorm = k.rnorm;
    sa.k_pitch = k.idx_row_bytes;
    sa.ks_pitch = k.sign_row_bytes;
    sa.k_stride = k.seq_stride;
    sa.vidx = static_cast<const char*>(v.idx);
    sa.vscale = v.scale;
    sa.v_stride = v.seq_stride;
    sa.kcent = kcb->dev.cent;
    sa.vcent = vcb->dev.cent;
    sa.lk = kcb->L; sa.lv = vcb->L;
    sa.seq_lens = seq_lens;
    sa.n_ctx = plan.n_ctx;
    sa.Hq = (int)plan.Hq; sa.Hkv = (int)plan.Hkv; sa.g = plan.g; sa.qgroups = plan.qgroups;
    sa.d = d; sa.dp = dp; sa.m = kcb->p.qjl_m; sa.bv = vcb->p.bits;
    sa.g16 = (d + 15) / 16;
    sa.blk_bytes = 64 * sa.g16 * sa.bv;
    sa.chunk = plan.chunk;
    sa.n_parts = plan.n_parts;
    sa.n_wg = plan.n_wg;
    sa.part_o = part_o;
    sa.part_ml = part_ml;
    sa.logits = logits;
    sa.table = pm.table;
    sa.max_pages = pm.max_pages;
    sa.n_pages = pm.n_pages;
    sa.psh = 5 + pm.ppb_shift;
    if (pm.table && plan.page_tokens != (32 << pm.ppb_shift)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)plan.n_wg, (unsigned)plan.rows);
    ProfileScope prof(TQ_KERNEL_DECODE_SPLIT, stream);
    switch (kcb->p.bits) {
      case 1: launch_gsplit<1>(sa, grid, stream); break;
      case 2: launch_gsplit<2>(sa, grid, stream); break;
      case 3: launch_gsplit<3>(sa, grid, stream); break;
      case 4: launch_gsplit<4>(sa, grid, stream); break;
      case 5: launch_gsplit<5>(sa, grid, stream); break;
      case 6: launch_gsplit<6>(sa, grid, stream); break;
      case 7: launch_gsplit<7>(sa, grid, stream); break;
      default: launch_gsplit<8>(sa, grid, stream); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  GCArgs ca{};
  ca.part_o = part_o;
  ca.part_ml = part_ml;
  ca.rotV = vcb->dev.rot;
  ca.Hq = (int)plan.Hq; ca.Hkv = (int)plan.Hkv; ca.g = plan.g; ca.qgroups = plan.qgroups;
  ca.n_wg = plan.n_wg;
  ca.d = d; ca.dp = dp;
  ca.out = out;
  hipLaunchKernelGGL(k_gcombine, dim3(8, (unsigned)plan.rows), dim3(256), 0, stream, ca);
  return hipGetLastError();
}

}  // namespace tq
