// Decode attention from packed codes for the shapes the d = 128 MFMA kernels
// of decode.hip do not take: any head dimension 3 <= d <= 256, scalar key and
// value codes of 1..8 bits, sketches of up to 256 rows.
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog), "如何实现 TurboQuant" item 1
// and "专业提示": the query is rotated once and the attention dot products are
// taken from the stored indices; "第二阶段" supplies the QJL correction.  The
// computation, the split of the context and the partial records are those of
// decode.hip:
//  1. k_gprologue, one workgroup per row (batch, KV head, <= 8 query heads):
//     q~ = Pi_K q' and t = sqrt(pi/2)/m S_K Pi_K q' in fp32 with
//     q' = sm_scale log2(e) q, stored coordinate-major ([i][8 queries]) so one
//     scalar load brings a coordinate's value for all 8 queries, and sum_j t_j.
//  2. k_gsplit<BK>, 8 waves per workgroup, each wave a chunk of the row in
//     64-token tiles.  Logits with lane = token: each key index goes through
//     an LDS centroid table and meets the 8 query values, read from LDS by
//     all lanes at one address (8 FMAs per coordinate); each sign bit takes
//     one FMA per query against t, and the sketch term is
//     rnorm (2 sum_{sign=1} t - sum t).  Online
//     softmax in base 2.  Weights x values with lane = coordinate (up to 4 per
//     lane): each 32-token tile32 block is staged in the wave's LDS slot and
//     every (token, coordinate) index is read from it.  The waves' partials
//     merge in LDS and each workgroup writes one record per query slot.
//  3. k_gcombine, one workgroup per (row, query slot): log-sum-exp merge of
//     the workgroup records in a fixed order, then out = Pi_V^T o~ / l.
// Every FMA is fp32; the operands are the fp32 centroids and the fp32 q~, t.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kGWaves = 8;                    // waves per split workgroup
constexpr int kGMaxD = 256;                   // largest head dimension
constexpr int kGMaxM = 256;                   // largest sketch
constexpr int kGTab = 256;                    // centroid table entries (8 bits)
constexpr int kGBlkMax = 64 * 16 * 8;         // tile32 block bytes at d = 256, 8 bits
constexpr int kGSlot = kGBlkMax + 16;         // a wave's value staging slot (+1 dword of slack)
constexpr int kGW = 64 * 8 * 4;               // a wave's weights: [64 tokens][8 queries] fp32
constexpr int kGWork = kGWaves * (kGW + kGSlot);          // staging of all waves
constexpr int kGMerge = kGWaves * 8 * kGMaxD * 4;         // partials of all waves
constexpr int kGLds = kGWork > kGMerge ? kGWork : kGMerge;
constexpr int kGMaxWg = 1024;                 // workgroup records per row

// Floats per row of the prologue's output: q~ [dp][8], t [256][8], sum t [8].
__host__ __device__ inline int64_t grow_floats(int dp) { return (int64_t)(dp + kGMaxM) * 8 + 8; }

// ------------------------------------------------------------ 1. prologue

struct GPArgs {
  const void* q;
  int qdt;
  int Hq, Hkv, g, qgroups;
  int d, dp, m, mp;
  float qscale;            // sm_scale * log2(e)
  const float* rotT;       // [dp][dp], rotT[k][i] = Pi_K[i][k], zero-padded
  const float* sprotT;     // [dp][mp], sqrt(pi/2)/m (S_K Pi_K)[j][k] at [k][j], or null
  float* gq;               // [rows][grow_floats(dp)]
};

__global__ void __launch_bounds__(256) k_gprologue(GPArgs a) {
  __shared__ float qs[8][kGMaxD];
  __shared__ float red[4][8];
  const int row = blockIdx.x;
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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
  float* dst = a.gq + (int64_t)row * grow_floats(a.dp);
  if (tid < a.dp) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < a.d; ++k) {
      const float r = a.rotT[(int64_t)k * a.dp + tid];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(r, qs[c][k], acc[c]);
    }
    const bool in = tid < a.d;
    *reinterpret_cast<f32x4*>(dst + 8 * tid) =
        in ? f32x4{acc[0], acc[1], acc[2], acc[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dst + 8 * tid + 4) =
        in ? f32x4{acc[4], acc[5], acc[6], acc[7]} : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (a.m > 0 && tid < a.mp) {
    for (int k = 0; k < a.d; ++k) {
      const float r = a.sprotT[(int64_t)k * a.mp + tid];
#pragma unroll
      for (int c = 0; c < 8; ++c) tv[c] = fmaf(r, qs[c][k], tv[c]);
    }
    if (tid >= a.m) {
#pragma unroll
      for (int c = 0; c < 8; ++c) tv[c] = 0.f;
    }
    float* tr = dst + (int64_t)(a.dp + tid) * 8;
    *reinterpret_cast<f32x4*>(tr) = f32x4{tv[0], tv[1], tv[2], tv[3]};
    *reinterpret_cast<f32x4*>(tr + 4) = f32x4{tv[4], tv[5], tv[6], tv[7]};
  }
  // sum_j t_j per query slot
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float s = tv[c];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
    if (lane == 0) red[wv][c] = s;
  }
  __syncthreads();
  if (tid < 8) dst[(int64_t)(a.dp + kGMaxM) * 8 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// ------------------------------------------------------------ 2. split

struct GSArgs {
  const float* gq;
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

// Bits [off, off + BK) of the little-endian words wd (compile-time offsets).
template <int BK>
__device__ inline uint32_t kfield(const uint32_t (&wd)[BK], int off) {
  const int i = off >> 5, s = off & 31;
  uint32_t v;
  if (s + BK <= 32 || i + 1 >= BK) v = wd[i] >> s;
  else v = __builtin_amdgcn_alignbit(wd[i + 1], wd[i], s);
  return v & ((1u << BK) - 1u);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int BK>
__global__ void __launch_bounds__(64 * kGWaves) k_gsplit(GSArgs a) {
  __shared__ __align__(16) float s_kc[kGTab];
  __shared__ __align__(16) float s_vc[kGTab];
  // the row's q~ [dp][8], t [mp][8] and sum t [8]
  __shared__ __align__(16) float s_q[(kGMaxD + kGMaxM) * 8 + 8];
  __shared__ __align__(16) char s_work[kGLds];
  __shared__ float s_M[kGWaves][8], s_l[kGWaves][8];
  const int tid = threadIdx.x;
  for (int i = tid; i < kGTab; i += 64 * kGWaves) {
    s_kc[i] = i < a.lk ? a.kcent[i] : 0.f;
    s_vc[i] = i < a.lv ? a.vcent[i] : 0.f;
  }
  {
    // q~ and t of the row; every lane of a wave later reads one coordinate's
    // 8 values at one address (a broadcast)
    const float* src = a.gq + (int64_t)blockIdx.y * grow_floats(a.dp);
    const int nqt = (a.dp + 32 * ((a.m + 31) >> 5)) * 8;
    for (int i = tid; i < nqt; i += 64 * kGWaves) s_q[i] = src[i];
    if (tid < 8) s_q[(kGMaxD + kGMaxM) * 8 + tid] = src[(int64_t)(a.dp + kGMaxM) * 8 + tid];
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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

  const float* trow = s_q + a.dp * 8;
  const float* tsum = s_q + (kGMaxD + kGMaxM) * 8;
  const int g32 = a.dp >> 5;
  const int ns = (a.m + 31) >> 5;
  const int nq = a.g - qg * 8 < 8 ? a.g - qg * 8 : 8;
  const char* kbase = a.kidx + seq * a.k_stride * a.k_pitch;
  const char* sbase = ns ? a.ksign + seq * a.k_stride * a.ks_pitch : nullptr;
  const int64_t vblk0 = seq * (a.v_stride >> 5);
  float* s_w = reinterpret_cast<float*>(s_work + wave * (kGW + kGSlot));     // [64][8]
  char* s_v = s_work + wave * (kGW + kGSlot) + kGW;                          // one tile32 block
  const uint32_t vmask = (1u << a.bv) - 1u;
  // value coordinates of this lane: i = lane + 64 r, bit offset of index i of
  // token 0 in a block (coordinates past the block's 16 g16 are clamped and
  // their sums discarded)
  const int nr = (a.dp + 63) >> 6;
  int cib[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int i = lane + 64 * r;
    if (i >= 16 * a.g16) i = 0;
    cib[r] = (((i & 15) * a.g16 + (i >> 4)) * 8) * a.bv;
  }

  auto phys = [&](int64_t pos) -> int64_t {
    if (!paged) return pos;
    int64_t lp = pos >> a.psh;
    lp = lp < a.max_pages ? lp : a.max_pages - 1;
    int64_t pg = a.table[(int64_t)b * a.max_pages + lp];
    pg = pg < 0 ? 0 : (pg >= a.n_pages ? a.n_pages - 1 : pg);
    return (pg << a.psh) | (pos & ((1LL << a.psh) - 1));
  };

  float M[8], l[8], o[8][4];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    M[c] = -INFINITY;
    l[c] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[c][r] = 0.f;
  }

  for (int64_t t0 = t_begin; t0 < t_end; t0 += 64) {
    const int64_t pos = t0 + lane;
    const bool valid = pos < t_end;
    const int64_t pp = phys(valid ? pos : t0);
    // ---- logits (lane = token)
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    {
      const uint32_t* kr = reinterpret_cast<const uint32_t*>(kbase + pp * a.k_pitch);
      uint32_t kw[BK];
#pragma unroll
      for (int j = 0; j < BK; ++j) kw[j] = kr[j];
      for (int gi = 0; gi < g32; ++gi) {
        uint32_t kn[BK];
        const int gn = gi + 1 < g32 ? gi + 1 : gi;
#pragma unroll
        for (int j = 0; j < BK; ++j) kn[j] = kr[gn * BK + j];
        const float* qv = s_q + gi * 256;
        // four coordinates per batch: all their LDS reads are issued before
        // the FMAs that consume them
#pragma unroll
        for (int u0 = 0; u0 < 32; u0 += 4) {
          float cv[4];
          f32x4 q0[4], q1[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            cv[k] = s_kc[kfield<BK>(kw, (u0 + k) * BK)];
            q0[k] = *reinterpret_cast<const f32x4*>(qv + (u0 + k) * 8);
            q1[k] = *reinterpret_cast<const f32x4*>(qv + (u0 + k) * 8 + 4);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(cv[k], q0[k][c], acc[c]);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[4 + c] = fmaf(cv[k], q1[k][c], acc[4 + c]);
          }
        }
#pragma unroll
        for (int j = 0; j < BK; ++j) kw[j] = kn[j];
      }
    }
    float accs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float rn = 0.f;
    if (ns) {
      const uint32_t* sr = reinterpret_cast<const uint32_t*>(sbase + pp * a.ks_pitch);
      rn = a.krnorm[seq * a.k_stride + pp];
      for (int gs = 0; gs < ns; ++gs) {
        const uint32_t sw = sr[gs];
        const float* tv = trow + gs * 256;
#pragma unroll
        for (int j0 = 0; j0 < 32; j0 += 4) {
          f32x4 t0[4], t1[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            t0[k] = *reinterpret_cast<const f32x4*>(tv + (j0 + k) * 8);
            t1[k] = *reinterpret_cast<const f32x4*>(tv + (j0 + k) * 8 + 4);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float f = (float)((sw >> (j0 + k)) & 1u);
#pragma unroll
            for (int c = 0; c < 4; ++c) accs[c] = fmaf(f, t0[k][c], accs[c]);
#pragma unroll
            for (int c = 0; c < 4; ++c) accs[4 + c] = fmaf(f, t1[k][c], accs[4 + c]);
          }
        }
      }
    }
    const float ks = a.kscale[seq * a.k_stride + pp];
    const float vs = a.vscale[seq * a.v_stride + pp];
    float s[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = ks * acc[c];
      if (ns) v = fmaf(rn, fmaf(2.f, accs[c], -tsum[c]), v);
      s[c] = valid ? v : -INFINITY;
    }
    if (a.logits && valid) {
      float* dst = a.logits + ((int64_t)b * a.Hq + (int64_t)h * a.g + qg * 8) * a.n_ctx + pos;
      for (int c = 0; c < nq; ++c) dst[(int64_t)c * a.n_ctx] = s[c] * kLn2;
    }
    // ---- online softmax (base 2); the tile holds at least one valid token
    float w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float tm = wave_max(s[c]);
      if (tm > M[c]) {
        const float al = __builtin_amdgcn_exp2f(M[c] - tm);   // 0 while M = -inf
        M[c] = tm;
        l[c] *= al;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[c][r] *= al;
      }
      const float p = valid ? __builtin_amdgcn_exp2f(s[c] - M[c]) : 0.f;
      l[c] += p;
      w[c] = valid ? p * vs : 0.f;
    }
    *reinterpret_cast<f32x4*>(s_w + lane * 8) = f32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<f32x4*>(s_w + lane * 8 + 4) = f32x4{w[4], w[5], w[6], w[7]};
    // ---- weights x values (lane = coordinate), one 32-token block at a time
    for (int bi = 0; bi < 2; ++bi) {
      const int64_t tb = t0 + 32 * bi;
      if (tb >= t_end) break;
      const int64_t blk = vblk0 + (phys(tb) >> 5);
      const f32x4* src = reinterpret_cast<const f32x4*>(a.vidx + blk * a.blk_bytes);
      f32x4* sv = reinterpret_cast<f32x4*>(s_v);
      for (int e = lane; e < (a.blk_bytes >> 4); e += 64) sv[e] = src[e];
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(s_v);
      const int ntb = t_end - tb < 32 ? (int)(t_end - tb) : 32;
      // two tokens per batch (weights of a token past ntb are 0)
      for (int t = 0; t < ntb; t += 2) {
        f32x4 w0[2], w1[2];
        float cv[2][4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int tk = t + k;
          w0[k] = *reinterpret_cast<const f32x4*>(s_w + (32 * bi + tk) * 8);
          w1[k] = *reinterpret_cast<const f32x4*>(s_w + (32 * bi + tk) * 8 + 4);
          const int tt = (16 * ((tk & 15) >> 2) * a.g16 * 8 + (tk & 3) + 4 * (tk >> 4)) * a.bv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            cv[k][r] = 0.f;
            if (r >= nr) break;
            const int p = cib[r] + tt;
            const uint32_t lo = s32[p >> 5], hi = s32[(p >> 5) + 1];
            cv[k][r] = s_vc[__builtin_amdgcn_alignbit(hi, lo, p & 31) & vmask];
          }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (r >= nr) break;
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c][r] = fmaf(w0[k][c], cv[k][r], o[c][r]);
#pragma unroll
            for (int c = 0; c < 4; ++c) o[4 + c][r] = fmaf(w1[k][c], cv[k][r], o[4 + c][r]);
          }
      }
    }
  }

  // positions of this wave's range that no tile covered (beyond len_b)
  if (a.logits && part < a.n_parts) {
    int64_t to = t_begin + a.chunk;
    if (to > a.n_ctx) to = a.n_ctx;
    const int64_t from = t_end > t_begin ? t_end : t_begin;
    for (int c = 0; c < nq; ++c) {
      float* dst = a.logits + ((int64_t)b * a.Hq + (int64_t)h * a.g + qg * 8 + c) * a.n_ctx;
      for (int64_t t = from + lane; t < to; t += 64) dst[t] = -INFINITY;
    }
  }

  // ---- wave partials -> LDS, then one record per workgroup (fixed order)
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v = l[c];
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) v += __shfl_xor(v, k);
    l[c] = v;
  }
  __syncthreads();
  float (*s_o)[8][kGMaxD] = reinterpret_cast<float (*)[8][kGMaxD]>(s_work);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = lane + 64 * r;
    if (i < a.dp) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s_o[wave][c][i] = i < a.d ? o[c][r] : 0.f;
    }
  }
  if (lane < 8) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (lane == c) { s_M[wave][c] = M[c]; s_l[wave][c] = l[c]; }
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
  hipLaunchKernelGGL(k_gsplit<BK>, grid, dim3(64 * kGWaves), 0, st, a);
}

}  // namespace

bool decode_generic_supported(const tq_codebook* kcb, const tq_codebook* vcb) {
  if (kcb->pq.polar || vcb->pq.polar) return false;
  const int d = kcb->p.d;
  return d == vcb->p.d && d >= 1 && d <= kGMaxD && kcb->p.qjl_m <= kGMaxM && kcb->p.bits >= 1 &&
         kcb->p.bits <= 8 && vcb->p.bits >= 1 && vcb->p.bits <= 8;
}

int64_t decode_generic_row_bytes(int d) { return grow_floats(pad32(d)) * 4; }

hipError_t launch_decode_generic(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, tq_dtype qdt,
                                 const DecodePlan& plan, const tq_codes& k, const tq_codes& v,
                                 const int32_t* seq_lens, float sm_scale, float* out, float* logits, void* ws,
                                 hipStream_t stream, const PageMap& pm) {
  char* w = static_cast<char*>(ws);
  float* gq = reinterpret_cast<float*>(w + plan.off_qop);
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
  pa.gq = gq;
  hipLaunchKernelGGL(k_gprologue, dim3((unsigned)plan.rows), dim3(256), 0, stream, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (plan.n_parts > 0) {
    GSArgs sa{};
    sa.gq = gq;
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
