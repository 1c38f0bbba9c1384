// Decode attention computed from packed codes (gfx950).
//
// Page "什么是TurboQuant？…" (a2a-mcp.org blog), "如何实现 TurboQuant" item 1
// and "专业提示": the query is rotated once and attention dot products are
// taken straight from the stored indices; "第二阶段" supplies the QJL
// correction of the inner product.
//
// Three launches:
//  1. prologue, grid (4, rows), a row = (batch, KV head, group of <= 8 query
//     heads), each workgroup 32 coordinates (and sketch rows) of all the
//     row's query slots: q~ = Pi_K q scaled by sm_scale*log2(e),
//     t = sqrt(pi/2)/m S_K q~, split into bf16 hi + lo
//     and written in the lane order of the B operand of
//     v_mfma_f32_16x16x32_bf16 (columns 0-7 = hi of the 8 queries, 8-15 =
//     lo of the same queries).
//  2. split: a workgroup of 8 waves covers 8 consecutive token chunks of one
//     row; each wave streams 32-token tiles (the next tile's loads in
//     flight) and computes on MFMA
//       S^T = K^ Q~^T   (16 tokens x 16 query columns per block),
//       the QJL term T^ (2 sigma) - sum(t)  (-sum(t) is the accumulator's
//       initial value; each sign bit stays at a bf16 exponent bit, one AND
//       per two signs),
//       O^T += V^ P^T   (in the value codebook's rotated domain),
//     with an online softmax in base 2 whose reference maximum is only moved
//     when a tile exceeds it by more than 2^8.  Code operands come from bf16
//     hi/lo tables in LDS (pair tables, a quad table for 2-bit keys)
//     indexed by packed indices; hi and lo sit next to each other in the
//     contraction dimension (operand dwords hi,lo,hi,lo against a duplicated
//     other operand), so a table read lands directly in the MFMA operand
//     registers.  The 8 waves' partial (max, sum, o~) are merged in LDS and
//     written once per workgroup.
//  3. combine, grid (4, rows): log-sum-exp merge of the workgroups'
//     partials in a fixed order, then out = Pi_V^T o~ / l.
// Other head dimensions, code widths and sketch sizes go to decode_gen.hip.
#include <algorithm>
#include <type_traits>

#include "decode_prologue.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

using prologue::D;
using prologue::QOP_Q;
using prologue::QOP_T;
using prologue::QOP_DWORDS;
using prologue::kSignShift;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float LAZY = 8.0f;           // max moves when a tile exceeds it by 2^8

using prologue::bf16_rne_bits;

__device__ inline float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ inline bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ inline f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ 1. prologue


// A D-row matrix (row-major, `cols` floats per row, cols a multiple of 4 and
// >= 4) is staged into LDS as dst[k][i], columns >= cols zero-filled.  The 16
// loads of a thread are issued together (clamped addresses, no branches) and
// stored once all have landed.
struct Stage {
  f32x4 r[16];
};

__device__ inline void stage_load(Stage& st, const float* src, int cols, int tid) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = tid + 256 * j;
    const int k = e >> 5, i4 = (e & 31) * 4;
    const int ic = i4 < cols ? i4 : cols - 4;
    st.r[j] = *reinterpret_cast<const f32x4*>(src + (int64_t)k * cols + ic);
  }
}

__device__ inline void stage_store(float (*dst)[D], const Stage& st, int cols, int tid) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = tid + 256 * j;
    const int k = e >> 5, i4 = (e & 31) * 4;
    f32x4 v = st.r[j];
    if (i4 >= cols) v = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(&dst[k][i4]) = v;
  }
}

// Grid (4, rows): workgroup (part, row) forms coordinates 32 part .. 32 part
// + 31 of q~ = Pi q' and rows 32 part .. 32 part + 31 of t = sqrt(pi/2)/m
// (S Pi) q' for all 8 query slots of the row (q' = sm_scale log2(e) q):
// exactly the operand dwords of lane group g4 = part.  Only the part's 32
// columns of the two matrices are staged (32 KB, one batch of coalesced
// 16-byte loads); thread (i, c) forms coordinate i of slot c, then the
// workgroup writes its lane group's operand dwords and its share of the
// QJL accumulator offsets.
__global__ void __launch_bounds__(256) k_prologue(PArgs a) {
  prologue::run(a, blockIdx.x, blockIdx.y, true);
}

// ------------------------------------------------------------ 2. split

struct SArgs {
  const uint32_t* qop;
  const uint8_t* kidx;
  const uint32_t* ksign;
  const float* kscale;
  const float* krnorm;
  int64_t k_pitch, ks_pitch, k_stride;
  const uint32_t* vidx;
  const float* vscale;
  int64_t v_stride;
  const uint32_t* ktab;
  const uint32_t* vtab;
  int ktab_dwords, vtab_dwords;
  const int32_t* seq_lens;
  int64_t n_ctx;
  int Hq, Hkv, g, qgroups, m;
  int chunk, n_parts, n_wg;
  float* part_o;     // [rows][n_wg][8][D]
  float* part_ml;    // [rows][n_wg][8][2]
  float* logits;     // [B][Hq][n_ctx] or null
  // paged pools (k_split<..., true>): plane h holds KV head h; logical page
  // i of batch b is page table[b * max_pages + i] (clamped to [0, n_pages))
  // of 2^psh positions
  const int32_t* table;
  int64_t max_pages, n_pages;
  int psh;
};

// Bits [off, off + w) of a little-endian multi-word field (w <= 16).
template <int NW>
__device__ inline uint32_t field(const uint32_t (&wd)[NW], int off, int w) {
  const int i = off >> 5, s = off & 31;
  uint32_t v;
  if (s + w <= 32 || i + 1 >= NW) v = wd[i] >> s;
  else v = __builtin_amdgcn_alignbit(wd[i + 1], wd[i], s);
  return v & ((1u << w) - 1u);
}

// The 32-bit window of a little-endian multi-word field starting at bit off.
template <int NW>
__device__ inline uint32_t window(const uint32_t (&wd)[NW], int off) {
  const int i = off >> 5, s = off & 31;
  if (i + 1 < NW) return __builtin_amdgcn_alignbit(wd[i + 1], wd[i], s);
  return wd[i] >> s;
}

// Byte address in the 2-bit quad key table of the operand of coordinates
// 4u .. 4u + 3 of a lane's key bits, with the lane's copy offset: one byte
// permute.
template <int BK>
__device__ inline uint32_t quad_addr(const uint32_t (&kw)[BK], int u, uint32_t laneoff16) {
  static_assert(BK == 2, "quad tables serve 2-bit keys");
  return __builtin_amdgcn_perm(kw[u >> 2], laneoff16, 0x0C0C0000u | ((4u + (u & 3)) << 8));
}

template <int B>
constexpr int table_entries() { return (B <= 4) ? (1 << (2 * B)) : (1 << B); }

// Random 8-byte reads of one small table from all 64 lanes collide in the LDS
// banks (a read of 8 bytes serves 32 lanes per pass).  A pair table can
// therefore be held as kCopies interleaved copies: entry e of copy c at byte
// e * 256 + c * 8, and lane l reads copy l % 32, so the 32 lanes of a pass
// always hit 32 distinct bank pairs.
constexpr int kWaves = 8;                  // waves per split workgroup
constexpr int kCopies = 32;
constexpr int kCopyBudget = 80 * 1024;     // LDS bytes for the two tables

constexpr int table_entries_rt(int b) { return (b <= 4) ? (1 << (2 * b)) : (1 << b); }
constexpr int plain_bytes(int b) { return (b <= 4) ? table_entries_rt(b) * 8 : table_entries_rt(b) * 4; }

// Polar keys (BK == 0): codes of (b1, br) = (4, 2) at d = 128, seven angle
// levels; the key table holds (cos, sin) of every centroid angle, level 1's
// 16 first, then 4 per higher level.
constexpr int kPolarTrigEntries = 16 + 6 * 4;
constexpr int kPolarKeyDwords = 5;      // code dwords a lane reads per token

// Keys of 2 bits use a quad table: one 16-byte entry per four coordinates
// (an 8-bit index, one byte of the packed row) holds the operand dwords
// {hi, lo} of both coordinate pairs, so one ds_read_b128 lands a whole MFMA
// operand.  The table (4 KB) is held as 16 interleaved copies (entry e of
// copy c at byte e * 256 + c * 16: the 16 lanes of a read pass hit distinct
// banks).  Keys of 3 bits read a pair table whose index is a byte of the key
// bits (see kw3_addr): a 3-bit quad table (64 KB) fits in LDS only once, and
// its random 16-byte reads then collide in the banks.
template <int BK>
struct QuadKeys {
  static constexpr bool on = BK == 2;
  static constexpr int copies = 16;
  static constexpr int bytes = on ? (16 << (4 * BK)) * copies : 0;
};

template <int BK, int BV>
struct SplitLds {
  static constexpr bool VC = BV <= 4 && table_entries_rt(BV) * 8 * kCopies <= kCopyBudget;
  static constexpr int VBYTES = VC ? table_entries_rt(BV) * 8 * kCopies : plain_bytes(BV);
  static constexpr bool KQ = QuadKeys<BK>::on;
  static constexpr bool KW = BK == 3;   // pair table indexed by key-bit windows (256 entries, 32 copies)
  static constexpr bool KC = !KQ && !KW && BK >= 1 && BK <= 4 && VBYTES + table_entries_rt(BK) * 8 * kCopies <= kCopyBudget;
  static constexpr int KBYTES = BK == 0 ? kPolarTrigEntries * 8
                                        : KQ ? QuadKeys<BK>::bytes
                                        : KW ? 256 * 8 * kCopies
                                             : (KC ? table_entries_rt(BK) * 8 * kCopies : plain_bytes(BK));
  static constexpr int OBYTES = kWaves * 8 * D * 4;    // merge buffer, aliases the tables
  static constexpr int RAW = (KBYTES + VBYTES > OBYTES) ? KBYTES + VBYTES : OBYTES;
};

// hi and lo operand dwords of two codes: for B <= 4 entry e = a | b << B is
// the dword pair {hi(c[a]) | hi(c[b]) << 16, lo(c[a]) | lo(c[b]) << 16} (one
// 64-bit read lands both in consecutive registers), read from the lane's copy
// when the table is interleaved; for B > 4 a single-code table holds
// hi | lo << 16.
template <int B, bool COPIED>
__device__ inline uint2 lookup(const char* tab, uint32_t pair, uint32_t laneoff) {
  if constexpr (B <= 4) {
    if constexpr (COPIED) return *reinterpret_cast<const uint2*>(tab + ((pair << 8) | laneoff));
    else return *reinterpret_cast<const uint2*>(tab + (pair << 3));
  } else {
    const uint32_t* t = reinterpret_cast<const uint32_t*>(tab);
    const uint32_t e0 = t[pair & ((1u << B) - 1u)];
    const uint32_t e1 = t[pair >> B];
    return make_uint2(__builtin_amdgcn_perm(e1, e0, 0x05040100u),
                      __builtin_amdgcn_perm(e1, e0, 0x07060302u));
  }
}

// Sign operand dword K (0..15) of a lane's 32 sign bits w (r = w rotated
// left by 8): one bit per bf16 half, left where it lies.  A single set bit at
// position P (7..14) of a half is the normal bf16 2^(2^(P-7) - 127); the
// matching entry of the sketch-query operand is pre-scaled by 2 / that value
// times 2^-kSignShift, so every product is exactly 2 t_j sigma_j 2^-kSignShift.
// Dword K < 8 takes bits 14-K and 30-K of w at P = 14-K; dword K >= 8 takes
// bits 14-K (31 for K = 15) and 30-K through r at P = 22-K.
template <int K>
__device__ inline uint32_t sgn(uint32_t w, uint32_t r) {
  constexpr int P = (K < 8) ? 14 - K : 22 - K;
  constexpr uint32_t m = (1u << P) | (1u << (P + 16));
  return ((K < 8) ? w : r) & m;
}

// Value-code group db (8 token slots of one coordinate) from a lane's tile32
// record of 2*BV dwords.
template <int BV>
__device__ inline uint32_t vgroup(const uint32_t* rec, int db, uint32_t& hi32) {
  hi32 = 0u;
  if constexpr (BV == 4) return rec[db];
  else if constexpr (BV == 2) return rec[db >> 1] >> (16 * (db & 1));
  else if constexpr (BV == 8) { hi32 = rec[2 * db + 1]; return rec[2 * db]; }
  else {   // BV == 3: 24-bit groups
    const int bit = 24 * db, w = bit >> 5, sh = bit & 31;
    if (sh + 24 <= 32) return rec[w] >> sh;
    return __builtin_amdgcn_alignbit(rec[w + 1], rec[w], sh);
  }
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Operand dword pair of two values: {hi(y0) | hi(y1) << 16, lo(y0) |
// lo(y1) << 16}, hi the bf16 rounding of y and lo that of y - hi.
__device__ inline uint2 split_pair(float y0, float y1) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y0, y1}, bf16x2));
  const float r0 = y0 - __uint_as_float(h << 16);
  const float r1 = y1 - __uint_as_float(h & 0xFFFF0000u);
  return make_uint2(h, __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){r0, r1}, bf16x2)));
}

// Key operands of one token's 32 coordinates 32 g4 .. 32 g4 + 31 (the
// lane's subtree of five polar levels) from its polar codes, (b1, br) =
// (4, 2), d = 128: kw[0..1] = level-1 fields of the subtree (4 bits each),
// kw[2] >> sh2 = its 8 level-2 fields, kw[3] >> sh3 its 4 level-3 fields,
// kw[4] the level-4 (at sh4), level-5 (sh5), level-6 (sh6) and level-7 (bit
// 28) fields.  The subtree's radius is the product of the level-7 and
// level-6 factors on its path (cos for a lower child, sin for an upper);
// each level below multiplies a radius by (cos, sin) of its centroid angle.
struct PolarLane {
  int sh2, sh3, sh4, sh5, sh6;
  bool up7, up6;
};

__device__ inline void polar_operands(const uint32_t (&kw)[kPolarKeyDwords], const PolarLane& pl,
                                      const f32x2* tt, uint2 (&ek)[8][2]) {
  const uint32_t w4 = kw[4];
  const f32x2 t7 = tt[36 + ((w4 >> 28) & 3u)];
  const f32x2 t6 = tt[32 + ((w4 >> pl.sh6) & 3u)];
  const float rho = (pl.up7 ? t7.y : t7.x) * (pl.up6 ? t6.y : t6.x);
  const f32x2 t5 = tt[28 + ((w4 >> pl.sh5) & 3u)];
  float r4[2] = {rho * t5.x, rho * t5.y};
  float r3[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const f32x2 t = tt[24 + ((w4 >> (pl.sh4 + 2 * j)) & 3u)];
    r3[2 * j] = r4[j] * t.x;
    r3[2 * j + 1] = r4[j] * t.y;
  }
  const uint32_t w3 = kw[3] >> pl.sh3;
  float r2[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 t = tt[20 + ((w3 >> (2 * j)) & 3u)];
    r2[2 * j] = r3[j] * t.x;
    r2[2 * j + 1] = r3[j] * t.y;
  }
  const uint32_t w2 = kw[2] >> pl.sh2;
  float r1[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f32x2 t = tt[16 + ((w2 >> (2 * j)) & 3u)];
    r1[2 * j] = r2[j] * t.x;
    r1[2 * j + 1] = r2[j] * t.y;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    // level-1 pairs 2u and 2u + 1 give coordinates 4u .. 4u + 3
    const uint32_t w = kw[u >> 2];
    const f32x2 ta = tt[(w >> (8 * (u & 3))) & 15u];
    const f32x2 tb = tt[(w >> (8 * (u & 3) + 4)) & 15u];
    ek[u][0] = split_pair(r1[2 * u] * ta.x, r1[2 * u] * ta.y);
    ek[u][1] = split_pair(r1[2 * u + 1] * tb.x, r1[2 * u + 1] * tb.y);
  }
}

// 3-bit keys: the 16 six-bit pair fields of a lane's 96 key bits (pair j at
// bit 6j) sit at byte 0 or byte 3 of eight 32-bit windows: window
// (j & 3) + 4 (j >> 3) starts at the bit of pair j & 11, and pair j + 4 lies
// 24 bits above pair j.  Seven funnel shifts form them.
__device__ inline void kw3_windows(const uint32_t (&kw)[3], uint32_t (&w)[8]) {
  w[0] = kw[0];
  w[1] = __builtin_amdgcn_alignbit(kw[1], kw[0], 6);
  w[2] = __builtin_amdgcn_alignbit(kw[1], kw[0], 12);
  w[3] = __builtin_amdgcn_alignbit(kw[1], kw[0], 18);
  w[4] = __builtin_amdgcn_alignbit(kw[2], kw[1], 16);
  w[5] = __builtin_amdgcn_alignbit(kw[2], kw[1], 22);
  w[6] = __builtin_amdgcn_alignbit(kw[2], kw[1], 28);
  w[7] = kw[2] >> 2;
}
// Byte address of pair j in the 256-entry pair table, whose index is the
// window byte (the pair's six bits and two bits of the next field; entry e
// holds pair e & 63), with the lane's copy offset: one byte permute.  The
// table is held as 32 interleaved copies like the value table (64 KB).
__device__ inline uint32_t kw3_addr(const uint32_t (&w)[8], int j, uint32_t laneoff) {
  const int wi = (j & 3) + 4 * (j >> 3);
  const uint32_t t = ((j >> 2) & 1) ? 3u : 0u;
  return __builtin_amdgcn_perm(w[wi], laneoff, 0x0C0C0000u | ((4u + t) << 8));
}

// Global loads of one 32-token tile for one lane.
template <int BK, int BV>
struct Tile {
  uint32_t kw[2][BK == 0 ? kPolarKeyDwords : BK];   // key code bits of this lane's token (per 16-token block)
  uint32_t sw[2];       // QJL sign word
  uint32_t vr[2 * BV];  // value record: 8 coordinates x 8 token slots
  float ks, kr, vs;     // per-token scalars of token (lane % 32), staged through LDS
};

template <int BK, int BV, bool QJL, bool PG>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) k_split(SArgs a) {
  using L = SplitLds<BK, BV>;
  constexpr int NT = 64 * kWaves;
  __shared__ __align__(16) char s_raw[L::RAW];              // tables; merge buffer afterwards
  __shared__ __align__(16) float s_sc[kWaves][96];          // per wave: kscale[32], rnorm[32], vscale[32]
  __shared__ float s_M[kWaves][8], s_l[kWaves][8];
  const char* s_kt = s_raw;
  // value table: a key table of >= 64 KB puts it past the reach of a
  // ds_read's immediate offset, so its base is carried in the lane offset
  // (bit 16 up, clear of the entry and copy bits) instead
  constexpr bool kVBaseInLane = L::KBYTES >= 65536 && L::VC;
  static_assert(!kVBaseInLane || L::KBYTES % 65536 == 0, "value table base must be a multiple of 64 KB");
  const char* s_vt = s_raw + (kVBaseInLane ? 0 : L::KBYTES);
  const int tid = threadIdx.x;
  {
    // interleaved copy i of 8-byte entry i / 32 sits at byte 8 i (quad
    // tables: copy i of 16-byte entry i / copies at byte 16 i)
    const uint2* vt = reinterpret_cast<const uint2*>(a.vtab);
    uint2* dv = reinterpret_cast<uint2*>(s_raw + L::KBYTES);
    if constexpr (L::KQ) {
      const uint4* kt = reinterpret_cast<const uint4*>(a.ktab);
      uint4* dk = reinterpret_cast<uint4*>(s_raw);
      for (int i = tid; i < L::KBYTES / 16; i += NT) dk[i] = kt[i / QuadKeys<BK>::copies];
    } else if constexpr (L::KW) {
      const uint2* kt = reinterpret_cast<const uint2*>(a.ktab);
      uint2* dk = reinterpret_cast<uint2*>(s_raw);
      for (int i = tid; i < L::KBYTES / 8; i += NT) dk[i] = kt[(i >> 5) & 63];
    } else {
      const uint2* kt = reinterpret_cast<const uint2*>(a.ktab);
      uint2* dk = reinterpret_cast<uint2*>(s_raw);
      for (int i = tid; i < L::KBYTES / 8; i += NT) dk[i] = kt[L::KC ? (i >> 5) : i];
    }
    for (int i = tid; i < L::VBYTES / 8; i += NT) dv[i] = vt[L::VC ? (i >> 5) : i];
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int part = blockIdx.x * kWaves + wave;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const uint32_t laneoff16 = (uint32_t)(lane & 15) << 4;
  const uint32_t vlaneoff = laneoff | (kVBaseInLane ? (uint32_t)L::KBYTES : 0u);
  const int row = blockIdx.y;
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int64_t seq = PG ? h : bh;                          // code plane: b * Hkv + h, or pool plane h
  int64_t n_valid = a.n_ctx;
  if (a.seq_lens) {
    // lengths outside [0, n_ctx] are a caller error; clamping keeps every
    // tile inside the sequence's planes
    const int64_t lb = a.seq_lens[b];
    n_valid = lb < 0 ? 0 : (lb < a.n_ctx ? lb : a.n_ctx);
  }
  const int64_t t_begin = (int64_t)part * a.chunk;
  int64_t t_end = t_begin + a.chunk;
  if (t_end > n_valid) t_end = n_valid;
  if (part >= a.n_parts) t_end = t_begin;
  // paged: lane i holds the page of logical page lp0 + i; a wave's chunk is
  // whole pages, at most 64 of them
  const int lp0 = PG ? (int)(t_begin >> a.psh) : 0;
  int32_t win = 0;
  if constexpr (PG) {
    int64_t lp = (int64_t)lp0 + lane;
    lp = lp < a.max_pages ? lp : a.max_pages - 1;
    const int32_t pg = a.table[(int64_t)b * a.max_pages + lp];
    win = pg < 0 ? 0 : (pg >= a.n_pages ? (int32_t)(a.n_pages - 1) : pg);
  }

  // query operands (per row): qa[u] = dims 32*g4 + 4u + (0,1,0,1,2,3,2,3)
  const u32x4* qop = reinterpret_cast<const u32x4*>(a.qop + (int64_t)row * QOP_DWORDS);
  bf16x8 qa[8], ta[4];
#pragma unroll
  for (int u = 0; u < 8; ++u) qa[u] = __builtin_bit_cast(bf16x8, qop[u * 64 + lane]);
  if constexpr (QJL) {
#pragma unroll
    for (int c = 0; c < 4; ++c) ta[c] = __builtin_bit_cast(bf16x8, qop[QOP_Q / 4 + c * 64 + lane]);
  }
  float cinit = 0.f;
  if constexpr (QJL) {
    // the prologue's four parts of the offset, summed in a fixed order
    const float* ci = reinterpret_cast<const float*>(a.qop + (int64_t)row * QOP_DWORDS) + QOP_Q + QOP_T + c16;
    cinit = ((ci[0] + ci[16]) + ci[32]) + ci[48];
  }
  const float sel_lo = (c16 >= 8) ? 1.f : 0.f;
  static_assert(kSignShift == 64, "the staged residual norms carry 2^kSignShift");

  float M = -INFINITY, l = 0.f;
  float Meff = 0.f, nhm = 0.f, lazy_thr = -INFINITY;   // see the softmax below
  f32x4 acc_o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc_o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Tile loads are raw buffer loads: one descriptor per plane of the
  // sequence (uniform), a per-lane byte offset that is the same for every
  // tile (VGPR) and the tile's uniform byte offset (SGPR).  Offsets stay below
  // 2^31: the host checks the size of a sequence's planes.
  auto rsrc = [](const void* base) {
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    // (readfirstlane returns int: widen through uint32_t, never by sign extension)
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;    // uniform by construction
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0, (int)0x7FFFFFFF, 0x00020000);
  };
  const auto rk = rsrc(reinterpret_cast<const char*>(a.kidx) + seq * a.k_stride * a.k_pitch);
  constexpr int KW = BK == 0 ? kPolarKeyDwords : BK;
  // byte offset of key code dword i of this lane's token in block 0: BK
  // consecutive dwords at g4 * BK for scalar codes; for polar codes the
  // dwords holding the lane's subtree (see polar_operands)
  int koff[KW];
  PolarLane pl{};
#pragma unroll
  for (int i = 0; i < KW; ++i) {
    int dw = g4 * BK + i;
    if constexpr (BK == 0) {
      const int pd[kPolarKeyDwords] = {2 * g4, 2 * g4 + 1, 8 + (g4 >> 1), 10, 11};
      dw = pd[i];
    }
    koff[i] = c16 * (int)a.k_pitch + 4 * dw;
  }
  if constexpr (BK == 0) {
    pl.sh2 = 16 * (g4 & 1);
    pl.sh3 = 8 * g4;
    pl.sh4 = 4 * g4;
    pl.sh5 = 16 + 2 * g4;
    pl.sh6 = 24 + 2 * (g4 >> 1);
    pl.up7 = g4 >= 2;
    pl.up6 = (g4 & 1) != 0;
  }
  const int kblk1 = 16 * (int)a.k_pitch;
  const auto rs = rsrc(QJL ? reinterpret_cast<const char*>(a.ksign) + seq * a.k_stride * a.ks_pitch
                           : reinterpret_cast<const char*>(a.kidx));
  // sign word g4 of the row; lanes past the row read word 0 (their sketch
  // rows have t = 0 in the query operand, so those bits add nothing)
  const int slane0 = c16 * (int)a.ks_pitch + 4 * (4 * g4 < a.ks_pitch ? g4 : 0);
  const int slane1 = slane0 + 16 * (int)a.ks_pitch;
  constexpr int VBLK = 64 * 8 * BV / 4;                  // dwords per tile32 block (d = 128)
  const auto rv = rsrc(a.vidx + seq * (a.v_stride / 32) * (int64_t)VBLK);
  const int vlane = (16 * g4 + c16) * 2 * BV * 4;
  const auto rks = rsrc(a.kscale + seq * a.k_stride);
  const auto rkr = rsrc(QJL ? a.krnorm + seq * a.k_stride : a.kscale);
  const auto rvs = rsrc(a.vscale + seq * a.v_stride);
  const int sl4 = (lane & 31) * 4;
  float* stage = &s_sc[wave][0];

  auto load = [&](Tile<BK, BV>& T, const int64_t t0) {
    int t = __builtin_amdgcn_readfirstlane((int)t0);
    if constexpr (PG) {
      // the tile's 32 positions lie in one page: map the logical position
      int li = (t >> a.psh) - lp0;
      li = li < 0 ? 0 : (li > 63 ? 63 : li);
      const int pg = __builtin_amdgcn_readlane(win, li);
      t = (pg << a.psh) | (t & ((1 << a.psh) - 1));
    }
    const int kt = t * (int)a.k_pitch;
#pragma unroll
    for (int i = 0; i < KW; ++i) {
      T.kw[0][i] = __builtin_amdgcn_raw_buffer_load_b32(rk, koff[i], kt, 0);
      T.kw[1][i] = __builtin_amdgcn_raw_buffer_load_b32(rk, koff[i] + kblk1, kt, 0);
    }
    T.sw[0] = T.sw[1] = 0u;
    if constexpr (QJL) {
      const int st = t * (int)a.ks_pitch;
      T.sw[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, slane0, st, 0);
      T.sw[1] = __builtin_amdgcn_raw_buffer_load_b32(rs, slane1, st, 0);
    }
    const int vt = (t >> 5) * VBLK * 4;
    if constexpr (BV == 4 || BV == 2 || BV == 8) {
#pragma unroll
      for (int i = 0; i < 2 * BV; i += 4) {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vlane + 4 * i, vt, 0));
        T.vr[i] = v[0]; T.vr[i + 1] = v[1]; T.vr[i + 2] = v[2]; T.vr[i + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2 * BV; i += 2) {
        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
        const u32x2v v = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(rv, vlane + 4 * i, vt, 0));
        T.vr[i] = v[0]; T.vr[i + 1] = v[1];
      }
    }
    T.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, sl4, 4 * t, 0));
    T.kr = QJL ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rkr, sl4, 4 * t, 0)) : 0.f;
    T.vs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, sl4, 4 * t, 0));
  };

  // value operands of coordinate block db (4 lookups = token slot pairs)
  auto vlook = [&](const Tile<BK, BV>& T, const int db, uint2 (&e)[4]) {
    uint32_t fhi;
    const uint32_t f = vgroup<BV>(T.vr, db, fhi);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (BV == 4 && L::VC) {
        // byte q of f is the pair index: (index << 8) | laneoff in one byte permute
        // (bytes 2-3 of the address from the lane offset: the table base)
        const uint32_t addr = __builtin_amdgcn_perm(f, vlaneoff, 0x03020000u | ((4u + q) << 8));
        e[q] = *reinterpret_cast<const uint2*>(s_vt + addr);
      } else {
        uint32_t pr;
        if constexpr (BV == 8) pr = ((q < 2 ? f : fhi) >> (16 * (q & 1))) & 0xFFFFu;
        else pr = (f >> (2 * q * BV)) & ((1u << (2 * BV)) - 1u);
        e[q] = lookup<BV, L::VC>(s_vt, pr, vlaneoff);
      }
    }
  };

  auto compute = [&](const Tile<BK, BV>& T, const int64_t t0, auto partial_tag) {
    constexpr bool partial = decltype(partial_tag)::value;
    // per-token scalars: 96 floats through the wave's LDS slot (the residual
    // norms carry back the power of two the sign operand takes out)
    stage[lane] = (QJL && lane >= 32) ? T.kr * 0x1p64f : T.ks;
    stage[64 + (lane & 31)] = T.vs;
    // ---- key operands of block 0: all 16 lookups in flight (polar codes:
    // the token's coordinates rebuilt from its angle codes)
    uint2 ek[8][2];
    uint4 eq[8];
    if constexpr (L::KQ) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        eq[u] = *reinterpret_cast<const uint4*>(s_kt + quad_addr<BK>(T.kw[0], u, laneoff16));
    } else if constexpr (BK == 0) {
      polar_operands(T.kw[0], pl, reinterpret_cast<const f32x2*>(s_kt), ek);
    } else if constexpr (L::KW) {
      uint32_t w8[8];
      kw3_windows(T.kw[0], w8);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ek[u][0] = *reinterpret_cast<const uint2*>(s_kt + kw3_addr(w8, 2 * u, laneoff));
        ek[u][1] = *reinterpret_cast<const uint2*>(s_kt + kw3_addr(w8, 2 * u + 1, laneoff));
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ek[u][0] = lookup<BK, L::KC>(s_kt, field<BK>(T.kw[0], (4 * u) * BK, 2 * BK), laneoff);
        ek[u][1] = lookup<BK, L::KC>(s_kt, field<BK>(T.kw[0], (4 * u + 2) * BK, 2 * BK), laneoff);
      }
    }
    __builtin_amdgcn_s_setprio(1);
    // ---- QJL sign products (VALU work while the lookups land)
    f32x4 accq[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      accq[blk] = (f32x4){cinit, cinit, cinit, cinit};
      if constexpr (QJL) {
        const uint32_t w = T.sw[blk];
        const uint32_t r = __builtin_amdgcn_alignbit(w, w, 24);     // w rotated left by 8
        accq[blk] = mfma(as_bf16x8(sgn<0>(w, r), sgn<1>(w, r), sgn<2>(w, r), sgn<3>(w, r)), ta[0], accq[blk]);
        accq[blk] = mfma(as_bf16x8(sgn<4>(w, r), sgn<5>(w, r), sgn<6>(w, r), sgn<7>(w, r)), ta[1], accq[blk]);
        accq[blk] = mfma(as_bf16x8(sgn<8>(w, r), sgn<9>(w, r), sgn<10>(w, r), sgn<11>(w, r)), ta[2], accq[blk]);
        accq[blk] = mfma(as_bf16x8(sgn<12>(w, r), sgn<13>(w, r), sgn<14>(w, r), sgn<15>(w, r)), ta[3], accq[blk]);
      }
    }
    // ---- S^T block 0; block 1's lookups replace each consumed pair
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if constexpr (L::KQ) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[0] = mfma(__builtin_bit_cast(bf16x8, eq[u]), qa[u], acc[0]);
        eq[u] = *reinterpret_cast<const uint4*>(s_kt + quad_addr<BK>(T.kw[1], u, laneoff16));
      }
    } else if constexpr (BK == 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc[0] = mfma(as_bf16x8(ek[u][0].x, ek[u][0].y, ek[u][1].x, ek[u][1].y), qa[u], acc[0]);
      polar_operands(T.kw[1], pl, reinterpret_cast<const f32x2*>(s_kt), ek);
    } else if constexpr (L::KW) {
      uint32_t w8[8];
      kw3_windows(T.kw[1], w8);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[0] = mfma(as_bf16x8(ek[u][0].x, ek[u][0].y, ek[u][1].x, ek[u][1].y), qa[u], acc[0]);
        ek[u][0] = *reinterpret_cast<const uint2*>(s_kt + kw3_addr(w8, 2 * u, laneoff));
        ek[u][1] = *reinterpret_cast<const uint2*>(s_kt + kw3_addr(w8, 2 * u + 1, laneoff));
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[0] = mfma(as_bf16x8(ek[u][0].x, ek[u][0].y, ek[u][1].x, ek[u][1].y), qa[u], acc[0]);
        ek[u][0] = lookup<BK, L::KC>(s_kt, field<BK>(T.kw[1], (4 * u) * BK, 2 * BK), laneoff);
        ek[u][1] = lookup<BK, L::KC>(s_kt, field<BK>(T.kw[1], (4 * u + 2) * BK, 2 * BK), laneoff);
      }
    }
    // ---- S^T block 1; the value operands of coordinate blocks 0..3 go in flight
    uint2 ev[4][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (L::KQ) acc[1] = mfma(__builtin_bit_cast(bf16x8, eq[u]), qa[u], acc[1]);
      else acc[1] = mfma(as_bf16x8(ek[u][0].x, ek[u][0].y, ek[u][1].x, ek[u][1].y), qa[u], acc[1]);
      if (u & 1) vlook(T, u >> 1, ev[u >> 1]);
    }
    __builtin_amdgcn_s_setprio(0);
    // lg = logit - Meff (base 2): the scales are applied per column before the
    // hi and lo columns are summed (both columns of a row share the token), and
    // each column carries -Meff/2
    float lg[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const f32x4 ks = *reinterpret_cast<const f32x4*>(stage + 16 * blk + 4 * g4);
      f32x4 kr = ks;
      if constexpr (QJL) kr = *reinterpret_cast<const f32x4*>(stage + 32 + 16 * blk + 4 * g4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float u = fmaf(ks[r], acc[blk][r], nhm);
        if constexpr (QJL) u = fmaf(kr[r], accq[blk][r], u);
        lg[blk][r] = u + dpp_ror8(u);
      }
    }
    if constexpr (partial) {
      const int lim = (int)(t_end - t0);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * blk + 4 * g4 + r >= lim) lg[blk][r] = -INFINITY;
    }
    if (a.logits) {
      if (c16 < 8 && qg * 8 + c16 < a.g) {
        float* dst = a.logits + ((int64_t)b * a.Hq + h * a.g + qg * 8 + c16) * a.n_ctx + t0;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tt = 16 * blk + 4 * g4 + r;
            if (t0 + tt < a.n_ctx) dst[tt] = (lg[blk][r] + Meff) * LN2;
          }
      }
    }

    // ---- online softmax in base 2; the reference maximum M moves only when
    // a logit exceeds it by more than LAZY (then exactly, per query column).
    // lg holds logit - Meff with Meff = M (0 while M = -inf).
    float lm = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                     fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
    if (__builtin_expect(__ballot(lm > lazy_thr) != 0ull, 0)) {
      float mt = fmaxf(lm, __shfl_xor(lm, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float Mn = fmaxf(M, mt + Meff);
      const float alpha = (Mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(M - Mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc_o[db] *= alpha;
      const float Mneff = (Mn == -INFINITY) ? 0.f : Mn;
      const float shift = Meff - Mneff;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[blk][r] += shift;
      M = Mn;
      Meff = Mneff;
      nhm = -0.5f * Meff;
      lazy_thr = (M == -INFINITY) ? -INFINITY : LAZY;
    }
    const f32x4 vs0 = *reinterpret_cast<const f32x4*>(stage + 64 + 4 * g4);
    const f32x4 vs1 = *reinterpret_cast<const f32x4*>(stage + 80 + 4 * g4);
    float w[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(lg[blk][r]);
        l += p;
        w[blk][r] = p * (blk == 0 ? vs0[r] : vs1[r]);
      }
    if constexpr (partial) {
      const int lim = (int)(t_end - t0);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * blk + 4 * g4 + r >= lim) w[blk][r] = 0.f;
    }

    // ---- P^T operand: slot e = token 4*g4 + e (e < 4) or 16 + 4*g4 + e - 4;
    // hi columns take the bf16-truncated weight, lo columns the remainder
    uint32_t pb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = w[q >> 1][2 * (q & 1)], x1 = w[q >> 1][2 * (q & 1) + 1];
      const float v0 = fmaf(-sel_lo, __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u), x0);
      const float v1 = fmaf(-sel_lo, __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u), x1);
      pb[q] = __builtin_amdgcn_perm(__float_as_uint(v1), __float_as_uint(v0), 0x07060302u);
    }
    const bf16x8 pop0 = as_bf16x8(pb[0], pb[0], pb[1], pb[1]);
    const bf16x8 pop1 = as_bf16x8(pb[2], pb[2], pb[3], pb[3]);

    __builtin_amdgcn_s_setprio(1);
    // ---- O^T += V^ P^T (coordinates 16*db + c16); operand dwords
    // (hi, lo, hi, lo) of token slot pairs against duplicated weights; the
    // lookups of block db + 4 replace those of block db
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint2 (&e)[4] = ev[db & 3];
      acc_o[db] = mfma(as_bf16x8(e[0].x, e[0].y, e[1].x, e[1].y), pop0, acc_o[db]);
      acc_o[db] = mfma(as_bf16x8(e[2].x, e[2].y, e[3].x, e[3].y), pop1, acc_o[db]);
      if (db < 4) vlook(T, db + 4, ev[db & 3]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // two-stage pipeline over full tiles: the next tile's loads are in flight
  // while the current one is computed.  Every pass issues them (past the
  // last full tile they repeat that tile), so the number of loads in flight
  // is the same on every path into a tile's computation and its waits only
  // cover the tile's own loads; with a conditional load the count differs
  // between paths and the wait falls back to draining every load.
  const int64_t nfull = (t_end > t_begin) ? (t_end - t_begin) / 32 : 0;
  const int64_t t_last = t_begin + 32 * (nfull - 1);
  int64_t t0 = t_begin;
  Tile<BK, BV> A, Bt;
  if (nfull > 0) load(A, t0);
  for (int64_t i = 0; i < nfull; i += 2) {
    load(Bt, t0 + 32 < t_last ? t0 + 32 : t_last);
    compute(A, t0, std::false_type{});
    t0 += 32;
    if (i + 1 >= nfull) break;
    load(A, t0 + 32 < t_last ? t0 + 32 : t_last);
    compute(Bt, t0, std::false_type{});
    t0 += 32;
  }
  if (t0 < t_end) {
    load(A, t0);
    compute(A, t0, std::true_type{});
    t0 += 32;
  }

  // positions of this wave's range that no tile covered (beyond len_b)
  if (a.logits && part < a.n_parts) {
    int64_t to = t_begin + a.chunk;
    if (to > a.n_ctx) to = a.n_ctx;
    for (int c = 0; c < 8; ++c) {
      if (qg * 8 + c >= a.g) break;
      float* dst = a.logits + ((int64_t)b * a.Hq + h * a.g + qg * 8 + c) * a.n_ctx;
      for (int64_t t = t0 + lane; t < to; t += 64) dst[t] = -INFINITY;
    }
  }

  // ---- wave partial -> LDS (the merge buffer reuses the table space)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();
  float (*s_o)[8][D] = reinterpret_cast<float (*)[8][D]>(s_raw);
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = acc_o[db][r] + dpp_ror8(acc_o[db][r]);
    if (c16 < 8) *reinterpret_cast<f32x4*>(&s_o[wave][c16][16 * db + 4 * g4]) = o;
  }
  if (c16 < 8 && g4 == 0) {
    s_M[wave][c16] = M;
    s_l[wave][c16] = l;
  }
  __syncthreads();

  // ---- merge the waves (fixed order) and write one partial per workgroup
  const int64_t rec0 = ((int64_t)row * a.n_wg + blockIdx.x) * 8;
  for (int e = tid; e < 8 * D; e += NT) {
    const int c = e / D, i = e % D;
    float Mx = s_M[0][c];
#pragma unroll
    for (int wv = 1; wv < kWaves; ++wv) Mx = fmaxf(Mx, s_M[wv][c]);
    float o = 0.f, ls = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        if (s_M[wv][c] == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f(s_M[wv][c] - Mx);
        o += sc * s_o[wv][c][i];
        ls += sc * s_l[wv][c];
      }
    }
    a.part_o[(rec0 + c) * D + i] = o;
    if (i == 0) {
      a.part_ml[(rec0 + c) * 2 + 0] = Mx;
      a.part_ml[(rec0 + c) * 2 + 1] = ls;
    }
  }
}

// ------------------------------------------------------------ 3. combine

struct CArgs {
  const float* part_o;
  const float* part_ml;
  const float* rotV;   // [D][D] row-major Pi_V
  int Hq, Hkv, g, qgroups, n_wg;
  float* out;          // [B][Hq][D]
};

// Grid (4, rows): workgroup (part, row) finishes query slots 2 part and
// 2 part + 1 of the row.  The row's workgroup partials of a slot are merged
// with the usual max / rescale rule: the maximum and the normaliser are
// reduced over the workgroup (thread t visits partials p = t/2 + 128 j of
// local slot t%2), the per-partial factors 2^(M_p - M) go to LDS, and thread
// (i, c) sums coordinate i of local slot c in partial order.  Finally
// out = Pi_V^T o~ / l with Pi_V staged in LDS.
constexpr int kMaxWg = 1024;   // workgroup partials per row; launch_decode rejects plans beyond it

__global__ void __launch_bounds__(256) k_combine(CArgs a) {
  __shared__ __align__(16) float mat[D][D];
  __shared__ __align__(16) float scl[kMaxWg * 2];
  __shared__ __align__(16) float ov[2][D];
  __shared__ float red[2][4][2];
  const int part = blockIdx.x, row = blockIdx.y;
  const int qg = row % a.qgroups;
  const int bh = row / a.qgroups;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t base = (int64_t)row * a.n_wg * 8 + 2 * part;   // record (p, slot) = base + 8p + local slot
  Stage st;
  stage_load(st, a.rotV, D, tid);
  const int cr = tid & 1;
  float Mx = -INFINITY;
  for (int p = tid >> 1; p < a.n_wg; p += 128) Mx = fmaxf(Mx, a.part_ml[(base + 8 * p + cr) * 2]);
#pragma unroll
  for (int o = 2; o < 64; o <<= 1) Mx = fmaxf(Mx, __shfl_xor(Mx, o));
  if (lane < 2) red[0][wv][lane] = Mx;
  __syncthreads();
  Mx = fmaxf(fmaxf(red[0][0][cr], red[0][1][cr]), fmaxf(red[0][2][cr], red[0][3][cr]));
  float ls = 0.f;
  for (int p = tid >> 1; p < a.n_wg; p += 128) {
    const float Mp = a.part_ml[(base + 8 * p + cr) * 2];
    const float lp = a.part_ml[(base + 8 * p + cr) * 2 + 1];
    const float f = (Mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mp - Mx);
    scl[2 * p + cr] = f;
    ls += f * lp;
  }
#pragma unroll
  for (int o = 2; o < 64; o <<= 1) ls += __shfl_xor(ls, o);
  if (lane < 2) red[1][wv][lane] = ls;
  stage_store(mat, st, D, tid);
  __syncthreads();
  const int i = tid & (D - 1), c = tid >> 7;
  float o = 0.f;
  {
    const float* po = a.part_o + (base + c) * D + i;
#pragma unroll 8
    for (int p = 0; p < a.n_wg; ++p) o = fmaf(scl[2 * p + c], po[(int64_t)p * 8 * D], o);
  }
  {
    const float l = ((red[1][0][c] + red[1][1][c]) + red[1][2][c]) + red[1][3][c];
    ov[c][i] = o * (l > 0.f ? 1.0f / l : 0.f);
  }
  __syncthreads();
  float r = 0.f;
#pragma unroll 4
  for (int k = 0; k < D; k += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&ov[c][k]);
#pragma unroll
    for (int u = 0; u < 4; ++u) r = fmaf(mat[k + u][i], v[u], r);
  }
  const int jq = qg * 8 + 2 * part + c;
  if (jq < a.g) a.out[((int64_t)b * a.Hq + h * a.g + jq) * D + i] = r;
}

template <int BK, int BV>
void launch_split_bits(const SArgs& a, bool qjl, dim3 grid, hipStream_t st) {
  if (a.table) {
    if (qjl) hipLaunchKernelGGL((k_split<BK, BV, true, true>), grid, dim3(64 * kWaves), 0, st, a);
    else hipLaunchKernelGGL((k_split<BK, BV, false, true>), grid, dim3(64 * kWaves), 0, st, a);
  } else {
    if (qjl) hipLaunchKernelGGL((k_split<BK, BV, true, false>), grid, dim3(64 * kWaves), 0, st, a);
    else hipLaunchKernelGGL((k_split<BK, BV, false, false>), grid, dim3(64 * kWaves), 0, st, a);
  }
}

template <int BK>
void launch_split_bv(const SArgs& a, int bv, bool qjl, dim3 grid, hipStream_t st) {
  switch (bv) {
    case 2: launch_split_bits<BK, 2>(a, qjl, grid, st); break;
    case 3: launch_split_bits<BK, 3>(a, qjl, grid, st); break;
    case 4: launch_split_bits<BK, 4>(a, qjl, grid, st); break;
    default: launch_split_bits<BK, 8>(a, qjl, grid, st); break;
  }
}

bool bits_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 8; }

}  // namespace

bool decode_supported(const tq_codebook* kcb, const tq_codebook* vcb) {
  if (vcb->pq.polar || kcb->p.d != D || vcb->p.d != D || !bits_ok(vcb->p.bits) || kcb->p.qjl_m > 128) return false;
  if (kcb->pq.polar) return kcb->pq.b1 == 4 && kcb->pq.br == 2;
  return bits_ok(kcb->p.bits);
}

DecodePlan plan_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_ctx, int d, int page_tokens) {
  DecodePlan p{};
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.n_ctx = n_ctx; p.d = d;
  p.page_tokens = page_tokens;
  p.g = Hkv > 0 ? (int)(Hq / Hkv) : 0;
  p.qgroups = (p.g + 7) / 8;
  p.rows = B * Hkv * p.qgroups;
  // one round of 8-wave workgroups on each of the 256 CUs (one workgroup per
  // CU at a time): against two rounds of half-length chunks this measured 2%
  // faster at a 128K context, with half the partials to combine
  const int64_t target_waves = 2048;
  int64_t parts = p.rows > 0 ? (target_waves + p.rows - 1) / p.rows : 1;
  if (parts < 1) parts = 1;
  int64_t chunk = (n_ctx + parts - 1) / parts;
  chunk = (chunk + 31) / 32 * 32;
  if (chunk < 32) chunk = 32;
  if (page_tokens > 0) {
    // whole pages per wave, at most 64 (the page window a wave holds)
    chunk = (chunk + page_tokens - 1) / page_tokens * page_tokens;
    if (chunk > 64LL * page_tokens) chunk = 64LL * page_tokens;
  }
  p.chunk = (int)chunk;
  p.n_parts = n_ctx > 0 ? (int)((n_ctx + chunk - 1) / chunk) : 0;
  p.n_wg = (p.n_parts + kWaves - 1) / kWaves;
  size_t off = 0;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  // query operands: the d = 128 kernels' or the any-shape kernels' per row,
  // whichever is larger, so one size serves every codebook of this d
  const size_t qrow = std::max<size_t>((size_t)QOP_DWORDS * 4, (size_t)decode_generic_row_bytes(d));
  p.off_qop = off; off = al(off + (size_t)p.rows * qrow);
  p.off_part_o = off; off = al(off + (size_t)p.rows * p.n_wg * 8 * pad32(d) * 4);
  p.off_part_ml = off; off = al(off + (size_t)p.rows * p.n_wg * 8 * 2 * 4);
  p.bytes = off;
  return p;
}

bool make_decode_prologue(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, tq_dtype qdt,
                          const DecodePlan& plan, float sm_scale, void* ws, PArgs* out) {
  if (!decode_supported(kcb, vcb)) return false;
  PArgs pa{};
  pa.q = q; pa.qdt = qdt;
  pa.Hq = (int)plan.Hq; pa.Hkv = (int)plan.Hkv; pa.g = plan.g; pa.qgroups = plan.qgroups;
  pa.m = kcb->p.qjl_m;
  pa.mp = kcb->mp;
  pa.qscale = sm_scale * LOG2E;
  pa.rotKT = kcb->dev.rotT;
  pa.sprotKT = kcb->dev.sprotT;
  pa.qop = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + plan.off_qop);
  *out = pa;
  return true;
}

hipError_t launch_decode(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                         tq_dtype qdt, const DecodePlan& plan, const tq_codes& k,
                         const tq_codes& v, const int32_t* seq_lens, float sm_scale,
                         float* out, float* logits, void* ws, hipStream_t stream, const PageMap& pm,
                         bool prologue_done) {
  char* w = static_cast<char*>(ws);
  uint32_t* qop = reinterpret_cast<uint32_t*>(w + plan.off_qop);
  float* part_o = reinterpret_cast<float*>(w + plan.off_part_o);
  float* part_ml = reinterpret_cast<float*>(w + plan.off_part_ml);
  if (plan.rows == 0) return hipSuccess;
  if (plan.n_wg > kMaxWg) return hipErrorInvalidValue;
  if (!decode_supported(kcb, vcb))
    return launch_decode_generic(kcb, vcb, q, qdt, plan, k, v, seq_lens, sm_scale, out, logits, ws, stream, pm);

  if (!prologue_done) {
    PArgs pa{};
    make_decode_prologue(kcb, vcb, q, qdt, plan, sm_scale, ws, &pa);
    hipLaunchKernelGGL(k_prologue, dim3(4, (unsigned)plan.rows), dim3(256), 0, stream, pa);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (plan.n_parts > 0) {
    SArgs sa{};
    sa.qop = qop;
    sa.kidx = static_cast<const uint8_t*>(k.idx);
    sa.ksign = static_cast<const uint32_t*>(k.sign);
    sa.kscale = k.scale;
    sa.krnorm = k.rnorm;
    sa.k_pitch = k.idx_row_bytes;
    sa.ks_pitch = k.sign_row_bytes;
    sa.k_stride = k.seq_stride;
    sa.vidx = static_cast<const uint32_t*>(v.idx);
    sa.vscale = v.scale;
    sa.v_stride = v.seq_stride;
    sa.ktab = kcb->pq.polar ? reinterpret_cast<const uint32_t*>(kcb->dev.ptrig)
                            : (kcb->p.bits == 2 ? kcb->dev.quad_tab : kcb->dev.pair_tab);
    sa.vtab = vcb->dev.pair_tab;
    sa.ktab_dwords = kcb->dev.pair_tab_dwords;
    sa.vtab_dwords = vcb->dev.pair_tab_dwords;
    sa.seq_lens = seq_lens;
    sa.n_ctx = plan.n_ctx;
    sa.Hq = (int)plan.Hq; sa.Hkv = (int)plan.Hkv; sa.g = plan.g; sa.qgroups = plan.qgroups;
    sa.m = kcb->p.qjl_m;
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
    const bool qjl = kcb->p.qjl_m > 0;
    ProfileScope prof(TQ_KERNEL_DECODE_SPLIT, stream);
    switch (kcb->pq.polar ? 0 : kcb->p.bits) {
      case 0: launch_split_bv<0>(sa, vcb->p.bits, qjl, grid, stream); break;
      case 2: launch_split_bv<2>(sa, vcb->p.bits, qjl, grid, stream); break;
      case 3: launch_split_bv<3>(sa, vcb->p.bits, qjl, grid, stream); break;
      case 4: launch_split_bv<4>(sa, vcb->p.bits, qjl, grid, stream); break;
      default: launch_split_bv<8>(sa, vcb->p.bits, qjl, grid, stream); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  CArgs ca{};
  ca.part_o = part_o;
  ca.part_ml = part_ml;
  ca.rotV = vcb->dev.rot;
  ca.Hq = (int)plan.Hq; ca.Hkv = (int)plan.Hkv; ca.g = plan.g; ca.qgroups = plan.qgroups;
  ca.n_wg = plan.n_wg;
  ca.out = out;
  hipLaunchKernelGGL(k_combine, dim3(4, (unsigned)plan.rows), dim3(256), 0, stream, ca);
  return hipGetLastError();
}

}  // namespace tq
