// C-ABI front end: argument validation, codebook upload, kernel dispatch.
// Every exported function catches everything and reports through
// tq_last_error(); no exception crosses the ABI.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "tq_internal.hpp"

namespace tq {
namespace {
thread_local std::string g_err;
std::atomic<int> g_topk_force_scan{0};   // tq_ip_topk_exact_scan

uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float bf16_to_f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
// x rounded to the nearest fp16 (ties to even), 0 below the fp16 normal
// range; |x| < 65504 assumed
uint16_t f16_normal_rne(double x) {
  const double ax = std::fabs(x);
  if (!(ax >= 0x1p-14)) return 0;
  int e = 0;
  (void)std::frexp(ax, &e);               // ax in [2^(e-1), 2^e)
  int E = e - 1;
  double qm = std::nearbyint(std::ldexp(ax, 10 - E));   // in [1024, 2048]
  if (qm >= 2048.0) { qm = 1024.0; ++E; }
  return (uint16_t)((x < 0 ? 0x8000u : 0u) | (uint32_t)(E + 15) << 10 | ((uint32_t)qm - 1024u));
}
double f16_to_double(uint16_t b) {
  const int E = (b >> 10) & 31;
  if (E == 0) return 0.0;                 // only zeros are produced
  const double v = std::ldexp(1.0 + (b & 1023) / 1024.0, E - 15);
  return (b & 0x8000u) ? -v : v;
}
// c ~ hi + lo, both bf16
void split_bf16(double c, uint16_t& hi, uint16_t& lo) {
  hi = bf16_rne((float)c);
  lo = bf16_rne((float)(c - (double)bf16_to_f(hi)));
}

// bf16 MFMA operands of Pi (row-major, 128 x 128) in three parts hi + lo +
// lo2 (Pi - hi - lo - lo2 is below 2^-26 |Pi|): uint4 [4][8][3][64], lane l
// of wave w at k-step s holds Pi[32w + l%32][16s + 8(l/32) + j], j = 0..7,
// two bf16 per dword (lower column in the low half).
void build_q128_operands(const std::vector<double>& M, std::vector<uint32_t>& out) {
  out.assign((size_t)4 * 8 * 3 * 64 * 4, 0u);
  for (int w = 0; w < 4; ++w)
    for (int s = 0; s < 8; ++s)
      for (int l = 0; l < 64; ++l) {
        const int r = 32 * w + (l & 31);
        for (int j = 0; j < 8; ++j) {
          const int c = 16 * s + 8 * (l >> 5) + j;
          double rest = M[(size_t)r * 128 + c];
          for (int part = 0; part < 3; ++part) {
            const uint16_t h = bf16_rne((float)rest);
            rest -= (double)bf16_to_f(h);
            const size_t base = ((((size_t)w * 8 + s) * 3 + part) * 64 + l) * 4;
            out[base + j / 2] |= (uint32_t)h << (16 * (j & 1));
          }
        }
      }
}

// Column order of the d = 128 dequantize operands: k-step s, lane half h,
// element j of an MFMA operand is column 64h + 8s + j of M (so a lane's codes
// of two consecutive steps are one contiguous run of a code row).
std::vector<double> dq_permute_columns(const std::vector<double>& M) {
  std::vector<double> out((size_t)128 * 128);
  for (int r = 0; r < 128; ++r)
    for (int s = 0; s < 8; ++s)
      for (int h = 0; h < 2; ++h)
        for (int j = 0; j < 8; ++j)
          out[(size_t)r * 128 + 16 * s + 8 * h + j] = M[(size_t)r * 128 + 64 * h + 8 * s + j];
  return out;
}

// Index cells over y in [-1, 1] for the fp32 boundaries t: cell width 1/G is
// below 0.9 x the smallest gap between consecutive boundaries, so a cell holds
// at most one.  Entry c = {#t < c/G - 1, bits of (t G + G) for the t inside
// the cell, or of FLT_MAX}: the kernel compares the cell coordinate y G + G
// itself.  Returns false when the table would exceed kQ128Cells entries.
bool build_q128_cells(const std::vector<float>& t, std::vector<uint32_t>& out, float& G_out) {
  double gap = 2.0;
  for (size_t k = 1; k < t.size(); ++k) gap = std::min(gap, (double)t[k] - (double)t[k - 1]);
  if (!(gap > 0.0)) return false;
  const double G = std::ceil(1.0 / (0.9 * gap));
  const int64_t cells = 2 * (int64_t)G + 1;
  if (cells > kQ128Cells) return false;
  out.assign((size_t)cells * 2, 0u);
  for (int64_t c = 0; c < cells; ++c) {
    const double lo = (double)c / G - 1.0, hi = (double)(c + 1) / G - 1.0;
    uint32_t below = 0, inside = 0;
    float p = 3.0e38f;
    for (float v : t) {
      if ((double)v < lo) ++below;
      else if ((double)v < hi) { ++inside; p = (float)((double)v * G + G); }
    }
    if (inside > 1) return false;
    uint32_t pb;
    std::memcpy(&pb, &p, 4);
    out[2 * c] = below;
    out[2 * c + 1] = pb;
  }
  G_out = (float)G;
  return true;
}

// Argument trace: with TQ_LOG set to anything but "0" in the environment
// (read once), every hot-path entry point prints its arguments, and every
// failure its status and message, as one line on stderr.
bool log_on() {
  static const bool on = [] {
    const char* e = std::getenv("TQ_LOG");
    return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
  }();
  return on;
}

__attribute__((format(printf, 1, 2))) void log_call(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[tq] %s\n", buf);
}

tq_status fail(tq_status s, const std::string& msg) {
  g_err = msg;
  if (log_on()) std::fprintf(stderr, "[tq] -> status %d: %s\n", (int)s, msg.c_str());
  return s;
}

tq_status hip_fail(hipError_t e, const char* what) {
  return fail(TQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// a dtype arrives as a plain integer and is checked before it becomes a tq_dtype
bool dtype_ok(int32_t v) { return v == TQ_F32 || v == TQ_BF16 || v == TQ_F16; }

void free_dev(DeviceCodebook& d) {
  if (d.cent) (void)hipFree(d.cent);
  if (d.bnd) (void)hipFree(d.bnd);
  if (d.rot) (void)hipFree(d.rot);
  if (d.qjl) (void)hipFree(d.qjl);
  if (d.rotT) (void)hipFree(d.rotT);
  if (d.qjlT) (void)hipFree(d.qjlT);
  if (d.sprotT) (void)hipFree(d.sprotT);
  if (d.sprot) (void)hipFree(d.sprot);
  if (d.dqop) (void)hipFree(d.dqop);
  if (d.dqs) (void)hipFree(d.dqs);
  if (d.dqcs) (void)hipFree(d.dqcs);
  if (d.pair_tab) (void)hipFree(d.pair_tab);
  if (d.quad_tab) (void)hipFree(d.quad_tab);
  if (d.rotT64) (void)hipFree(d.rotT64);
  if (d.qjlT64) (void)hipFree(d.qjlT64);
  if (d.cent64) (void)hipFree(d.cent64);
  if (d.pair_tab16) (void)hipFree(d.pair_tab16);
  if (d.rop) (void)hipFree(d.rop);
  if (d.qtab) (void)hipFree(d.qtab);
  if (d.sop) (void)hipFree(d.sop);
  if (d.ptrig) (void)hipFree(d.ptrig);
  if (d.pbnd) (void)hipFree(d.pbnd);
  d = DeviceCodebook{};
}

template <typename T>
hipError_t upload(T** dst, const std::vector<T>& src) {
  hipError_t e = hipMalloc((void**)dst, src.size() * sizeof(T));
  if (e != hipSuccess) return e;
  return hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
}

tq_status check_params(const tq_params* p) {
  if (!p) return fail(TQ_ERR_INVALID, "params is NULL");
  if (p->d < 3 || p->d > 256) return fail(TQ_ERR_INVALID, "d must be in 3..256");
  if (p->bits < 1 || p->bits > 8) return fail(TQ_ERR_INVALID, "bits must be in 1..8");
  if (p->qjl_m < 0 || p->qjl_m > 256) return fail(TQ_ERR_INVALID, "qjl_m must be in 0..256");
  if (p->norm_correction != 0 && p->norm_correction != 1)
    return fail(TQ_ERR_INVALID, "norm_correction must be 0 or 1");
  return TQ_OK;
}

// Minimum ROW-layout index pitch of a codebook's codes.
int64_t min_idx_row_bytes(const tq_codebook* cb) {
  if (cb->pq.polar) return 4LL * ((cb->pq.field_bits + 31) / 32);
  return 4LL * cb->p.bits * ((cb->p.d + 31) / 32);
}

tq_status check_polar_params(const tq_polar_params* p) {
  if (!p) return fail(TQ_ERR_INVALID, "params is NULL");
  if (p->d < 2 || p->d > 256 || (p->d & (p->d - 1)))
    return fail(TQ_ERR_INVALID, "polar d must be a power of two in 2..256");
  if (p->bits_first < 1 || p->bits_first > 8 || p->bits_rest < 1 || p->bits_rest > 8)
    return fail(TQ_ERR_INVALID, "bits_first and bits_rest must be in 1..8");
  if (p->qjl_m < 0 || p->qjl_m > 256) return fail(TQ_ERR_INVALID, "qjl_m must be in 0..256");
  return TQ_OK;
}

tq_status check_codes(const tq_codebook* cb, const tq_codes* c, int64_t needed_len,
                      const char* name, bool need_stride32) {
  const std::string n(name);
  if (!c) return fail(TQ_ERR_INVALID, n + ": codes descriptor is NULL");
  if (!c->idx || !c->scale) return fail(TQ_ERR_INVALID, n + ": idx and scale must be non-NULL");
  if (!aligned(c->idx, 4) || !aligned(c->scale, 16))
    return fail(TQ_ERR_INVALID, n + ": idx must be 4-byte and scale 16-byte aligned");
  const bool qjl = cb->p.qjl_m > 0;
  if (qjl != (c->sign != nullptr) || qjl != (c->rnorm != nullptr))
    return fail(TQ_ERR_INVALID, n + ": sign/rnorm must be non-NULL exactly when qjl_m > 0");
  if (qjl && (!aligned(c->sign, 4) || !aligned(c->rnorm, 16)))
    return fail(TQ_ERR_INVALID, n + ": sign must be 4-byte and rnorm 16-byte aligned");
  if (c->seq_stride < needed_len || c->seq_stride < 0)
    return fail(TQ_ERR_INVALID, n + ": seq_stride too small");
  if (c->layout == TQ_LAYOUT_ROW) {
    const int64_t min_idx = min_idx_row_bytes(cb);
    if (c->idx_row_bytes < min_idx || c->idx_row_bytes % 4)
      return fail(TQ_ERR_INVALID, n + ": idx_row_bytes below minimum or not a multiple of 4");
    if (qjl) {
      const int64_t min_s = 4LL * ((cb->p.qjl_m + 31) / 32);
      if (c->sign_row_bytes < min_s || c->sign_row_bytes % 4)
        return fail(TQ_ERR_INVALID, n + ": sign_row_bytes below minimum or not a multiple of 4");
    }
    if (need_stride32 && c->seq_stride % 32)
      return fail(TQ_ERR_INVALID, n + ": seq_stride must be a multiple of 32");
  } else if (c->layout == TQ_LAYOUT_TILE32) {
    if (cb->pq.polar) return fail(TQ_ERR_UNSUPPORTED, n + ": polar codes use the row layout");
    if (c->seq_stride % 32) return fail(TQ_ERR_INVALID, n + ": tile32 seq_stride must be a multiple of 32");
    if (qjl) return fail(TQ_ERR_UNSUPPORTED, n + ": QJL signs are not supported in the tile32 layout");
  } else {
    return fail(TQ_ERR_INVALID, n + ": unknown layout");
  }
  return TQ_OK;
}

tq_status current_device_matches(const tq_codebook* cb) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != cb->device) return fail(TQ_ERR_INVALID, "codebook was built on another device");
  return TQ_OK;
}

}  // namespace

void set_error(const std::string& msg) { g_err = msg; }

namespace {
struct EventPair { hipEvent_t a = nullptr, b = nullptr; };
struct ProfileState {
  bool on = false;
  std::vector<EventPair> rec[4];
  ~ProfileState() {
    for (auto& v : rec)
      for (auto& p : v) { (void)hipEventDestroy(p.a); (void)hipEventDestroy(p.b); }
  }
};
thread_local ProfileState g_prof;
}  // namespace

ProfileScope::ProfileScope(int k, hipStream_t s) : kernel(k), stream(s) {
  if (!g_prof.on) return;
  // timing-only events: without the system-scope fence a record costs no
  // cache writeback / invalidate, so it does not slow the work around it
  EventPair p;
  if (hipEventCreateWithFlags(&p.a, hipEventDisableSystemFence) != hipSuccess) return;
  if (hipEventCreateWithFlags(&p.b, hipEventDisableSystemFence) != hipSuccess) {
    (void)hipEventDestroy(p.a);
    return;
  }
  (void)hipEventRecord(p.a, stream);
  g_prof.rec[kernel].push_back(p);
  stop = p.b;
}

ProfileScope::~ProfileScope() {
  if (stop) (void)hipEventRecord(static_cast<hipEvent_t>(stop), stream);
}

bool quantize_supported(const tq_codebook* cb);

}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_last_error(void) { return g_err.c_str(); }

tq_status tq_codebook_build(const tq_params* params, tq_codebook** out) {
  if (params)
    log_call("tq_codebook_build d=%d bits=%d qjl_m=%d nc=%d rot_seed=%llu qjl_seed=%llu", params->d,
             params->bits, params->qjl_m, params->norm_correction, (unsigned long long)params->rot_seed,
             (unsigned long long)params->qjl_seed);
  // set while a codebook is under construction, so that an exception thrown
  // part-way (a host allocation) releases it and the tables already uploaded
  tq_codebook* pending = nullptr;
  auto release_pending = [&]() {
    if (pending) {
      free_dev(pending->dev);
      delete pending;
      pending = nullptr;
    }
  };
  try {
    if (!out) return fail(TQ_ERR_INVALID, "out is NULL");
    *out = nullptr;
    tq_status s = check_params(params);
    if (s != TQ_OK) return s;
    tq_codebook* cb = new (std::nothrow) tq_codebook();
    if (!cb) return fail(TQ_ERR_ALLOC, "host allocation failed");
    pending = cb;
    cb->p = *params;
    cb->L = 1 << params->bits;
    cb->dp = pad32(params->d);
    cb->mp = params->qjl_m > 0 ? pad32(params->qjl_m) : 0;
    std::string err;
    if (!build_codebook_host(cb->p, cb->host, err)) {
      release_pending();
      return fail(TQ_ERR_NUMERIC, err);
    }
    hipError_t e = hipGetDevice(&cb->device);
    if (e != hipSuccess) { release_pending(); return hip_fail(e, "hipGetDevice"); }
    const int d = cb->p.d, dp = cb->dp, L = cb->L, m = cb->p.qjl_m, mp = cb->mp;
    std::vector<float> cent(L), bnd(L - 1), rot((size_t)dp * dp, 0.f), rotT((size_t)dp * dp, 0.f);
    for (int k = 0; k < L; ++k) cent[k] = (float)cb->host.centroids[k];
    for (int k = 0; k < L - 1; ++k) bnd[k] = (float)cb->host.boundaries[k];
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        rot[(size_t)i * dp + j] = (float)cb->host.rot[(size_t)i * d + j];
        rotT[(size_t)j * dp + i] = (float)cb->host.rot[(size_t)i * d + j];
      }
    std::vector<uint32_t> tab;
    if (cb->p.bits <= 4) {
      const int b = cb->p.bits;
      tab.resize((size_t)2 << (2 * b));
      for (int x = 0; x < L; ++x)
        for (int y = 0; y < L; ++y) {
          uint16_t hx, lx, hy, ly;
          split_bf16(cb->host.centroids[x], hx, lx);
          split_bf16(cb->host.centroids[y], hy, ly);
          const size_t e2 = (size_t)(x | (y << b));
          tab[2 * e2 + 0] = (uint32_t)hx | ((uint32_t)hy << 16);
          tab[2 * e2 + 1] = (uint32_t)lx | ((uint32_t)ly << 16);
        }
    } else {
      tab.resize(L);
      for (int x = 0; x < L; ++x) {
        uint16_t hx, lx;
        split_bf16(cb->host.centroids[x], hx, lx);
        tab[x] = (uint32_t)hx | ((uint32_t)lx << 16);
      }
    }
    cb->dev.pair_tab_dwords = (int)tab.size();
    {
      // fp16 hi/lo parts of 2^6 c for the top-k score kernel
      std::vector<uint16_t> h16(L), l16(L);
      double emax = 0.0;
      for (int x = 0; x < L; ++x) {
        const double v = std::ldexp(cb->host.centroids[x], 6);
        h16[x] = f16_normal_rne(v);
        l16[x] = f16_normal_rne(v - f16_to_double(h16[x]));
        const double back = std::ldexp(f16_to_double(h16[x]) + f16_to_double(l16[x]), -6);
        emax = std::max(emax, std::fabs(cb->host.centroids[x] - back));
      }
      cb->emax_c16 = emax;
      std::vector<uint32_t> t16(tab.size());
      if (cb->p.bits <= 4) {
        const int b = cb->p.bits;
        for (int x = 0; x < L; ++x)
          for (int y = 0; y < L; ++y) {
            const size_t e2 = (size_t)(x | (y << b));
            t16[2 * e2 + 0] = (uint32_t)h16[x] | ((uint32_t)h16[y] << 16);
            t16[2 * e2 + 1] = (uint32_t)l16[x] | ((uint32_t)l16[y] << 16);
          }
      } else {
        for (int x = 0; x < L; ++x) t16[x] = (uint32_t)h16[x] | ((uint32_t)l16[x] << 16);
      }
      if ((e = upload(&cb->dev.pair_tab16, t16)) != hipSuccess) {
        release_pending();
        return hip_fail(e, "codebook upload");
      }
    }
    {
      // float64 tables of the exact top-k refinement
      std::vector<double> rt((size_t)d * d), st(m > 0 ? (size_t)d * m : 0);
      for (int i = 0; i < d; ++i)
        for (int k2 = 0; k2 < d; ++k2) rt[(size_t)k2 * d + i] = cb->host.rot[(size_t)i * d + k2];
      for (int j = 0; j < m; ++j)
        for (int i = 0; i < d; ++i) st[(size_t)i * m + j] = cb->host.qjl[(size_t)j * d + i];
      if ((e = upload(&cb->dev.rotT64, rt)) != hipSuccess || (e = upload(&cb->dev.cent64, cb->host.centroids)) != hipSuccess ||
          (m > 0 && (e = upload(&cb->dev.qjlT64, st)) != hipSuccess)) {
        release_pending();
        return hip_fail(e, "codebook upload");
      }
    }
    if (cb->p.bits == 2) {
      const int b = cb->p.bits;
      const size_t n4 = (size_t)1 << (4 * b);
      std::vector<uint32_t> quad(4 * n4);
      std::vector<uint16_t> hi(L), lo(L);
      for (int x = 0; x < L; ++x) split_bf16(cb->host.centroids[x], hi[x], lo[x]);
      const uint32_t msk = (uint32_t)L - 1u;
      for (size_t e4 = 0; e4 < n4; ++e4) {
        const uint32_t a = e4 & msk, bb = (e4 >> b) & msk, c = (e4 >> (2 * b)) & msk, dd = (e4 >> (3 * b)) & msk;
        quad[4 * e4 + 0] = (uint32_t)hi[a] | ((uint32_t)hi[bb] << 16);
        quad[4 * e4 + 1] = (uint32_t)lo[a] | ((uint32_t)lo[bb] << 16);
        quad[4 * e4 + 2] = (uint32_t)hi[c] | ((uint32_t)hi[dd] << 16);
        quad[4 * e4 + 3] = (uint32_t)lo[c] | ((uint32_t)lo[dd] << 16);
      }
      if ((e = upload(&cb->dev.quad_tab, quad)) != hipSuccess) {
        release_pending();
        return hip_fail(e, "codebook upload");
      }
    }
    if ((e = upload(&cb->dev.cent, cent)) != hipSuccess ||
        (e = upload(&cb->dev.bnd, bnd.empty() ? std::vector<float>{0.f} : bnd)) != hipSuccess ||
        (e = upload(&cb->dev.rot, rot)) != hipSuccess ||
        (e = upload(&cb->dev.rotT, rotT)) != hipSuccess ||
        (e = upload(&cb->dev.pair_tab, tab)) != hipSuccess) {
      release_pending();
      return hip_fail(e, "codebook upload");
    }
    if (m > 0) {
      std::vector<float> qjl((size_t)mp * dp, 0.f), qjlT((size_t)dp * mp, 0.f), sprotT((size_t)dp * mp, 0.f),
          sprot((size_t)mp * dp, 0.f);
      for (int j = 0; j < m; ++j)
        for (int i = 0; i < d; ++i) {
          qjl[(size_t)j * dp + i] = (float)cb->host.qjl[(size_t)j * d + i];
          qjlT[(size_t)i * mp + j] = (float)cb->host.qjl[(size_t)j * d + i];
        }
      // sqrt(pi/2)/m S Pi in double, rounded once
      const double cq = std::sqrt(std::acos(-1.0) / 2.0) / (double)m;
      std::vector<double> sp((size_t)m * d, 0.0);   // cq (S Pi)[j][k]
      for (int j = 0; j < m; ++j)
        for (int k = 0; k < d; ++k) {
          double acc = 0.0;
          for (int i = 0; i < d; ++i)
            acc += cb->host.qjl[(size_t)j * d + i] * cb->host.rot[(size_t)i * d + k];
          sp[(size_t)j * d + k] = cq * acc;
          sprotT[(size_t)k * mp + j] = (float)(cq * acc);
          sprot[(size_t)j * dp + k] = (float)(cq * acc);
        }
      if ((e = upload(&cb->dev.sprot, sprot)) != hipSuccess) {
        release_pending();
        return hip_fail(e, "codebook upload");
      }
      if (d == 128 && m <= 128) {
        // dequantize operands: column j of (S Pi)^T scaled by 2^(127 - 2^(j % 8))
        // to meet the sign bit of row j left at bf16 bit 7 + j % 8
        std::vector<double> a2((size_t)128 * 128, 0.0);
        std::vector<float> cs(128, 0.f);
        for (int k = 0; k < 128; ++k) {
          double sum = 0.0;
          for (int j = 0; j < m; ++j) {
            const double v = sp[(size_t)j * d + k];
            sum += v;
            a2[(size_t)k * 128 + j] = std::ldexp(v, 127 - (1 << (j % 8)));
          }
          cs[k] = (float)sum;
        }
        std::vector<uint32_t> dqs;
        build_q128_operands(dq_permute_columns(a2), dqs);
        if ((e = upload(&cb->dev.dqs, dqs)) != hipSuccess || (e = upload(&cb->dev.dqcs, cs)) != hipSuccess) {
          release_pending();
          return hip_fail(e, "codebook upload");
        }
      }
      if ((e = upload(&cb->dev.qjl, qjl)) != hipSuccess ||
          (e = upload(&cb->dev.qjlT, qjlT)) != hipSuccess ||
          (e = upload(&cb->dev.sprotT, sprotT)) != hipSuccess) {
        release_pending();
        return hip_fail(e, "codebook upload");
      }
    }
    if (d == 128) {
      // Pi^T operands of the d = 128 dequantize kernel
      std::vector<double> pt((size_t)128 * 128);
      for (int r = 0; r < 128; ++r)
        for (int c = 0; c < 128; ++c) pt[(size_t)r * 128 + c] = cb->host.rot[(size_t)c * 128 + r];
      std::vector<uint32_t> dqop;
      build_q128_operands(dq_permute_columns(pt), dqop);
      if ((e = upload(&cb->dev.dqop, dqop)) != hipSuccess) {
        release_pending();
        return hip_fail(e, "codebook upload");
      }
    }
    if (d == 128 && m <= 128) {
      // operands and index cells of the d = 128 quantize kernel, and the
      // sketch operands of keys with m <= 128 rows
      std::vector<uint32_t> rop, qtab, sop;
      float qG = 0.f;
      build_q128_operands(cb->host.rot, rop);
      if (m > 0) {
        std::vector<double> sp((size_t)128 * 128, 0.0);
        for (int j = 0; j < m; ++j)
          for (int i = 0; i < 128; ++i) sp[(size_t)j * 128 + i] = cb->host.qjl[(size_t)j * 128 + i];
        build_q128_operands(sp, sop);
      }
      if (build_q128_cells(bnd, qtab, qG)) {
        if ((e = upload(&cb->dev.rop, rop)) != hipSuccess ||
            (e = upload(&cb->dev.qtab, qtab)) != hipSuccess ||
            (m > 0 && (e = upload(&cb->dev.sop, sop)) != hipSuccess)) {
          release_pending();
          return hip_fail(e, "codebook upload");
        }
        cb->dev.qcells = (int)(qtab.size() / 2);
        cb->dev.qG = qG;
      }
    }
    pending = nullptr;
    *out = cb;
    return TQ_OK;
  } catch (const std::exception& ex) {
    release_pending();
    return fail(TQ_ERR_ALLOC, std::string("tq_codebook_build: ") + ex.what());
  } catch (...) {
    release_pending();
    return fail(TQ_ERR_ALLOC, "tq_codebook_build: unknown exception");
  }
}

tq_status tq_codebook_values(const tq_params* params, double* centroids, double* boundaries,
                             double* rot, double* qjl) {
  try {
    tq_status s = check_params(params);
    if (s != TQ_OK) return s;
    HostCodebook hc;
    std::string err;
    if (!build_codebook_host(*params, hc, err)) return fail(TQ_ERR_NUMERIC, err);
    if (centroids) std::memcpy(centroids, hc.centroids.data(), hc.centroids.size() * sizeof(double));
    if (boundaries) std::memcpy(boundaries, hc.boundaries.data(), hc.boundaries.size() * sizeof(double));
    if (rot) std::memcpy(rot, hc.rot.data(), hc.rot.size() * sizeof(double));
    if (qjl && !hc.qjl.empty()) std::memcpy(qjl, hc.qjl.data(), hc.qjl.size() * sizeof(double));
    return TQ_OK;
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_codebook_values: unexpected exception");
  }
}

tq_status tq_polar_codebook_build(const tq_polar_params* params, tq_codebook** out) {
  if (params)
    log_call("tq_polar_codebook_build d=%d b1=%d br=%d qjl_m=%d", params->d, params->bits_first,
             params->bits_rest, params->qjl_m);
  tq_codebook* pending = nullptr;
  auto release_pending = [&]() {
    if (pending) {
      free_dev(pending->dev);
      delete pending;
      pending = nullptr;
    }
  };
  try {
    if (!out) return fail(TQ_ERR_INVALID, "out is NULL");
    *out = nullptr;
    tq_status s = check_polar_params(params);
    if (s != TQ_OK) return s;
    tq_codebook* cb = new (std::nothrow) tq_codebook();
    if (!cb) return fail(TQ_ERR_ALLOC, "host allocation failed");
    pending = cb;
    cb->p.d = params->d;
    cb->p.bits = params->bits_first;
    cb->p.qjl_m = params->qjl_m;
    cb->p.norm_correction = 0;
    cb->p.rot_seed = params->rot_seed;
    cb->p.qjl_seed = params->qjl_seed;
    cb->dp = pad32(params->d);
    cb->mp = params->qjl_m > 0 ? pad32(params->qjl_m) : 0;
    std::vector<int> coff, boff;
    std::string err;
    if (!build_polar_codebook_host(*params, cb->host, coff, boff, err)) {
      release_pending();
      return fail(TQ_ERR_NUMERIC, err);
    }
    PolarInfo& pq = cb->pq;
    pq.polar = true;
    pq.b1 = params->bits_first;
    pq.br = params->bits_rest;
    pq.levels = (int)coff.size() - 2;
    for (size_t i = 0; i < coff.size() && i < (size_t)kPolarMaxLevels + 2; ++i) {
      pq.cent_off[i] = coff[i];
      pq.bnd_off[i] = boff[i];
    }
    pq.field_bits = (params->d / 2) * pq.b1 + (params->d / 2 - 1) * pq.br;
    cb->L = 1 << pq.b1;
    hipError_t e = hipGetDevice(&cb->device);
    if (e != hipSuccess) { release_pending(); return hip_fail(e, "hipGetDevice"); }
    const int d = cb->p.d, dp = cb->dp, m = cb->p.qjl_m, mp = cb->mp;
    std::vector<float> trig(2 * cb->host.centroids.size()), pb(cb->host.boundaries.size());
    for (size_t j = 0; j < cb->host.centroids.size(); ++j) {
      trig[2 * j] = (float)std::cos(cb->host.centroids[j]);
      trig[2 * j + 1] = (float)std::sin(cb->host.centroids[j]);
    }
    for (size_t j = 0; j < pb.size(); ++j) pb[j] = (float)cb->host.boundaries[j];
    std::vector<float> rot((size_t)dp * dp, 0.f), rotT((size_t)dp * dp, 0.f);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        rot[(size_t)i * dp + j] = (float)cb->host.rot[(size_t)i * d + j];
        rotT[(size_t)j * dp + i] = (float)cb->host.rot[(size_t)i * d + j];
      }
    if ((e = upload(&cb->dev.ptrig, trig)) != hipSuccess ||
        (e = upload(&cb->dev.pbnd, pb.empty() ? std::vector<float>{0.f} : pb)) != hipSuccess ||
        (e = upload(&cb->dev.rot, rot)) != hipSuccess || (e = upload(&cb->dev.rotT, rotT)) != hipSuccess) {
      release_pending();
      return hip_fail(e, "codebook upload");
    }
    if (m > 0) {
      // S (quantize), and sqrt(pi/2)/m S Pi in both orientations (the decode
      // prologue's t = sqrt(pi/2)/m S Pi q, the dequantize sketch term)
      std::vector<float> qjl((size_t)mp * dp, 0.f), sprotT((size_t)dp * mp, 0.f), sprot((size_t)mp * dp, 0.f);
      for (int j = 0; j < m; ++j)
        for (int i = 0; i < d; ++i) qjl[(size_t)j * dp + i] = (float)cb->host.qjl[(size_t)j * d + i];
      const double cq = std::sqrt(std::acos(-1.0) / 2.0) / (double)m;
      for (int j = 0; j < m; ++j)
        for (int k = 0; k < d; ++k) {
          double acc = 0.0;
          for (int i = 0; i < d; ++i) acc += cb->host.qjl[(size_t)j * d + i] * cb->host.rot[(size_t)i * d + k];
          sprotT[(size_t)k * mp + j] = (float)(cq * acc);
          sprot[(size_t)j * dp + k] = (float)(cq * acc);
        }
      if ((e = upload(&cb->dev.qjl, qjl)) != hipSuccess || (e = upload(&cb->dev.sprotT, sprotT)) != hipSuccess ||
          (e = upload(&cb->dev.sprot, sprot)) != hipSuccess) {
        release_pending();
        return hip_fail(e, "codebook upload");
      }
    }
    pending = nullptr;
    *out = cb;
    return TQ_OK;
  } catch (const std::exception& ex) {
    release_pending();
    return fail(TQ_ERR_ALLOC, std::string("tq_polar_codebook_build: ") + ex.what());
  } catch (...) {
    release_pending();
    return fail(TQ_ERR_ALLOC, "tq_polar_codebook_build: unknown exception");
  }
}

tq_status tq_polar_codebook_values(const tq_polar_params* params, double* centroids, double* boundaries,
                                   double* rot, double* qjl) {
  try {
    tq_status s = check_polar_params(params);
    if (s != TQ_OK) return s;
    HostCodebook hc;
    std::vector<int> coff, boff;
    std::string err;
    if (!build_polar_codebook_host(*params, hc, coff, boff, err)) return fail(TQ_ERR_NUMERIC, err);
    if (centroids) std::memcpy(centroids, hc.centroids.data(), hc.centroids.size() * sizeof(double));
    if (boundaries) std::memcpy(boundaries, hc.boundaries.data(), hc.boundaries.size() * sizeof(double));
    if (rot) std::memcpy(rot, hc.rot.data(), hc.rot.size() * sizeof(double));
    if (qjl && !hc.qjl.empty()) std::memcpy(qjl, hc.qjl.data(), hc.qjl.size() * sizeof(double));
    return TQ_OK;
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_polar_codebook_values: unexpected exception");
  }
}

tq_status tq_codebook_solver_limits(int32_t lloyd_iters, int32_t newton_iters) {
  set_solver_limits(lloyd_iters, newton_iters);
  return TQ_OK;
}

tq_status tq_codebook_destroy(tq_codebook* cb) {
  if (!cb) return TQ_OK;
  free_dev(cb->dev);
  delete cb;
  return TQ_OK;
}

tq_status tq_codebook_export(const tq_codebook* cb, double* centroids, double* boundaries,
                             double* rot, double* qjl) {
  if (!cb) return fail(TQ_ERR_INVALID, "codebook is NULL");
  if (centroids)
    std::memcpy(centroids, cb->host.centroids.data(), cb->host.centroids.size() * sizeof(double));
  if (boundaries)
    std::memcpy(boundaries, cb->host.boundaries.data(), cb->host.boundaries.size() * sizeof(double));
  if (rot) std::memcpy(rot, cb->host.rot.data(), cb->host.rot.size() * sizeof(double));
  if (qjl && !cb->host.qjl.empty())
    std::memcpy(qjl, cb->host.qjl.data(), cb->host.qjl.size() * sizeof(double));
  return TQ_OK;
}

tq_status tq_code_row_bytes(const tq_codebook* cb, int64_t* idx_row_bytes,
                            int64_t* sign_row_bytes) {
  if (!cb) return fail(TQ_ERR_INVALID, "codebook is NULL");
  if (idx_row_bytes) *idx_row_bytes = min_idx_row_bytes(cb);
  if (sign_row_bytes) *sign_row_bytes = cb->p.qjl_m > 0 ? 4LL * ((cb->p.qjl_m + 31) / 32) : 0;
  return TQ_OK;
}

}  // extern "C"

namespace {

// Validation and dispatch shared by tq_quantize_kv and tq_quantize_kv_paged:
// code planes must hold need_len positions; pm maps a sequence's blocks to
// its output plane and blocks.
tq_status quantize_impl(const tq_codebook* kcb, const tq_codebook* vcb, const void* k, const void* v,
                        tq_dtype dt, int64_t n_seq, int64_t n_tok, int64_t tok_offset,
                        const tq_codes* k_out, const tq_codes* v_out, void* stream, int64_t need_len,
                        const PageMap& pm, const PArgs* pro = nullptr, int64_t pro_rows = 0,
                        bool* pro_done = nullptr) {
  const void* xs[2] = {k, v};
  const tq_codebook* cbs[2] = {kcb, vcb};
  const tq_codes* outs[2] = {k_out, v_out};
  const char* names[2] = {"k", "v"};
  for (int t = 0; t < 2; ++t) {
    if (!xs[t]) continue;
    if (!cbs[t]) return fail(TQ_ERR_INVALID, std::string(names[t]) + ": codebook is NULL");
    tq_status s = check_codes(cbs[t], outs[t], need_len, names[t], false);
    if (s != TQ_OK) return s;
    if (cbs[t]->pq.polar ? !polar_quantize_supported(cbs[t]) : !quantize_supported(cbs[t]))
      return fail(TQ_ERR_UNSUPPORTED, std::string(names[t]) + (cbs[t]->pq.polar
                                          ? ": polar quantize supports d <= 128 and qjl_m <= 128"
                                          : ": quantize supports d <= 256 and qjl_m <= 256"));
    s = current_device_matches(cbs[t]);
    if (s != TQ_OK) return s;
  }
  // polar codebooks: one kernel serves appends and bulk calls
  for (int t = 0; t < 2; ++t) {
    if (!xs[t] || !cbs[t]->pq.polar) continue;
    QuantJob job{xs[t], dt, n_seq, n_tok, tok_offset, *outs[t], pm};
    hipError_t e = launch_polar_quantize(cbs[t], job, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    xs[t] = nullptr;
  }
  if (!xs[0] && !xs[1]) return TQ_OK;
  if (n_tok <= kSmallMaxTok && n_seq * n_tok <= 0x7FFFFFFF) {
    const tq_codebook* sc[2];
    QuantJob sj[2];
    int nj = 0;
    for (int t = 0; t < 2; ++t) {
      if (!xs[t]) continue;
      sc[nj] = cbs[t];
      sj[nj++] = QuantJob{xs[t], dt, n_seq, n_tok, tok_offset, *outs[t], pm};
    }
    hipError_t e = launch_quantize_small(sc, sj, nj, static_cast<hipStream_t>(stream), pro, pro_rows);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    if (pro_done) *pro_done = pro != nullptr;
    return TQ_OK;
  }
  for (int t = 0; t < 2; ++t) {
    if (!xs[t]) continue;
    QuantJob job{xs[t], dt, n_seq, n_tok, tok_offset, *outs[t], pm};
    hipError_t e = launch_quantize(cbs[t], job, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
  }
  return TQ_OK;
}

// Page size and table of a paged call; n_pages comes from the pool planes.
tq_status check_pages(int32_t page_tokens, const int32_t* block_table, int64_t max_pages, int64_t n_logical,
                      const tq_codes* k_pool, const tq_codes* v_pool, PageMap& pm, int64_t hkv) {
  if (page_tokens < 32 || page_tokens > 65536 || (page_tokens & (page_tokens - 1)))
    return fail(TQ_ERR_INVALID, "page_tokens must be a power of two in 32..65536");
  if (!block_table) return fail(TQ_ERR_INVALID, "block_table is NULL");
  if (max_pages < 1 || max_pages * page_tokens < n_logical)
    return fail(TQ_ERR_INVALID, "max_pages * page_tokens must cover every position of the call");
  int64_t n_pages = -1;
  const tq_codes* pools[2] = {k_pool, v_pool};
  for (const tq_codes* c : pools) {
    if (!c) continue;
    if (c->seq_stride < page_tokens || c->seq_stride % page_tokens)
      return fail(TQ_ERR_INVALID, "a pool's seq_stride must be a positive multiple of page_tokens");
    const int64_t np = c->seq_stride / page_tokens;
    n_pages = n_pages < 0 ? np : (np < n_pages ? np : n_pages);
  }
  if (n_pages > 0x7FFFFFFFLL) return fail(TQ_ERR_UNSUPPORTED, "at most 2^31 - 1 pages per pool");
  pm.table = block_table;
  pm.max_pages = max_pages;
  pm.n_pages = n_pages < 1 ? 1 : n_pages;
  pm.hkv = hkv;
  int sh = 0;
  while ((32 << sh) < page_tokens) ++sh;
  pm.ppb_shift = sh;
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_quantize_kv(const tq_codebook* kcb, const tq_codebook* vcb, const void* k,
                         const void* v, int32_t dt_in, int64_t n_seq, int64_t n_tok,
                         int64_t tok_offset, const tq_codes* k_out, const tq_codes* v_out,
                         void* stream) {
  log_call("tq_quantize_kv kcb=%p vcb=%p k=%p v=%p dt=%d n_seq=%lld n_tok=%lld tok_offset=%lld stream=%p",
           (const void*)kcb, (const void*)vcb, k, v, dt_in, (long long)n_seq, (long long)n_tok,
           (long long)tok_offset, stream);
  try {
    if (!dtype_ok(dt_in)) return fail(TQ_ERR_INVALID, "bad dtype");
    const tq_dtype dt = static_cast<tq_dtype>(dt_in);
    if (n_seq < 0 || n_tok < 0 || tok_offset < 0)
      return fail(TQ_ERR_INVALID, "n_seq, n_tok and tok_offset must be >= 0");
    if (n_seq == 0 || n_tok == 0) return TQ_OK;   // nothing is read or written
    if (!k && !v) return fail(TQ_ERR_INVALID, "k and v are both NULL");
    return quantize_impl(kcb, vcb, k, v, dt, n_seq, n_tok, tok_offset, k_out, v_out, stream,
                         tok_offset + n_tok, PageMap{});
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_quantize_kv: unexpected exception");
  }
}

tq_status tq_quantize_kv_paged(const tq_codebook* kcb, const tq_codebook* vcb, const void* k,
                               const void* v, int32_t dt_in, int64_t B, int64_t Hkv, int64_t n_tok,
                               int64_t tok_offset, const int32_t* block_table, int64_t max_pages,
                               int32_t page_tokens, const tq_codes* k_pool, const tq_codes* v_pool,
                               void* stream) {
  log_call("tq_quantize_kv_paged dt=%d B=%lld Hkv=%lld n_tok=%lld tok_offset=%lld max_pages=%lld page_tokens=%d",
           dt_in, (long long)B, (long long)Hkv, (long long)n_tok, (long long)tok_offset, (long long)max_pages,
           page_tokens);
  try {
    if (!dtype_ok(dt_in)) return fail(TQ_ERR_INVALID, "bad dtype");
    const tq_dtype dt = static_cast<tq_dtype>(dt_in);
    if (B < 0 || Hkv <= 0 || n_tok < 0 || tok_offset < 0)
      return fail(TQ_ERR_INVALID, "need B, n_tok, tok_offset >= 0 and Hkv > 0");
    if (B == 0 || n_tok == 0) return TQ_OK;
    if (!k && !v) return fail(TQ_ERR_INVALID, "k and v are both NULL");
    PageMap pm;
    tq_status s = check_pages(page_tokens, block_table, max_pages, tok_offset + n_tok, k ? k_pool : nullptr,
                              v ? v_pool : nullptr, pm, Hkv);
    if (s != TQ_OK) return s;
    return quantize_impl(kcb, vcb, k, v, dt, B * Hkv, n_tok, tok_offset, k_pool, v_pool, stream, page_tokens, pm);
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_quantize_kv_paged: unexpected exception");
  }
}

tq_status tq_attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_ctx,
                                   int32_t d, size_t* bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID, "bytes is NULL");
  if (B < 0 || Hq < 0 || Hkv <= 0 || n_ctx < 0 || Hq % Hkv)
    return fail(TQ_ERR_INVALID, "need B, n_ctx >= 0, Hkv > 0, Hq a multiple of Hkv");
  if (d < 3 || d > 256) return fail(TQ_ERR_INVALID, "d must be in 3..256");
  *bytes = plan_decode(B, Hq, Hkv, n_ctx, d).bytes;
  return TQ_OK;
}

}  // extern "C"

namespace {

// Validation and launch shared by tq_attn_decode and tq_attn_decode_paged.
tq_status decode_impl(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, int32_t qdt_in, int64_t B,
                      int64_t Hq, int64_t Hkv, const tq_codes* k, const tq_codes* v, const int32_t* seq_lens,
                      int64_t n_ctx, float sm_scale, float* out, float* logits, void* workspace,
                      size_t ws_bytes, void* stream, int64_t need_len, int page_tokens, const PageMap& pm,
                      bool launch = true, bool prologue_done = false, DecodePlan* plan_out = nullptr) {
  if (!kcb || !vcb) return fail(TQ_ERR_INVALID, "codebook is NULL");
  if (!dtype_ok(qdt_in)) return fail(TQ_ERR_INVALID, "bad dtype");
  const tq_dtype qdt = static_cast<tq_dtype>(qdt_in);
  if (B < 0 || Hq < 0 || Hkv <= 0 || n_ctx < 0 || Hq % Hkv)
    return fail(TQ_ERR_INVALID, "need B, n_ctx >= 0, Hkv > 0, Hq a multiple of Hkv");
  if (kcb->p.d != vcb->p.d) return fail(TQ_ERR_INVALID, "key and value codebooks differ in d");
  if (!decode_supported(kcb, vcb) && !decode_generic_supported(kcb, vcb))
    return fail(TQ_ERR_UNSUPPORTED,
                "decode takes scalar codebooks, or polar keys with (b1, br) = (4, 2) at d = 128 and "
                "qjl_m <= 128 with scalar values of 2, 3, 4 or 8 bits");
  if (!std::isfinite(sm_scale)) return fail(TQ_ERR_INVALID, "sm_scale must be finite");
  if (B * Hq == 0) return TQ_OK;
  if (!q || !out) return fail(TQ_ERR_INVALID, "q and out must be non-NULL");
  if (!k || k->layout != TQ_LAYOUT_ROW) return fail(TQ_ERR_INVALID, "key codes must use the row layout");
  if (!v || v->layout != TQ_LAYOUT_TILE32)
    return fail(TQ_ERR_INVALID, "value codes must use the tile32 layout");
  tq_status s = check_codes(kcb, k, need_len, "k", true);
  if (s != TQ_OK) return s;
  s = check_codes(vcb, v, need_len, "v", true);
  if (s != TQ_OK) return s;
  if ((s = current_device_matches(kcb)) != TQ_OK) return s;
  if ((s = current_device_matches(vcb)) != TQ_OK) return s;
  {
    // the split kernel addresses one sequence's (or pool plane's) planes
    // with 32-bit byte offsets
    const int64_t lim = 0x7FFFFFFFLL;
    const int64_t vblk = 64LL * ((vcb->p.d + 15) / 16) * vcb->p.bits;
    if (k->seq_stride * k->idx_row_bytes >= lim || k->seq_stride * k->sign_row_bytes >= lim ||
        (v->seq_stride / 32) * vblk >= lim || 4 * k->seq_stride >= lim || 4 * v->seq_stride >= lim)
      return fail(TQ_ERR_UNSUPPORTED, "a sequence's code planes must each stay below 2 GiB");
  }
  const DecodePlan plan = plan_decode(B, Hq, Hkv, n_ctx, kcb->p.d, page_tokens);
  if (plan.rows > 65535 || B * Hq > 0x7FFFFFFF)
    return fail(TQ_ERR_UNSUPPORTED, "B * Hkv * ceil(g/8) must be <= 65535");
  if (plan.n_wg > 1024) return fail(TQ_ERR_UNSUPPORTED, "context too long for the split plan");
  if (!workspace || ws_bytes < plan.bytes)
    return fail(TQ_ERR_INVALID, "workspace missing or smaller than the workspace query");
  if (!aligned(workspace, 256)) return fail(TQ_ERR_INVALID, "workspace must be 256-byte aligned");
  if (!aligned(out, 16)) return fail(TQ_ERR_INVALID, "out must be 16-byte aligned");
  if (plan_out) *plan_out = plan;
  if (!launch) return TQ_OK;
  hipError_t e = launch_decode(kcb, vcb, q, qdt, plan, *k, *v, seq_lens, sm_scale, out,
                               logits, workspace, static_cast<hipStream_t>(stream), pm, prologue_done);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_attn_decode(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                         int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv, const tq_codes* k,
                         const tq_codes* v, const int32_t* seq_lens, int64_t n_ctx,
                         float sm_scale, float* out, float* logits, void* workspace,
                         size_t ws_bytes, void* stream) {
  log_call("tq_attn_decode qdt=%d B=%lld Hq=%lld Hkv=%lld n_ctx=%lld sm_scale=%g seq_lens=%p out=%p logits=%p "
           "workspace=%p ws_bytes=%zu stream=%p",
           qdt, (long long)B, (long long)Hq, (long long)Hkv, (long long)n_ctx, (double)sm_scale,
           (const void*)seq_lens, (void*)out, (void*)logits, workspace, ws_bytes, stream);
  try {
    return decode_impl(kcb, vcb, q, qdt, B, Hq, Hkv, k, v, seq_lens, n_ctx, sm_scale, out, logits,
                       workspace, ws_bytes, stream, n_ctx, 0, PageMap{});
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_attn_decode: unexpected exception");
  }
}

tq_status tq_attn_decode_append(const tq_codebook* kcb, const tq_codebook* vcb, const void* k_new,
                                const void* v_new, int32_t kv_dtype, int64_t n_new, int64_t tok_offset,
                                const void* q, int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv,
                                const tq_codes* k, const tq_codes* v, const int32_t* seq_lens, int64_t n_ctx,
                                float sm_scale, float* out, float* logits, void* workspace, size_t ws_bytes,
                                void* stream) {
  log_call("tq_attn_decode_append kv_dtype=%d n_new=%lld tok_offset=%lld qdt=%d B=%lld Hq=%lld Hkv=%lld "
           "n_ctx=%lld sm_scale=%g seq_lens=%p out=%p logits=%p workspace=%p ws_bytes=%zu stream=%p",
           kv_dtype, (long long)n_new, (long long)tok_offset, qdt, (long long)B, (long long)Hq, (long long)Hkv,
           (long long)n_ctx, (double)sm_scale, (const void*)seq_lens, (void*)out, (void*)logits, workspace,
           ws_bytes, stream);
  try {
    if (!k_new || !v_new) return fail(TQ_ERR_INVALID, "k_new and v_new must be non-NULL");
    if (!dtype_ok(kv_dtype)) return fail(TQ_ERR_INVALID, "bad dtype");
    if (n_new < 1 || tok_offset < 0 || tok_offset + n_new > n_ctx)
      return fail(TQ_ERR_INVALID, "need n_new >= 1 and 0 <= tok_offset, tok_offset + n_new <= n_ctx");
    // every check of both calls before anything is launched
    DecodePlan plan{};
    tq_status s = decode_impl(kcb, vcb, q, qdt, B, Hq, Hkv, k, v, seq_lens, n_ctx, sm_scale, out, logits,
                              workspace, ws_bytes, stream, n_ctx, 0, PageMap{}, false, false, &plan);
    if (s != TQ_OK) return s;
    if (B * Hq == 0)
      return quantize_impl(kcb, vcb, k_new, v_new, static_cast<tq_dtype>(kv_dtype), B * Hkv, n_new, tok_offset, k, v,
                           stream, tok_offset + n_new, PageMap{});
    PArgs pro{};
    const bool fuse = n_new <= kSmallMaxTok && !kcb->pq.polar && !vcb->pq.polar &&
                      make_decode_prologue(kcb, vcb, q, static_cast<tq_dtype>(qdt), plan, sm_scale, workspace, &pro);
    bool pro_done = false;
    s = quantize_impl(kcb, vcb, k_new, v_new, static_cast<tq_dtype>(kv_dtype), B * Hkv, n_new, tok_offset, k, v,
                      stream, tok_offset + n_new, PageMap{}, fuse ? &pro : nullptr, plan.rows, &pro_done);
    if (s != TQ_OK) return s;
    return decode_impl(kcb, vcb, q, qdt, B, Hq, Hkv, k, v, seq_lens, n_ctx, sm_scale, out, logits, workspace,
                       ws_bytes, stream, n_ctx, 0, PageMap{}, true, pro_done, nullptr);
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_attn_decode_append: unexpected exception");
  }
}

tq_status tq_attn_decode_noalloc(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                                 int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv, const tq_codes* k,
                                 const tq_codes* v, const int32_t* seq_lens, int64_t n_ctx,
                                 float sm_scale, float* out, float* logits, void* stream) {
  log_call("tq_attn_decode_noalloc qdt=%d B=%lld Hq=%lld Hkv=%lld n_ctx=%lld sm_scale=%g", qdt, (long long)B,
           (long long)Hq, (long long)Hkv, (long long)n_ctx, (double)sm_scale);
  try {
    if (B < 0 || Hq < 0 || Hkv <= 0 || n_ctx < 0 || Hq % Hkv)
      return fail(TQ_ERR_INVALID, "need B, n_ctx >= 0, Hkv > 0, Hq a multiple of Hkv");
    if (!kcb || !vcb) return fail(TQ_ERR_INVALID, "codebook is NULL");
    const size_t need = plan_decode(B, Hq, Hkv, n_ctx, kcb->p.d).bytes;
    if (need > kNoallocScratchBytes)
      return fail(TQ_ERR_UNSUPPORTED, "tq_attn_decode_noalloc: this shape needs " + std::to_string(need) +
                                          " bytes of scratch, above the fixed " +
                                          std::to_string(kNoallocScratchBytes) + "; use tq_attn_decode");
    void* ws = nullptr;
    hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
    // no profiling events either: this path creates nothing
    const bool prof = g_prof.on;
    g_prof.on = false;
    tq_status s = decode_impl(kcb, vcb, q, qdt, B, Hq, Hkv, k, v, seq_lens, n_ctx, sm_scale, out, logits, ws,
                              kNoallocScratchBytes, stream, n_ctx, 0, PageMap{});
    g_prof.on = prof;
    return s;
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_attn_decode_noalloc: unexpected exception");
  }
}

tq_status tq_attn_decode_paged_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_ctx, int32_t d,
                                         int32_t page_tokens, size_t* bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID, "bytes is NULL");
  if (B < 0 || Hq < 0 || Hkv <= 0 || n_ctx < 0 || Hq % Hkv)
    return fail(TQ_ERR_INVALID, "need B, n_ctx >= 0, Hkv > 0, Hq a multiple of Hkv");
  if (page_tokens < 32 || page_tokens > 65536 || (page_tokens & (page_tokens - 1)))
    return fail(TQ_ERR_INVALID, "page_tokens must be a power of two in 32..65536");
  if (d < 3 || d > 256) return fail(TQ_ERR_INVALID, "d must be in 3..256");
  *bytes = plan_decode(B, Hq, Hkv, n_ctx, d, page_tokens).bytes;
  return TQ_OK;
}

tq_status tq_attn_decode_paged(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                               int32_t qdt, int64_t B, int64_t Hq, int64_t Hkv, const tq_codes* k_pool,
                               const tq_codes* v_pool, const int32_t* block_table, int64_t max_pages,
                               int32_t page_tokens, const int32_t* seq_lens, int64_t n_ctx, float sm_scale,
                               float* out, float* logits, void* workspace, size_t ws_bytes, void* stream) {
  log_call("tq_attn_decode_paged qdt=%d B=%lld Hq=%lld Hkv=%lld max_pages=%lld page_tokens=%d n_ctx=%lld "
           "sm_scale=%g ws_bytes=%zu",
           qdt, (long long)B, (long long)Hq, (long long)Hkv, (long long)max_pages, page_tokens, (long long)n_ctx,
           (double)sm_scale, ws_bytes);
  try {
    if (B < 0 || Hq < 0 || Hkv <= 0 || n_ctx < 0)
      return fail(TQ_ERR_INVALID, "need B, Hq, n_ctx >= 0 and Hkv > 0");
    PageMap pm;
    tq_status s = check_pages(page_tokens, block_table, max_pages, n_ctx, k_pool, v_pool, pm, Hkv);
    if (s != TQ_OK) return s;
    return decode_impl(kcb, vcb, q, qdt, B, Hq, Hkv, k_pool, v_pool, seq_lens, n_ctx, sm_scale, out, logits,
                       workspace, ws_bytes, stream, page_tokens, page_tokens, pm);
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_attn_decode_paged: unexpected exception");
  }
}

tq_status tq_ip_topk_workspace(int64_t nq, int64_t n_db, int32_t k, int32_t d, size_t* bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID, "bytes is NULL");
  if (nq < 0 || n_db < 0 || k < 0 || d < 3 || d > 256)
    return fail(TQ_ERR_INVALID, "need nq, n_db, k >= 0 and d in 3..256");
  if (k > kIpTopkMax) return fail(TQ_ERR_UNSUPPORTED, "k must be <= 32");
  *bytes = plan_topk(nq, n_db, k, d, 256).bytes;     // sized for any qjl_m <= 256
  return TQ_OK;
}

tq_status tq_ip_topk_scan_count(const tq_codebook* cb, const void* workspace, int64_t nq, int64_t n_db,
                                int32_t k, void* stream, int64_t* count) {
  try {
    if (!cb || !count) return fail(TQ_ERR_INVALID, "codebook and count must be non-NULL");
    if (nq < 0 || n_db < 0 || k < 0 || k > kIpTopkMax) return fail(TQ_ERR_INVALID, "invalid nq, n_db or k");
    *count = 0;
    if (nq == 0 || k == 0) return TQ_OK;
    if (!workspace) return fail(TQ_ERR_INVALID, "workspace is NULL");
    const TopkPlan plan = plan_topk(nq, n_db, k, cb->p.d, cb->p.qjl_m);
    uint32_t c = 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(&c, static_cast<const char*>(workspace) + plan.off_bounds + 12, 4,
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "scan count read");
    *count = (int64_t)c;
    return TQ_OK;
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_ip_topk_scan_count: unexpected exception");
  }
}

tq_status tq_ip_topk_exact_scan(int32_t always) {
  if (always != 0 && always != 1) return fail(TQ_ERR_INVALID, "always must be 0 or 1");
  g_topk_force_scan.store(always);
  return TQ_OK;
}

tq_status tq_ip_topk(const tq_codebook* cb, const float* queries, int64_t nq,
                     const tq_codes* db, int64_t n_db, int32_t k, int64_t* out_idx,
                     float* out_score, void* workspace, size_t ws_bytes, void* stream) {
  log_call("tq_ip_topk cb=%p queries=%p nq=%lld n_db=%lld k=%d workspace=%p ws_bytes=%zu stream=%p",
           (const void*)cb, (const void*)queries, (long long)nq, (long long)n_db, k, workspace, ws_bytes, stream);
  try {
    if (!cb) return fail(TQ_ERR_INVALID, "codebook is NULL");
    if (nq < 0 || n_db < 0 || k < 0) return fail(TQ_ERR_INVALID, "need nq, n_db, k >= 0");
    if (k > kIpTopkMax) return fail(TQ_ERR_UNSUPPORTED, "k must be <= 32");
    if (k > n_db) return fail(TQ_ERR_INVALID, "k must be <= n_db");
    if (nq == 0 || k == 0) return TQ_OK;
    if (!queries || !out_idx || !out_score)
      return fail(TQ_ERR_INVALID, "queries, out_idx and out_score must be non-NULL");
    if (!db || db->layout != TQ_LAYOUT_ROW)
      return fail(TQ_ERR_INVALID, "database codes must use the row layout");
    if (cb->pq.polar) return fail(TQ_ERR_UNSUPPORTED, "top-k takes scalar codes, not polar codes");
    tq_status s = check_codes(cb, db, n_db, "db", false);
    if (s != TQ_OK) return s;
    if (db->idx_row_bytes > kIpMaxRowBytes || (cb->p.qjl_m > 0 && db->sign_row_bytes > kIpMaxSignRowBytes))
      return fail(TQ_ERR_UNSUPPORTED, "top-k supports idx_row_bytes <= 256 and sign_row_bytes <= 32");
    if ((s = current_device_matches(cb)) != TQ_OK) return s;
    if (n_db > 0x7FFFFFF0LL) return fail(TQ_ERR_UNSUPPORTED, "n_db must fit in 31 bits");
    const TopkPlan plan = plan_topk(nq, n_db, k, cb->p.d, cb->p.qjl_m);
    if (plan.nqb > 65535) return fail(TQ_ERR_UNSUPPORTED, "nq must be <= 524280");
    size_t need = 0;
    (void)tq_ip_topk_workspace(nq, n_db, k, cb->p.d, &need);
    if (!workspace || ws_bytes < need)
      return fail(TQ_ERR_INVALID, "workspace missing or smaller than tq_ip_topk_workspace()");
    if (!aligned(workspace, 256)) return fail(TQ_ERR_INVALID, "workspace must be 256-byte aligned");
    if (!aligned(queries, 4) || !aligned(out_idx, 8) || !aligned(out_score, 4))
      return fail(TQ_ERR_INVALID, "queries, out_idx and out_score must be naturally aligned");
    hipError_t e = launch_topk(cb, queries, plan, *db, out_idx, out_score, workspace,
                               static_cast<hipStream_t>(stream), g_topk_force_scan.load() != 0);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return TQ_OK;
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_ip_topk: unexpected exception");
  }
}

tq_status tq_dequantize(const tq_codebook* cb, const tq_codes* codes, int64_t n_seq,
                        int64_t n_tok, int64_t tok_offset, void* out, int32_t out_dt_in,
                        void* stream) {
  log_call("tq_dequantize cb=%p n_seq=%lld n_tok=%lld tok_offset=%lld out=%p out_dt=%d stream=%p",
           (const void*)cb, (long long)n_seq, (long long)n_tok, (long long)tok_offset, out, out_dt_in, stream);
  try {
    if (!cb) return fail(TQ_ERR_INVALID, "codebook is NULL");
    if (!dtype_ok(out_dt_in)) return fail(TQ_ERR_INVALID, "bad out dtype");
    const tq_dtype out_dt = static_cast<tq_dtype>(out_dt_in);
    if (n_seq < 0 || n_tok < 0 || tok_offset < 0)
      return fail(TQ_ERR_INVALID, "n_seq, n_tok and tok_offset must be >= 0");
    if (n_seq == 0 || n_tok == 0) return TQ_OK;
    if (!out) return fail(TQ_ERR_INVALID, "out is NULL");
    if (!aligned(out, 16)) return fail(TQ_ERR_INVALID, "out must be 16-byte aligned");
    tq_status s = check_codes(cb, codes, tok_offset + n_tok, "codes", false);
    if (s != TQ_OK) return s;
    if (cb->pq.polar ? !polar_quantize_supported(cb) : !quantize_supported(cb))
      return fail(TQ_ERR_UNSUPPORTED, "dequantize supports d <= 256 and qjl_m <= 256 (polar: d <= 128, qjl_m <= 128)");
    if (n_seq * n_tok > 0x7FFFFFFF || n_seq > 0x7FFFFFFF)
      return fail(TQ_ERR_UNSUPPORTED, "n_seq * n_tok must stay below 2^31");
    s = current_device_matches(cb);
    if (s != TQ_OK) return s;
    DequantJob job{*codes, n_seq, n_tok, tok_offset, out, out_dt};
    hipError_t e = cb->pq.polar ? launch_polar_dequantize(cb, job, static_cast<hipStream_t>(stream))
                                : launch_dequantize(cb, job, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dequantize launch");
    return TQ_OK;
  } catch (...) {
    return fail(TQ_ERR_ALLOC, "tq_dequantize: unexpected exception");
  }
}

tq_status tq_profile_enable(int32_t on) {
  if (on) {
    for (auto& v : g_prof.rec) {
      for (auto& p : v) { (void)hipEventDestroy(p.a); (void)hipEventDestroy(p.b); }
      v.clear();
    }
  }
  g_prof.on = on != 0;
  return TQ_OK;
}

tq_status tq_profile_durations(int32_t kernel, double* ms, int64_t capacity, int64_t* launches) {
  if (kernel < 0 || kernel > 3) return fail(TQ_ERR_INVALID, "unknown kernel id");
  if (capacity < 0 || (capacity > 0 && !ms)) return fail(TQ_ERR_INVALID, "ms is NULL");
  int64_t i = 0;
  for (auto& p : g_prof.rec[kernel]) {
    if (i >= capacity) break;
    hipError_t e = hipEventSynchronize(p.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float v = 0.f;
    e = hipEventElapsedTime(&v, p.a, p.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    ms[i++] = v;
  }
  if (launches) *launches = (int64_t)g_prof.rec[kernel].size();
  return TQ_OK;
}

tq_status tq_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(TQ_ERR_INVALID, "bytes must be a non-negative multiple of 16");
  if (bytes == 0) return TQ_OK;
  if (!buf || !sink) return fail(TQ_ERR_INVALID, "buf and sink must be non-NULL");
  if (!aligned(buf, 16)) return fail(TQ_ERR_INVALID, "buf must be 16-byte aligned");
  hipError_t e = launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return TQ_OK;
}

tq_status tq_stream_write(void* buf, int64_t bytes, uint32_t value, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(TQ_ERR_INVALID, "bytes must be a non-negative multiple of 16");
  if (bytes == 0) return TQ_OK;
  if (!buf) return fail(TQ_ERR_INVALID, "buf must be non-NULL");
  if (!aligned(buf, 16)) return fail(TQ_ERR_INVALID, "buf must be 16-byte aligned");
  hipError_t e = launch_stream_write(buf, bytes, value, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream write launch");
  return TQ_OK;
}

tq_status tq_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel > 3) return fail(TQ_ERR_INVALID, "unknown kernel id");
  double tot = 0.0;
  for (auto& p : g_prof.rec[kernel]) {
    hipError_t e = hipEventSynchronize(p.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, p.a, p.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    tot += ms;
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = (int64_t)g_prof.rec[kernel].size();
  return TQ_OK;
}

}  // extern "C"
