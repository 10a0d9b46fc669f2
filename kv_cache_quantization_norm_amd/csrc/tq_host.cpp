// Host half of libtq: the seeded Pi/S generator, the Lloyd-Max codebook
// solver, plane and workspace sizing, status strings.
//
// Pages: "TurboQuant QJL投影深度剖析", section 2 (rotation from a QR
// decomposition, Lloyd-Max codebook for the rotated-coordinate law, Gaussian
// QJL sketch) and section 6 (seed 42 + 7 * layer per layer).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {

namespace {
thread_local char g_last_error[512] = "";
}

tq_status fail(tq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

tq_status check_format(const tq_format* f, bool device) {
  if (!f) return fail(TQ_ERR_INVALID_ARG, "format is NULL");
  if (f->d < 8 || f->d % 8 != 0) return fail(TQ_ERR_INVALID_ARG, "d=%d must be a positive multiple of 8", f->d);
  if (f->k_bits < 0 || f->k_bits == 1 || (f->k_bits > 5 && f->k_bits != 8))
    return fail(TQ_ERR_UNSUPPORTED, "k_bits=%d (0 for fp16 keys, else 2..5 or 8)", f->k_bits);
  if (f->v_bits < 0 || f->v_bits > 4)
    return fail(TQ_ERR_UNSUPPORTED, "v_bits=%d (0 for fp16 values, else 1 to 4)", f->v_bits);
  if (device && f->d != 128) return fail(TQ_ERR_UNSUPPORTED, "device kernels need d=128, got %d", f->d);
  return TQ_OK;
}

SplitPlan plan_decode(int d, int n_layers, int batch, int n_kv_heads, int n_q_heads,
                      int64_t max_seq_len, int max_workgroups) {
  SplitPlan p;
  const int group = n_q_heads / n_kv_heads;
  p.n_head_groups = (group + kMaxGroup - 1) / kMaxGroup;
  p.problems = int64_t(n_layers) * batch * n_kv_heads * p.n_head_groups;
  const int64_t len = max_seq_len > 0 ? max_seq_len : 1;
  const int64_t cpp = (len + kChunk - 1) / kChunk;
  const int64_t total = p.problems * cpp;
  // Balanced split: one workgroup per CU, equal runs of chunks, each with at
  // least one chunk per wave; a run may cross from one problem into the next.
  int64_t wgs = (total + kDecodeWaves - 1) / kDecodeWaves;
  if (wgs > max_workgroups) wgs = max_workgroups;
  const int64_t cpw_b = (total + wgs - 1) / wgs;
  p.chunks_per_problem = cpp;
  p.chunks_per_wg = cpw_b;
  // Aligned split: each problem cut into k equal runs (k workgroups per
  // problem, k = CUs / problems), so that no run crosses a problem boundary.
  // A crossing costs a workgroup about kCrossingChunks chunks of time (a
  // second pipeline start and a second merge), so the aligned split is taken
  // when its runs are at most that much longer than the balanced ones.  The
  // problem is then padded to k runs of equal length; padding chunks hold no
  // tokens and are never dealt.
  int64_t k = max_workgroups / p.problems;
  if (k > cpp / kDecodeWaves) k = cpp / kDecodeWaves;   // at least one chunk per wave
  if (k >= 1 && cpp % cpw_b != 0) {
    const int64_t cpw_a = (cpp + k - 1) / k;
    if (cpw_a <= cpw_b + kCrossingChunks) {
      p.chunks_per_problem = k * cpw_a;
      p.chunks_per_wg = cpw_a;
    }
  }
  p.n_workgroups = (p.problems * p.chunks_per_problem + p.chunks_per_wg - 1) / p.chunks_per_wg;
  // A problem of C chunks overlaps at most ceil((C - 1) / W) + 1 ranges of W.
  p.seg_max = (p.chunks_per_problem - 1 + p.chunks_per_wg - 1) / p.chunks_per_wg + 1;
  // Ragged split: ranges of at least half the balanced length (so a batch
  // whose sequences fill at least half of max_len is split evenly).
  p.cpp_real = cpp;
  p.cpw_min = cpw_b / 2 > 1 ? cpw_b / 2 : 1;
  const int64_t pad_max = kRaggedCrossChunks + kContainChunks;
  const int64_t seg_r = batch > 1 ? (cpp + pad_max - 1 + p.cpw_min - 1) / p.cpw_min + 1 : 0;
  p.seg_cap = seg_r > p.seg_max ? seg_r : p.seg_max;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  p.qprep_bytes = align(size_t(n_layers) * batch * n_q_heads * 2 * d * sizeof(float));
  p.counter_offset = p.qprep_bytes;
  p.counter_bytes = align(size_t(p.problems + n_layers + 1) * sizeof(uint32_t));
  p.partial_offset = p.counter_offset + p.counter_bytes;
  p.partial_bytes = align(size_t(n_layers) * batch * n_q_heads * p.seg_cap * (d + 2) * sizeof(float));
  p.red_offset = p.partial_offset + p.partial_bytes;
  p.red_bytes = align(size_t(p.n_workgroups) * kDecodeWaves * kMaxGroup * d * sizeof(float));
  p.total_bytes = p.red_offset + p.red_bytes;
  return p;
}

TailPlan plan_decode_tail(int d, int n_layers, int batch, int n_kv_heads, int n_q_heads, int64_t max_seq_len,
                          int64_t max_tail_len) {
  TailPlan t;
  t.packed = plan_decode(d, n_layers, batch, n_kv_heads, n_q_heads, max_seq_len);
  t.tail = plan_decode(d, n_layers, batch, n_kv_heads, n_q_heads, max_tail_len);
  t.seg_total = t.packed.seg_cap + t.tail.seg_cap;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  t.qplain_offset = t.packed.qprep_bytes;
  t.partial_offset = 2 * t.packed.qprep_bytes;
  t.counter_offset =
      t.partial_offset + align(size_t(n_layers) * batch * n_q_heads * t.seg_total * (d + 2) * sizeof(float));
  t.red_offset = t.counter_offset + t.packed.counter_bytes;
  t.total_bytes = t.red_offset + (t.packed.red_bytes > t.tail.red_bytes ? t.packed.red_bytes : t.tail.red_bytes);
  return t;
}

// ---------------------------------------------------------------------------
// Seeded normal stream: SplitMix64 (Steele, Lea, Flood 2014) output n of seed
// s is mix(s + (n+1) * 0x9E3779B97F4A7C15); a uniform is
// ((z >> 11) + 0.5) * 2^-53; normal i = sqrt(-2 ln u_{2i}) cos(2 pi u_{2i+1})
// (Box-Muller, cosine branch).
namespace {

inline uint64_t splitmix_at(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline double uniform_at(uint64_t seed, uint64_t n) {
  return (double(splitmix_at(seed, n) >> 11) + 0.5) * 0x1.0p-53;
}

inline double normal_at(uint64_t seed, uint64_t i) {
  const double u1 = uniform_at(seed, 2 * i);
  const double u2 = uniform_at(seed, 2 * i + 1);
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(2.0 * M_PI * u2);
}

// Householder QR of the row-major n x n matrix a (overwritten by R); returns
// Q explicitly in q (row-major).
void householder_qr(int n, std::vector<double>& a, std::vector<double>& q) {
  std::vector<double> vs(size_t(n) * n, 0.0);  // reflector k stored in row k (entries k..n-1)
  std::vector<double> w(n);
  for (int k = 0; k < n; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < n; ++i) norm2 += a[size_t(i) * n + k] * a[size_t(i) * n + k];
    const double norm = std::sqrt(norm2);
    double* v = &vs[size_t(k) * n];
    if (norm == 0.0) continue;
    const double x0 = a[size_t(k) * n + k];
    const double alpha = x0 >= 0 ? -norm : norm;  // reflect onto alpha e_k, no cancellation
    for (int i = k; i < n; ++i) v[i] = a[size_t(i) * n + k];
    v[k] -= alpha;
    double vn2 = 0.0;
    for (int i = k; i < n; ++i) vn2 += v[i] * v[i];
    const double vn = std::sqrt(vn2);
    if (vn == 0.0) continue;
    for (int i = k; i < n; ++i) v[i] /= vn;
    // A[k:, k:] -= 2 v (v^T A[k:, k:])
    for (int j = k; j < n; ++j) {
      double dot = 0.0;
      for (int i = k; i < n; ++i) dot += v[i] * a[size_t(i) * n + j];
      for (int i = k; i < n; ++i) a[size_t(i) * n + j] -= 2.0 * v[i] * dot;
    }
  }
  // Q = H_0 H_1 ... H_{n-1}: apply the reflectors to I from the last one.
  q.assign(size_t(n) * n, 0.0);
  for (int i = 0; i < n; ++i) q[size_t(i) * n + i] = 1.0;
  for (int k = n - 1; k >= 0; --k) {
    const double* v = &vs[size_t(k) * n];
    for (int j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int i = k; i < n; ++i) dot += v[i] * q[size_t(i) * n + j];
      if (dot == 0.0) continue;
      for (int i = k; i < n; ++i) q[size_t(i) * n + j] -= 2.0 * v[i] * dot;
    }
  }
}

// ---------------------------------------------------------------------------
// Coordinate law f_d(t) = C (1 - t^2)^((d-3)/2) and its Lloyd-Max quantiser.

struct GaussLegendre {
  std::vector<double> x, w;  // nodes / weights on [-1, 1]
  explicit GaussLegendre(int n) : x(n), w(n) {
    // Newton iteration on P_n from the Chebyshev-like first guess.
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 1.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-17) break;
      }
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

struct CoordinateLaw {
  int d;
  double c;      // normalising constant
  double e;      // exponent (d-3)/2
  double scale;  // typical spread 1/sqrt(d)
  GaussLegendre gl{24};

  explicit CoordinateLaw(int d_) : d(d_) {
    c = std::exp(std::lgamma(d / 2.0) - std::lgamma((d - 1) / 2.0)) / std::sqrt(M_PI);
    e = (d - 3) / 2.0;
    scale = 1.0 / std::sqrt(double(d));
  }
  double density(double t) const {
    const double u = 1.0 - t * t;
    return u <= 0.0 ? 0.0 : c * std::pow(u, e);
  }
  // int_0^t f (t may be negative), composite Gauss-Legendre on panels no
  // wider than a quarter of the spread.
  double mass_from_zero(double t) const {
    if (t == 0.0) return 0.0;
    const double sgn = t < 0 ? -1.0 : 1.0;
    const double b = std::fmin(std::fabs(t), 1.0);
    int panels = int(std::ceil(b / (0.25 * scale)));
    if (panels < 1) panels = 1;
    const double h = b / panels;
    double sum = 0.0;
    for (int p = 0; p < panels; ++p) {
      const double a0 = p * h, mid = a0 + 0.5 * h;
      double ps = 0.0;
      for (size_t i = 0; i < gl.x.size(); ++i) ps += gl.w[i] * density(mid + 0.5 * h * gl.x[i]);
      sum += 0.5 * h * ps;
    }
    return sgn * sum;
  }
  // int_a^b f (a <= b), the same panels over [a, b] only.
  double mass(double a, double b) const {
    a = std::fmax(a, -1.0);
    b = std::fmin(b, 1.0);
    if (b <= a) return 0.0;
    int panels = int(std::ceil((b - a) / (0.25 * scale)));
    if (panels < 1) panels = 1;
    const double h = (b - a) / panels;
    double sum = 0.0;
    for (int p = 0; p < panels; ++p) {
      const double mid = a + (p + 0.5) * h;
      double ps = 0.0;
      for (size_t i = 0; i < gl.x.size(); ++i) ps += gl.w[i] * density(mid + 0.5 * h * gl.x[i]);
      sum += 0.5 * h * ps;
    }
    return sum;
  }
  // Closed-form first moment: int_a^b t f(t) dt.
  double first_moment(double a, double b) const {
    const double ex = (d - 1) / 2.0;
    const double ua = std::fmax(0.0, 1.0 - a * a), ub = std::fmax(0.0, 1.0 - b * b);
    return c / (d - 1) * (std::pow(ua, ex) - std::pow(ub, ex));
  }
};

}  // namespace
}  // namespace tq

extern "C" {

tq_status tq_tail_policy(int32_t batch, const int32_t* packed_len, const int32_t* tail_len,
                         int32_t min_compress_tokens, int32_t keep_recent, int32_t* n_flush) {
  using namespace tq;
  clear_error();
  if (batch < 0 || min_compress_tokens < 0 || keep_recent < 0)
    return fail(TQ_ERR_INVALID_ARG, "batch=%d min_compress_tokens=%d keep_recent=%d", batch, min_compress_tokens,
                keep_recent);
  if (batch > 0 && (!packed_len || !tail_len || !n_flush))
    return fail(TQ_ERR_INVALID_ARG, "packed_len, tail_len or n_flush is NULL");
  for (int32_t b = 0; b < batch; ++b)
    if (packed_len[b] < 0 || tail_len[b] < 0)
      return fail(TQ_ERR_INVALID_ARG, "sequence %d: packed_len=%d tail_len=%d", b, packed_len[b], tail_len[b]);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t total = int64_t(packed_len[b]) + tail_len[b];
    const int64_t movable = int64_t(tail_len[b]) - keep_recent;
    n_flush[b] = total >= min_compress_tokens && movable >= kVBlock ? int32_t(movable / kVBlock * kVBlock) : 0;
  }
  return TQ_OK;
}

uint64_t tq_layer_seed(int32_t layer) { return uint64_t(42 + 7 * int64_t(layer)); }

tq_status tq_make_rotations(int32_t d, uint64_t seed, float* pi, float* s, float* pi_s) {
  using namespace tq;
  clear_error();
  if (d < 3 || d > 1024) return fail(TQ_ERR_INVALID_ARG, "d=%d out of [3, 1024]", d);
  if (!pi || !s) return fail(TQ_ERR_INVALID_ARG, "pi and s must be non-NULL");
  const size_t n2 = size_t(d) * d;
  std::vector<double> g(n2), q;
  for (size_t i = 0; i < n2; ++i) g[i] = normal_at(seed, i);
  householder_qr(d, g, q);  // g now holds R
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      const double r = g[size_t(j) * d + j];
      const double sg = r < 0 ? -1.0 : 1.0;
      pi[size_t(i) * d + j] = float(q[size_t(i) * d + j] * sg);
    }
  for (size_t i = 0; i < n2; ++i) s[i] = float(normal_at(seed, n2 + i));
  if (pi_s) {
    // M = S Pi^T from the stored fp32 values, accumulated in double.
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += double(s[size_t(i) * d + k]) * double(pi[size_t(j) * d + k]);
        pi_s[size_t(i) * d + j] = float(acc);
      }
  }
  return TQ_OK;
}

tq_status tq_make_codebook(int32_t d, int32_t bits, double* centroids, double* boundaries) {
  using namespace tq;
  clear_error();
  if (d < 3 || d > 65536) return fail(TQ_ERR_INVALID_ARG, "d=%d out of [3, 65536]", d);
  if (bits < 1 || bits > 8) return fail(TQ_ERR_INVALID_ARG, "bits=%d out of [1, 8]", bits);
  if (!centroids || (bits > 0 && !boundaries)) return fail(TQ_ERR_INVALID_ARG, "NULL output");
  const int n = 1 << bits;
  CoordinateLaw law(d);
  // Start from the cell mid-quantiles (bisection on the CDF).
  std::vector<double> c(n), t(n - 1), cdf(n + 1);
  for (int k = 0; k < n; ++k) {
    const double target = (k + 0.5) / n - 0.5;  // mass from zero
    double lo = -1.0, hi = 1.0;
    for (int it = 0; it < 80; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (law.mass_from_zero(mid) < target) lo = mid; else hi = mid;
    }
    c[k] = 0.5 * (lo + hi);
  }
  // Lloyd iteration: boundaries at midpoints, centroids at cell means.  Up
  // to 16 levels the cell masses are differences of masses from zero and the
  // iteration runs to a step below 1e-15.  With more levels the cells are
  // narrow: each mass is integrated over its cell alone, and since Lloyd's
  // iteration then contracts slowly (rate about 1 - 6e-4 at 128 levels) and
  // the step settles at a rounding floor near 1e-13, it stops after 40000
  // iterations once the step is below 1e-12 (within about 2e-10 of the fixed
  // point).
  const bool wide = n > 16;
  for (int it = 0; it < 200000; ++it) {
    for (int k = 0; k + 1 < n; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    if (!wide) {
      cdf[0] = -0.5;
      cdf[n] = 0.5;
      for (int k = 0; k + 1 < n; ++k) cdf[k + 1] = law.mass_from_zero(t[k]);
    }
    double step = 0.0;
    for (int k = 0; k < n; ++k) {
      const double a = k == 0 ? -1.0 : t[k - 1];
      const double b = k == n - 1 ? 1.0 : t[k];
      const double m0 = wide ? law.mass(a, b) : cdf[k + 1] - cdf[k];
      const double ck = law.first_moment(a, b) / m0;
      step = std::fmax(step, std::fabs(ck - c[k]));
      c[k] = ck;
    }
    if (step < 1e-15 || (wide && it >= 40000 && step < 1e-12)) break;
  }
  // The law is symmetric: project onto exact antisymmetry (removes rounding
  // noise; the middle boundary becomes exactly 0).
  std::vector<double> cs(n);
  for (int k = 0; k < n; ++k) cs[k] = 0.5 * (c[k] - c[n - 1 - k]);
  for (int k = 0; k < n; ++k) centroids[k] = cs[k];
  for (int k = 0; k + 1 < n; ++k) boundaries[k] = 0.5 * (cs[k] + cs[k + 1]);
  return TQ_OK;
}

float tq_fp16_operand_scale(const float* centroids, int32_t n) {
  if (!centroids || n < 1 || n > 256) return 1.f;
  // distinct nonzero finite magnitudes, ascending
  std::vector<float> m;
  for (int k = 0; k < n; ++k) {
    const float a = std::fabs(centroids[k]);
    if (a > 0.f && std::isfinite(a)) m.push_back(a);
  }
  std::sort(m.begin(), m.end());
  m.erase(std::unique(m.begin(), m.end()), m.end());
  if (m.empty()) return 1.f;
  auto rel_err = [&](double alpha) {
    double worst = 0.0;
    for (float mk : m) {
      const float x = float(alpha * double(mk));
      const double r = double(float(_Float16(x)));
      worst = std::fmax(worst, std::fabs(r - double(x)) / double(x));
    }
    return worst;
  };
  double best = INFINITY, best_alpha = 1.0;
  for (float mi : m) {
    // the fp16 values v in [mi, 2 mi): alpha = v / mi
    int e = 0;
    std::frexp(double(mi), &e);   // mi in [2^(e-1), 2^e)
    const double ulp = std::ldexp(1.0, e - 1 - 10);
    for (double v = std::ceil(double(mi) / ulp) * ulp; v < 2.0 * double(mi);
         v += (v < std::ldexp(1.0, e) ? ulp : 2.0 * ulp)) {
      const double alpha = v / double(mi);
      if (!(alpha >= 1.0 && alpha < 2.0)) continue;
      const double err = rel_err(alpha);
      if (err < best || (err == best && alpha < best_alpha)) {
        best = err;
        best_alpha = alpha;
      }
    }
  }
  return float(best_alpha);
}

tq_status tq_cache_plane_bytes(const tq_format* fmt, int32_t n_layers, int32_t n_kv_heads,
                               int64_t capacity, size_t out_bytes[8]) {
  using namespace tq;
  clear_error();
  tq_status st = check_format(fmt, false);
  if (st) return st;
  if (!out_bytes) return fail(TQ_ERR_INVALID_ARG, "out_bytes is NULL");
  if (n_layers <= 0 || n_kv_heads <= 0 || capacity <= 0 || capacity % kVBlock)
    return fail(TQ_ERR_INVALID_ARG, "bad sizes (layers=%d heads=%d capacity=%lld; capacity must be a positive multiple of 32)",
                n_layers, n_kv_heads, (long long)capacity);
  const size_t slots = size_t(n_layers) * n_kv_heads * size_t(capacity);
  const size_t d = size_t(fmt->d);
  for (int i = 0; i < 8; ++i) out_bytes[i] = 0;
  if (fmt->k_bits > 0) {
    out_bytes[0] = slots * d * size_t(fmt->k_bits - 1) / 8;
    out_bytes[1] = slots * d / 8;
    out_bytes[2] = slots * 4;
    out_bytes[3] = slots * 4;
  } else {
    out_bytes[4] = slots * d * 2;
  }
  if (fmt->v_bits > 0) {
    out_bytes[5] = slots * d * size_t(fmt->v_bits) / 8;
    out_bytes[6] = slots * 4;
  } else {
    out_bytes[7] = slots * d * 2;
  }
  return TQ_OK;
}

tq_status tq_decode_split(const tq_format* fmt, int32_t n_layers, int32_t batch, int32_t n_kv_heads,
                          int32_t n_q_heads, int64_t max_seq_len, int64_t out[5]) {
  using namespace tq;
  clear_error();
  if (!out) return fail(TQ_ERR_INVALID_ARG, "out is NULL");
  tq_status st = check_format(fmt, false);
  if (st) return st;
  if (n_layers <= 0 || batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads ||
      max_seq_len < 0)
    return fail(TQ_ERR_INVALID_ARG, "sizes");
  const SplitPlan p = plan_decode(fmt->d, n_layers, batch, n_kv_heads, n_q_heads, max_seq_len);
  out[0] = p.problems;
  out[1] = p.chunks_per_problem;
  out[2] = p.chunks_per_wg;
  out[3] = p.n_workgroups;
  out[4] = p.seg_max;
  return TQ_OK;
}

size_t tq_decode_workspace_bytes(const tq_format* fmt, int32_t n_layers, int32_t batch,
                                 int32_t n_kv_heads, int32_t n_q_heads, int64_t max_seq_len) {
  using namespace tq;
  if (check_format(fmt, false) != TQ_OK || n_layers <= 0 || batch <= 0 || n_kv_heads <= 0 ||
      n_q_heads <= 0 || n_q_heads % n_kv_heads || max_seq_len < 0)
    return 0;
  return plan_decode(fmt->d, n_layers, batch, n_kv_heads, n_q_heads, max_seq_len).total_bytes;
}

size_t tq_decode_tail_workspace_bytes(const tq_format* fmt, int32_t n_layers, int32_t batch, int32_t n_kv_heads,
                                      int32_t n_q_heads, int64_t max_seq_len, int64_t max_tail_len) {
  using namespace tq;
  if (check_format(fmt, false) != TQ_OK || n_layers <= 0 || batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 ||
      n_q_heads % n_kv_heads || max_seq_len < 0 || max_tail_len < 0)
    return 0;
  return plan_decode_tail(fmt->d, n_layers, batch, n_kv_heads, n_q_heads, max_seq_len, max_tail_len).total_bytes;
}

const char* tq_status_string(tq_status st) {
  switch (st) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_APPEND_TIMEOUT: return "TQ_ERR_APPEND_TIMEOUT";
    default: return "TQ_ERR_UNKNOWN";
  }
}

const char* tq_last_error(void) { return tq::g_last_error; }

}  // extern "C"
