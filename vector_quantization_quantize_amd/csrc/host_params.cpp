// Host-side construction of the method's parameters: the seeded rotation Pi,
// the seeded Gaussian projection G and the Lloyd-Max codebook.
//
// Sources (web pages about TurboQuant, by title and section):
//  - "TurboQuant deep review" (freelamp.com), breakthrough section: keys are
//    first multiplied by a random orthogonal matrix.  Taken as Haar: QR of a
//    standard-normal matrix with the signs of diag(R) folded into Q.
//  - "TurboQuant tutorial" (gitcode.csdn.net), QJL section: a Gaussian JL
//    matrix with as many outputs as inputs acts on the residual.
//  - "Why KV-cache compression works ..." (nonndazone.ru), sections 3.2 and
//    3.4: centroids are placed where the probability is high and are
//    precomputed once for all tokens.  Taken as the minimum-MSE (Lloyd-Max)
//    quantizer for the law of one coordinate of a uniform unit vector in R^d,
//    density proportional to (1 - z^2)^((d-3)/2) on [-1, 1].
//
// Everything here is float64 and single-threaded per matrix column block;
// results are rounded to float32 once at the end.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "host_params.h"

namespace tqhost {

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood 2014) used as a counter-based generator.
// ---------------------------------------------------------------------------
static constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

static inline uint64_t fmix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t stream_state(uint64_t seed, uint32_t stream) {
  return fmix64(seed + (uint64_t(stream) + 1) * kGamma);
}

// counter c (0-based) of the stream whose state is `state`
static inline uint64_t counter_bits(uint64_t state, uint64_t c) { return fmix64(state + (c + 1) * kGamma); }

void normal_draws(uint64_t seed, uint32_t stream, size_t count, double* out) {
  const uint64_t state = stream_state(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
  const double scale = 1.0 / 9007199254740992.0;  // 2^-53
  for (size_t i = 0; 2 * i < count; ++i) {
    const uint64_t a = counter_bits(state, 2 * i);
    const uint64_t b = counter_bits(state, 2 * i + 1);
    const double u1 = (double(a >> 11) + 1.0) * scale;  // (0, 1]
    const double u2 = double(b >> 11) * scale;          // [0, 1)
    const double radius = std::sqrt(-2.0 * std::log(u1));
    const double theta = two_pi * u2;
    out[2 * i] = radius * std::cos(theta);
    if (2 * i + 1 < count) out[2 * i + 1] = radius * std::sin(theta);
  }
}

// ---------------------------------------------------------------------------
// Householder QR in float64 with the Haar sign convention.
// ---------------------------------------------------------------------------
namespace {

// Run f(j) for j in [lo, hi) on up to `threads` std::threads.
template <class F>
void parallel_columns(int lo, int hi, F&& f) {
  const int count = hi - lo;
  if (count <= 0) return;
  unsigned hw = std::thread::hardware_concurrency();
  int threads = int(std::min<unsigned>(hw == 0 ? 1u : hw, 16u));
  if (count < 64) threads = 1;
  threads = std::min(threads, count);
  if (threads <= 1) {
    for (int j = lo; j < hi; ++j) f(j);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t) {
    const int a = lo + int(int64_t(count) * t / threads);
    const int b = lo + int(int64_t(count) * (t + 1) / threads);
    pool.emplace_back([a, b, &f] {
      for (int j = a; j < b; ++j) f(j);
    });
  }
  for (auto& th : pool) th.join();
}

}  // namespace

// a: d x d row-major on entry.  q: d x d row-major Haar factor on exit.
void haar_from_gaussian(int d, const double* a_rowmajor, double* q_rowmajor) {
  // Work column-major so that reflections touch contiguous columns.
  std::vector<double> A(size_t(d) * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) A[size_t(j) * d + i] = a_rowmajor[size_t(i) * d + j];
  std::vector<double> V(size_t(d) * d, 0.0);  // reflector k stored in column k (rows k..d-1)
  std::vector<double> rdiag(d, 0.0);
  for (int k = 0; k < d; ++k) {
    double* col = &A[size_t(k) * d];
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += col[i] * col[i];
    const double norm = std::sqrt(norm2);
    double* v = &V[size_t(k) * d];
    if (k == d - 1 || norm == 0.0) {
      // nothing left to annihilate: identity reflector
      rdiag[k] = col[k];
      continue;
    }
    const double alpha = col[k] >= 0.0 ? -norm : norm;
    for (int i = k; i < d; ++i) v[i] = col[i];
    v[k] -= alpha;
    double vn2 = 0.0;
    for (int i = k; i < d; ++i) vn2 += v[i] * v[i];
    const double inv = 1.0 / std::sqrt(vn2);
    for (int i = k; i < d; ++i) v[i] *= inv;
    rdiag[k] = alpha;
    // A[k:, j] -= 2 v (v . A[k:, j]) for the trailing columns
    parallel_columns(k + 1, d, [&](int j) {
      double* c = &A[size_t(j) * d];
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * c[i];
      s *= 2.0;
      for (int i = k; i < d; ++i) c[i] -= s * v[i];
    });
  }
  // Q = H_0 H_1 ... H_{d-2}: apply to the identity from the right-most factor.
  std::vector<double> Q(size_t(d) * d, 0.0);  // column-major
  for (int i = 0; i < d; ++i) Q[size_t(i) * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &V[size_t(k) * d];
    bool identity = true;
    for (int i = k; i < d && identity; ++i) identity = (v[i] == 0.0);
    if (identity) continue;
    parallel_columns(k, d, [&](int j) {
      double* c = &Q[size_t(j) * d];
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * c[i];
      s *= 2.0;
      for (int i = k; i < d; ++i) c[i] -= s * v[i];
    });
  }
  // Haar convention: column j of Q times sign(R_jj)
  for (int j = 0; j < d; ++j) {
    const double sgn = rdiag[j] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) q_rowmajor[size_t(i) * d + j] = sgn * Q[size_t(j) * d + i];
  }
}

// ---------------------------------------------------------------------------
// Lloyd-Max codebook for the rotated-coordinate law, by quadrature.
//
// With z = sin(theta), dz = cos(theta) dtheta and the density becomes
// proportional to cos(theta)^(d-2) on (-pi/2, pi/2): smooth for every d >= 2,
// including d = 2 where the z-density has end-point singularities.  Cell
// integrals use composite Gauss-Legendre rules (nodes from Newton iterations
// on the Legendre recurrence).  The normaliser cancels in every centroid.
// ---------------------------------------------------------------------------
namespace {

constexpr int kGL = 20;

struct GaussLegendre {
  double x[kGL], w[kGL];
  GaussLegendre() {
    const double pi = 3.141592653589793238462643383280;
    for (int i = 0; i < kGL; ++i) {
      double t = std::cos(pi * (i + 0.75) / (kGL + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = t;
        for (int n = 2; n <= kGL; ++n) {
          const double p2 = ((2.0 * n - 1.0) * t * p1 - (n - 1.0) * p0) / n;
          p0 = p1;
          p1 = p2;
        }
        dp = kGL * (t * p1 - p0) / (t * t - 1.0);
        const double step = p1 / dp;
        t -= step;
        if (std::fabs(step) < 1e-17) break;
      }
      // recompute derivative at the converged node
      double p0 = 1.0, p1 = t;
      for (int n = 2; n <= kGL; ++n) {
        const double p2 = ((2.0 * n - 1.0) * t * p1 - (n - 1.0) * p0) / n;
        p0 = p1;
        p1 = p2;
      }
      dp = kGL * (t * p1 - p0) / (t * t - 1.0);
      x[i] = t;
      w[i] = 2.0 / ((1.0 - t * t) * dp * dp);
    }
  }
};

const GaussLegendre& gl() {
  static const GaussLegendre rule;
  return rule;
}

// mass and first moment (in z) of the cell z in [za, zb], up to a common
// constant factor
void cell_integrals(int d, double za, double zb, double* m0, double* m1) {
  const double e = double(d) - 2.0;  // exponent of cos(theta)
  const double width_scale = 1.0 / std::sqrt(std::max(e, 1.0));
  const double half_pi = 1.5707963267948966192313216916398;
  double ta = za <= -1.0 ? -half_pi : std::asin(za);
  double tb = zb >= 1.0 ? half_pi : std::asin(zb);
  // beyond 40 standard widths the weight is below exp(-800): drop it
  const double cut = 40.0 * width_scale;
  ta = std::max(ta, -cut);
  tb = std::min(tb, cut);
  *m0 = 0.0;
  *m1 = 0.0;
  if (!(tb > ta)) return;
  const double panel = 0.25 * width_scale;
  int panels = int(std::ceil((tb - ta) / panel));
  panels = std::max(panels, 8);
  const double h = (tb - ta) / panels;
  const GaussLegendre& rule = gl();
  double s0 = 0.0, s1 = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double mid = ta + (p + 0.5) * h;
    double q0 = 0.0, q1 = 0.0;
    for (int i = 0; i < kGL; ++i) {
      const double th = mid + 0.5 * h * rule.x[i];
      const double c = std::cos(th);
      const double wgt = rule.w[i] * (e == 0.0 ? 1.0 : std::exp(e * std::log(c)));
      q0 += wgt;
      q1 += wgt * std::sin(th);
    }
    s0 += 0.5 * h * q0;
    s1 += 0.5 * h * q1;
  }
  *m0 = s0;
  *m1 = s1;
}

// mass and first moment in theta of the cell [ta, tb] of (-pi/2, pi/2)
// under the weight cos(theta)^e (the polar angle laws), up to a common factor
void cell_integrals_theta(double e, double ta, double tb, double* m0, double* m1) {
  const double width_scale = 1.0 / std::sqrt(std::max(e, 1.0));
  const double cut = 40.0 * width_scale;
  ta = std::max(ta, -cut);
  tb = std::min(tb, cut);
  *m0 = 0.0;
  *m1 = 0.0;
  if (!(tb > ta)) return;
  const double panel = 0.25 * width_scale;
  int panels = int(std::ceil((tb - ta) / panel));
  panels = std::max(panels, 8);
  const double h = (tb - ta) / panels;
  const GaussLegendre& rule = gl();
  double s0 = 0.0, s1 = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double mid = ta + (p + 0.5) * h;
    double q0 = 0.0, q1 = 0.0;
    for (int i = 0; i < kGL; ++i) {
      const double th = mid + 0.5 * h * rule.x[i];
      const double wgt = rule.w[i] * (e == 0.0 ? 1.0 : std::exp(e * std::log(std::cos(th))));
      q0 += wgt;
      q1 += wgt * th;
    }
    s0 += 0.5 * h * q0;
    s1 += 0.5 * h * q1;
  }
  *m0 = s0;
  *m1 = s1;
}

// inverse standard normal CDF (Acklam's rational approximation, refined by
// one Halley step) - only used for the starting levels
double norm_ppf(double p) {
  static const double a[] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                             1.383577518672690e+02, -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                             6.680131188771972e+01, -1.328068155288572e+01};
  static const double c[] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                             -2.549671010115381e+00, 4.374664141464968e+00, 2.938163982698783e+00};
  static const double dd[] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                              3.754408661907416e+00};
  double x;
  if (p < 0.02425) {
    const double q = std::sqrt(-2.0 * std::log(p));
    x = (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((dd[0] * q + dd[1]) * q + dd[2]) * q + dd[3]) * q + 1.0);
  } else if (p > 1.0 - 0.02425) {
    const double q = std::sqrt(-2.0 * std::log(1.0 - p));
    x = -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((dd[0] * q + dd[1]) * q + dd[2]) * q + dd[3]) * q + 1.0);
  } else {
    const double q = p - 0.5, r = q * q;
    x = (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
        (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
  }
  const double e = 0.5 * std::erfc(-x / std::sqrt(2.0)) - p;
  const double u = e * std::sqrt(2.0 * 3.141592653589793) * std::exp(x * x / 2.0);
  return x - u / (1.0 + x * u / 2.0);
}

}  // namespace

int lloyd_max_sphere(int d, int levels, double* c) {
  if (levels == 1) {
    c[0] = 0.0;
    return 0;
  }
  std::vector<double> cur(levels), nxt(levels), t(levels + 1);
  for (int i = 0; i < levels; ++i) {
    const double v = norm_ppf((i + 0.5) / levels) / std::sqrt(double(d));
    cur[i] = std::max(-0.999, std::min(0.999, v));
  }
  int settle = -1, near = 0;
  for (int it = 0; it < 200000; ++it) {
    t[0] = -1.0;
    t[levels] = 1.0;
    for (int i = 1; i < levels; ++i) t[i] = 0.5 * (cur[i - 1] + cur[i]);
    for (int i = 0; i < levels; ++i) {
      double m0, m1;
      cell_integrals(d, t[i], t[i + 1], &m0, &m1);
      nxt[i] = m1 / m0;
    }
    double delta = 0.0, big = 0.0;
    for (int i = 0; i < levels; ++i) {
      const double sym = 0.5 * (nxt[i] - nxt[levels - 1 - i]);
      delta = std::max(delta, std::fabs(sym - cur[i]));
      big = std::max(big, std::fabs(sym));
      t[i] = sym;  // reuse as scratch
    }
    for (int i = 0; i < levels; ++i) cur[i] = t[i];
    const double rel = delta / big;
    if (settle < 0 && rel <= 1.4210854715202004e-14 /* 2^-46 */) settle = 20;
    near = rel <= 1e-11 ? near + 1 : 0;
    if (near >= 300 || (settle >= 0 && --settle <= 0)) {
      for (int i = 0; i < levels; ++i) c[i] = cur[i];
      return 0;
    }
  }
  return -1;
}

// ---------------------------------------------------------------------------
// Polar angle codebooks.  A level-l angle psi (l >= 2) compares the lengths of
// two m = 2^(l-1)-dimensional Gaussian blocks: its density is proportional to
// sin^(m-1) psi cos^(m-1) psi on [0, pi/2].  With theta = 2 psi - pi/2 that is
// cos(theta)^(m-1) on (-pi/2, pi/2); Lloyd-Max commutes with the linear map,
// so the levels are computed in theta and mapped back.
// ---------------------------------------------------------------------------
int lloyd_max_polar_level(int m, int levels, double* psi) {
  const double half_pi = 1.5707963267948966192313216916398;
  const double e = double(m) - 1.0;
  std::vector<double> cur(levels), nxt(levels), t(levels + 1);
  for (int i = 0; i < levels; ++i) {
    const double v = norm_ppf((i + 0.5) / levels) / std::sqrt(double(m));
    cur[i] = std::max(-0.999 * half_pi, std::min(0.999 * half_pi, v));
  }
  int settle = -1, near = 0;
  for (int it = 0; it < 200000; ++it) {
    t[0] = -half_pi;
    t[levels] = half_pi;
    for (int i = 1; i < levels; ++i) t[i] = 0.5 * (cur[i - 1] + cur[i]);
    for (int i = 0; i < levels; ++i) {
      double m0, m1;
      cell_integrals_theta(e, t[i], t[i + 1], &m0, &m1);
      nxt[i] = m1 / m0;
    }
    double delta = 0.0, big = 0.0;
    for (int i = 0; i < levels; ++i) {
      const double sym = 0.5 * (nxt[i] - nxt[levels - 1 - i]);
      delta = std::max(delta, std::fabs(sym - cur[i]));
      big = std::max(big, std::fabs(sym));
      t[i] = sym;
    }
    for (int i = 0; i < levels; ++i) cur[i] = t[i];
    const double rel = delta / big;
    if (settle < 0 && rel <= 1.4210854715202004e-14 /* 2^-46 */) settle = 20;
    near = rel <= 1e-11 ? near + 1 : 0;
    if (near >= 300 || (settle >= 0 && --settle <= 0)) {
      for (int i = 0; i < levels; ++i) psi[i] = 0.5 * cur[i] + 0.5 * half_pi;
      return 0;
    }
  }
  return -1;
}

int polar_level_codebook(int d, int bits, int level, float* levels, float* thresholds) {
  if (d < 2 || d > 4096 || (d & (d - 1)) != 0 || bits < 2 || bits > 5) return -1;
  int nl = 0;
  while ((1 << nl) < d) ++nl;
  if (level < 1 || level > nl) return -1;
  const int L = 1 << (bits - 1);
  std::vector<float> c32(L);
  if (level == 1) {
    // uniform quantizer of the circle: cells [k, k+1) 2 pi / L, levels at the centres
    const double two_pi = 6.283185307179586476925286766559;
    for (int i = 0; i < L; ++i) c32[i] = float((i + 0.5) * two_pi / L);
    if (levels) std::memcpy(levels, c32.data(), sizeof(float) * L);
    if (thresholds)
      for (int i = 0; i + 1 < L; ++i) thresholds[i] = float((i + 1) * two_pi / L);
    return 0;
  }
  std::vector<double> c(L);
  if (lloyd_max_polar_level(1 << (level - 1), L, c.data()) != 0) return -2;
  for (int i = 0; i < L; ++i) c32[i] = float(c[i]);
  if (levels) std::memcpy(levels, c32.data(), sizeof(float) * L);
  if (thresholds)
    for (int i = 0; i + 1 < L; ++i) thresholds[i] = float(0.5 * (double(c32[i]) + double(c32[i + 1])));
  return 0;
}

// ---------------------------------------------------------------------------
// Randomized Hadamard rotation: Pi = H diag(sigma) / sqrt(d), H the Sylvester
// Hadamard matrix (H[i][j] = (-1)^popcount(i & j)), sigma_j = -1 when the top
// bit of counter j of stream 2 is set, else +1.
// ---------------------------------------------------------------------------
int hadamard_rotation(int d, uint64_t seed, float* pi) {
  if (d < 2 || d > 4096 || (d & (d - 1)) != 0) return -1;
  const uint64_t state = stream_state(seed, 2);
  const float a = float(1.0 / std::sqrt(double(d)));
  std::vector<float> sigma(d);
  for (int j = 0; j < d; ++j) sigma[j] = (counter_bits(state, uint64_t(j)) >> 63) ? -a : a;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) pi[size_t(i) * d + j] = (__builtin_popcount(unsigned(i & j)) & 1) ? -sigma[j] : sigma[j];
  return 0;
}

// ---------------------------------------------------------------------------
// Public assembly
// ---------------------------------------------------------------------------
int build_params(int d, int bits, uint64_t seed, float* pi, float* g, float* centroids, float* thresholds) {
  if (d < 2 || d > 4096 || bits < 2 || bits > 5) return -1;
  const size_t dd = size_t(d) * d;
  std::vector<double> buf(dd);
  if (pi) {
    std::vector<double> q(dd);
    normal_draws(seed, 0, dd, buf.data());
    haar_from_gaussian(d, buf.data(), q.data());
    for (size_t i = 0; i < dd; ++i) pi[i] = float(q[i]);
  }
  if (g) {
    // float16 precision (one rounding from float64): exact as a matrix-core
    // operand, so the projection needs no second piece of G
    normal_draws(seed, 1, dd, buf.data());
    for (size_t i = 0; i < dd; ++i) g[i] = float(static_cast<_Float16>(buf[i]));
  }
  if (centroids || thresholds) {
    const int levels = 1 << (bits - 1);
    std::vector<double> c(levels);
    if (lloyd_max_sphere(d, levels, c.data()) != 0) return -2;
    std::vector<float> c32(levels);
    for (int i = 0; i < levels; ++i) c32[i] = float(c[i]);
    if (centroids) std::memcpy(centroids, c32.data(), sizeof(float) * levels);
    if (thresholds)
      for (int i = 0; i + 1 < levels; ++i)
        thresholds[i] = float(0.5 * (double(c32[i]) + double(c32[i + 1])));
  }
  return 0;
}

}  // namespace tqhost
