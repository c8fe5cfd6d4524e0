// C ABI of libtq: argument checking, handle management and dispatch to the
// HIP kernels.  See include/tq.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "host_params.h"
#include "tq_internal.h"

namespace {

bool trace_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("TQ_TRACE");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

void free_device(tq_ctx* h) {
  float** ptrs[] = {&h->d_pi, &h->d_piT, &h->d_g, &h->d_gT, &h->d_piT128, &h->d_sT128};
  for (float** p : ptrs) {
    if (*p) (void)hipFree(*p);
    *p = nullptr;
  }
  uint16_t** frags[] = {&h->d_pi_frag, &h->d_g_frag, &h->d_dq_frag, &h->d_ds_frag};
  for (uint16_t** p : frags) {
    if (*p) (void)hipFree(*p);
    *p = nullptr;
  }
  tqdev::free_quantize_gemm(h);
  if (h->d_polar_tab) (void)hipFree(h->d_polar_tab);
  h->d_polar_tab = nullptr;
  if (h->d_hsigma) (void)hipFree(h->d_hsigma);
  h->d_hsigma = nullptr;
}

uint16_t f16_bits(float x) {
  const _Float16 h = static_cast<_Float16>(x);
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

float f16_value(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

int upload_u16(uint16_t** dst, const std::vector<uint16_t>& src) {
  const size_t bytes = src.size() * sizeof(uint16_t);
  if (hipMalloc(reinterpret_cast<void**>(dst), bytes) != hipSuccess) {
    *dst = nullptr;
    return TQ_ENOMEM;
  }
  return hipMemcpy(*dst, src.data(), bytes, hipMemcpyHostToDevice) == hipSuccess ? TQ_OK : TQ_EHIP;
}

// Register fragments of the d = 128 matrix-core quantize kernel (see
// quantize_mfma.hip).  Rows of a wave's 32-row slice are permuted: MFMA row m
// carries coordinate 16((m/4)%2) + 4(m/8) + m%4 of word w, so accumulator
// element r of lane l is coordinate 32w + 16(l/32) + r.
//   Pi: two f16 pieces of 2^12 Pi; lane l of word w, step s holds
//       Pi[32w + row(l%32)][16s + 8(l/32) + e].
//   G:  two f16 pieces of 2^10 G; lane l holds G[32w + row(l%32)][j] with
//       j = 32(s/2) + 16(l/32) + 8(s%2) + e, the residual coordinate that lane
//       group l/32 supplies in K-slot e of step s.
int build_fragments(tq_ctx* h) {
  const int d = h->d;
  if (d != 128) return TQ_OK;
  auto row_of = [](int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); };
  std::vector<uint16_t> pf(size_t(4) * 8 * 2 * 64 * 8), gf(size_t(4) * 8 * 2 * 64 * 8);
  for (int w = 0; w < 4; ++w)
    for (int s = 0; s < 8; ++s)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
          const int row = 32 * w + row_of(l & 31);
          const float x = h->pi[size_t(row) * d + 16 * s + 8 * (l >> 5) + e] * 4096.0f;
          const uint16_t phi = f16_bits(x);
          pf[(((size_t(w) * 8 + s) * 2 + 0) * 64 + l) * 8 + e] = phi;
          pf[(((size_t(w) * 8 + s) * 2 + 1) * 64 + l) * 8 + e] = f16_bits(x - f16_value(phi));
          const int j = 32 * (s >> 1) + 16 * (l >> 5) + 8 * (s & 1) + e;
          const float gs = h->g[size_t(row) * d + j] * 1024.0f;
          const uint16_t ghi = f16_bits(gs);
          gf[(((size_t(w) * 8 + s) * 2 + 0) * 64 + l) * 8 + e] = ghi;
          gf[(((size_t(w) * 8 + s) * 2 + 1) * 64 + l) * 8 + e] = f16_bits(gs - f16_value(ghi));
        }
  // stage-1 reconstruction: lane l of word w, step s holds
  // 2^12 Pi[16s + 8(l/32) + e][32w + l%32] (B operand, N = output coordinate)
  std::vector<uint16_t> df(size_t(4) * 8 * 2 * 64 * 8);
  for (int w = 0; w < 4; ++w)
    for (int s = 0; s < 8; ++s)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
          const float x = h->pi[size_t(16 * s + 8 * (l >> 5) + e) * d + 32 * w + (l & 31)] * 4096.0f;
          const uint16_t hi = f16_bits(x);
          df[(((size_t(w) * 8 + s) * 2 + 0) * 64 + l) * 8 + e] = hi;
          df[(((size_t(w) * 8 + s) * 2 + 1) * 64 + l) * 8 + e] = f16_bits(x - f16_value(hi));
        }
  // corrected reconstruction: the same layout for 2^10 S, S = G Pi (computed
  // in float64 from the float32 matrices): lane l of word w, step s holds
  // 2^10 S[16s + 8(l/32) + e][32w + l%32]
  std::vector<double> sm(size_t(d) * d, 0.0);
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < d; ++k) {
      const double gik = h->g[size_t(i) * d + k];
      for (int j = 0; j < d; ++j) sm[size_t(i) * d + j] += gik * double(h->pi[size_t(k) * d + j]);
    }
  std::vector<uint16_t> sf(size_t(4) * 8 * 2 * 64 * 8);
  for (int w = 0; w < 4; ++w)
    for (int s = 0; s < 8; ++s)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
          const float x = float(sm[size_t(16 * s + 8 * (l >> 5) + e) * d + 32 * w + (l & 31)] * 1024.0);
          const uint16_t hi = f16_bits(x);
          sf[(((size_t(w) * 8 + s) * 2 + 0) * 64 + l) * 8 + e] = hi;
          sf[(((size_t(w) * 8 + s) * 2 + 1) * 64 + l) * 8 + e] = f16_bits(x - f16_value(hi));
        }
  int rc = upload_u16(&h->d_pi_frag, pf);
  if (rc != TQ_OK) return rc;
  if ((rc = upload_u16(&h->d_g_frag, gf)) != TQ_OK) return rc;
  if ((rc = upload_u16(&h->d_ds_frag, sf)) != TQ_OK) return rc;
  return upload_u16(&h->d_dq_frag, df);
}

int upload(float** dst, const std::vector<float>& src) {
  if (hipMalloc(reinterpret_cast<void**>(dst), src.size() * sizeof(float)) != hipSuccess) {
    *dst = nullptr;
    return TQ_ENOMEM;
  }
  if (hipMemcpy(*dst, src.data(), src.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess)
    return TQ_EHIP;
  return TQ_OK;
}

std::vector<float> transpose(const std::vector<float>& a, int d) {
  std::vector<float> t(a.size());
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) t[size_t(j) * d + i] = a[size_t(i) * d + j];
  return t;
}

// alpha_S = 2^-B sum_idx c[idx] prod_{p in S} s_p(idx), for odd |S| <= 3
void plane_expansion(const std::vector<float>& c, int code_bits, tqdev::PlaneExpansion* out) {
  const int levels = 1 << code_bits;
  out->count = 0;
  for (uint32_t mask = 1; mask < uint32_t(levels); ++mask) {
    const int size = __builtin_popcount(mask);
    if (size != 1 && size != 3) continue;
    double acc = 0.0;
    for (int idx = 0; idx < levels; ++idx) {
      double s = 1.0;
      for (int p = 0; p < code_bits; ++p)
        if (mask & (1u << p)) s *= ((idx >> p) & 1) ? 1.0 : -1.0;
      acc += double(c[idx]) * s;
    }
    out->mask[out->count] = mask;
    out->alpha[out->count] = float(acc / levels);
    ++out->count;
  }
}

// Scale sigma for the two-pass reconstruction table (tqdev::DequantTable):
// with magnitudes m1 > m0 > 0, sigma = S / m1 for the integer S in
// [1024, 2048) whose sigma m0 lies closest, relatively, to a float16 number
// (sigma m1 = S is one exactly); a single magnitude takes sigma = 1024 / m1.
// More than two magnitudes, or no S within 2^-19: three-pass form.
void dequant_table(const std::vector<float>& c, tqdev::DequantTable* out) {
  out->two_pass = 0;
  std::vector<double> mags;
  for (float x : c) {
    const double m = std::fabs(double(x));
    if (m > 0.0 && std::find(mags.begin(), mags.end(), m) == mags.end()) mags.push_back(m);
  }
  if (mags.empty() || mags.size() > 2) return;
  std::sort(mags.begin(), mags.end());
  const double m1 = mags.back();
  double sigma = 1024.0 / m1, best = 0.0;
  if (mags.size() == 2) {
    best = 1.0;
    for (int s = 1024; s < 2048; ++s) {
      const double v = double(s) / m1 * mags[0];
      const double err = std::fabs(double(f16_value(f16_bits(float(v)))) - v) / v;
      if (err < best) {
        best = err;
        sigma = double(s) / m1;
      }
    }
  }
  if (best > std::ldexp(1.0, -19)) return;
  for (size_t i = 0; i < c.size() && i < size_t(tqdev::kMaxLevels); ++i)
    out->v[i] = f16_value(f16_bits(float(sigma * double(c[i]))));
  out->out_scale = float(1.0 / (sigma * 4096.0));
  out->two_pass = 1;
}

int finish_init(tq_ctx* h) {
  const int d = h->d;
  h->code_bits = h->bits - 1;
  h->levels = 1 << h->code_bits;
  h->words = (d + 31) / 32;
  if (hipGetDevice(&h->device) != hipSuccess) return TQ_EHIP;
  if (hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess ||
      h->cus <= 0)
    return TQ_EHIP;
  if (hipDeviceGetAttribute(&h->lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, h->device) != hipSuccess)
    return TQ_EHIP;
  for (int i = 0; i < tqdev::kMaxLevels; ++i) {
    h->cb.c[i] = i < h->levels ? h->centroids[i] : 0.0f;
    h->cb.t[i] = i + 1 < h->levels ? h->thresholds[i] : INFINITY;
  }
  h->cb.levels = h->levels;
  if (h->hi > 0) {
    const int lh = 2 * h->levels;
    for (int i = 0; i < tqdev::kMaxLevels; ++i) {
      h->cbh.c[i] = i < lh ? h->centroids_hi[i] : 0.0f;
      h->cbh.t[i] = i + 1 < lh ? h->thresholds_hi[i] : INFINITY;
    }
    h->cbh.levels = lh;
    h->hi_words = (h->hi + 31) / 32;
  }
  plane_expansion(h->centroids, h->code_bits, &h->planes);
  dequant_table(h->centroids, &h->dqt);
  {
    // G with float16-exact entries (every seeded handle) takes one matrix-core
    // piece in the projection instead of two
    bool f16 = true;
    for (const float x : h->g) f16 = f16 && float(static_cast<_Float16>(x)) == x;
    h->g_f16 = f16;
  }
  {
    const int L = h->levels, M = L / 2;
    bool sym = h->thresholds[M - 1] == 0.0f;
    for (int i = 0; i < L; ++i) sym = sym && h->centroids[L - 1 - i] == -h->centroids[i];
    for (int i = 0; i + 1 < L; ++i) sym = sym && h->thresholds[L - 2 - i] == -h->thresholds[i];
    h->symmetric = sym;
    for (int j = 0; j < M; ++j) h->half.m[j] = h->centroids[M + j] * 4096.0f;
    for (int k = 0; k + 1 < M; ++k) h->half.u[k] = h->thresholds[M + k] * 4096.0f;
  }
  if (h->hi > 0) {
    // the finer level set of the first hi coordinates, the same way
    const int L = 2 * h->levels, M = L / 2;
    bool sym = h->thresholds_hi[M - 1] == 0.0f;
    for (int i = 0; i < L; ++i) sym = sym && h->centroids_hi[L - 1 - i] == -h->centroids_hi[i];
    for (int i = 0; i + 1 < L; ++i) sym = sym && h->thresholds_hi[L - 2 - i] == -h->thresholds_hi[i];
    h->symmetric_hi = sym;
    plane_expansion(h->centroids_hi, h->code_bits + 1, &h->planes_hi);
    for (int j = 0; j < M; ++j) h->half_hi.m[j] = h->centroids_hi[M + j] * 4096.0f;
    for (int k = 0; k + 1 < M; ++k) h->half_hi.u[k] = h->thresholds_hi[M + k] * 4096.0f;
  }
  int rc;
  if ((rc = upload(&h->d_pi, h->pi)) != TQ_OK) return rc;
  if ((rc = upload(&h->d_piT, transpose(h->pi, d))) != TQ_OK) return rc;
  if ((rc = upload(&h->d_g, h->g)) != TQ_OK) return rc;
  if ((rc = upload(&h->d_gT, transpose(h->g, d))) != TQ_OK) return rc;
  if (d <= 128) {
    // For the lookup-table scorer: Pi^T and S^T with S = G Pi (float64
    // products, one rounding; w = S q = G (Pi q) in one matrix-vector
    // product), both zero-padded to 128 x 128 row-major
    std::vector<float> pt(size_t(128) * 128, 0.0f), st(size_t(128) * 128, 0.0f);
    for (int j = 0; j < d; ++j)
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += double(h->g[size_t(j) * d + k]) * double(h->pi[size_t(k) * d + i]);
        st[size_t(i) * 128 + j] = float(acc);
        pt[size_t(i) * 128 + j] = h->pi[size_t(j) * d + i];
      }
    if ((rc = upload(&h->d_piT128, pt)) != TQ_OK) return rc;
    if ((rc = upload(&h->d_sT128, st)) != TQ_OK) return rc;
  }
  if ((rc = tqdev::build_quantize_gemm_tiles(h)) != TQ_OK) return rc;
  return build_fragments(h);
}

int check_device(const tq_ctx* h) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_EHIP;
  return dev == h->device ? TQ_OK : TQ_EINVAL;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// The matrix-core reconstruction reads a key's code row with 16-byte loads
// (8-byte loads for fractional widths); other addresses take the general
// kernel.
bool dequant_rows_aligned(const tq_ctx* h, const void* codes) {
  return (reinterpret_cast<uintptr_t>(codes) & (h->hi ? 7u : 15u)) == 0;
}

}  // namespace

namespace {

// Which scorer serves nq queries per group: the matrix-core kernel for many
// queries (register form for d <= 256, tiled form above), the lookup-table
// kernel for a few (d in (96, 128]),
// else the general kernel (also for TQ_KERNELS=ref).
enum class Scorer { kGeneral, kLut, kMfma, kPolar };

Scorer pick_scorer(const tq_ctx* h, int64_t nq);

}  // namespace

bool tqdev::force_reference_kernels() {
  const char* v = std::getenv("TQ_KERNELS");
  return v && std::strcmp(v, "ref") == 0;
}

bool tqdev::force_tiled_quantizer() {
  const char* v = std::getenv("TQ_QUANTIZER");
  return v && std::strcmp(v, "tiled") == 0;
}

namespace {

Scorer pick_scorer(const tq_ctx* h, int64_t nq) {
  if (h->polar) return Scorer::kPolar;
  if (tqdev::force_reference_kernels()) return Scorer::kGeneral;
  if (nq >= tqdev::kScoreMfmaMinQueries && tqdev::score_mfma_supported(h)) return Scorer::kMfma;
  if (tqdev::logits_lut128_supported(h)) return Scorer::kLut;
  return Scorer::kGeneral;
}

}  // namespace

extern "C" {

const char* tq_strerror(int code) {
  switch (code) {
    case TQ_OK: return "success";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_EHIP: return "HIP runtime error";
    case TQ_ENOMEM: return "out of memory";
    case TQ_ESCRATCH: return "request needs more than the library's static scratch buffer";
    default: return "unknown error";
  }
}

int tq_host_params(int32_t d, int32_t bits, uint64_t seed, float* pi, float* g, float* centroids,
                   float* thresholds) {
  if (d < 2 || d > 4096 || bits < 2 || bits > 5) return TQ_EINVAL;
  try {
    const int rc = tqhost::build_params(d, bits, seed, pi, g, centroids, thresholds);
    return rc == 0 ? TQ_OK : TQ_EUNSUPPORTED;
  } catch (const std::bad_alloc&) {
    return TQ_ENOMEM;
  } catch (...) {
    return TQ_EUNSUPPORTED;
  }
}

// rotation: kRotHaar (from the seed), kRotExplicit (pi_in, g_in given),
// kRotHadamard (randomized Hadamard from the seed, G from the seed)
enum { kRotHaar = 0, kRotExplicit = 1, kRotHadamard = 2 };

static int init_common(int32_t d, int32_t bits, const float* pi_in, const float* g_in, uint64_t seed,
                       tq_handle* out, int rotation = kRotHaar, int32_t hi = 0, bool polar = false) {
  if (!out) return TQ_EINVAL;
  *out = nullptr;
  if (d < 2 || d > 4096 || bits < 2 || bits > 5) return TQ_EINVAL;
  if (hi < 0 || hi > d || (hi > 0 && bits > 4)) return TQ_EINVAL;
  tq_ctx* h = nullptr;
  try {
    h = new tq_ctx();
    h->d = d;
    h->bits = bits;
    const size_t dd = size_t(d) * d;
    const int levels = 1 << (bits - 1);
    h->pi.resize(dd);
    h->g.resize(dd);
    h->centroids.resize(levels);
    h->thresholds.resize(levels - 1 > 0 ? levels - 1 : 1);
    int rc;
    if (rotation == kRotExplicit) {
      std::memcpy(h->pi.data(), pi_in, dd * sizeof(float));
      std::memcpy(h->g.data(), g_in, dd * sizeof(float));
      rc = tqhost::build_params(d, bits, 0, nullptr, nullptr, h->centroids.data(), h->thresholds.data());
    } else if (rotation == kRotHadamard) {
      rc = tqhost::hadamard_rotation(d, seed, h->pi.data());
      h->hadamard = 1;
      if (rc == 0)
        rc = tqhost::build_params(d, bits, seed, nullptr, h->g.data(), h->centroids.data(), h->thresholds.data());
    } else {
      rc = tqhost::build_params(d, bits, seed, h->pi.data(), h->g.data(), h->centroids.data(),
                                h->thresholds.data());
    }
    if (rc == 0 && hi > 0) {
      // the finer level set: the codebook of one more bit for the same d
      h->hi = hi;
      h->centroids_hi.resize(size_t(2) * levels);
      h->thresholds_hi.resize(size_t(2) * levels - 1);
      rc = tqhost::build_params(d, bits + 1, seed, nullptr, nullptr, h->centroids_hi.data(),
                                h->thresholds_hi.data());
    }
    if (rc == 0 && polar) {
      // per-level angle codebooks; thresholds padded with +inf, cos and sin
      // of each level in float64 rounded once
      int nl = 0;
      while ((1 << nl) < d) ++nl;
      h->polar = 1;
      h->polar_levels = nl;
      h->polar_tab.assign(size_t(nl) * tqdev::kPolarTab, 0.0f);
      const int L = 1 << (bits - 1);
      std::vector<float> lv(L), th(L);
      for (int l = 1; l <= nl && rc == 0; ++l) {
        rc = tqhost::polar_level_codebook(d, bits, l, lv.data(), th.data());
        float* tab = &h->polar_tab[size_t(l - 1) * tqdev::kPolarTab];
        for (int i = 0; i < 16; ++i) {
          tab[i] = i + 1 < L ? th[i] : INFINITY;
          tab[16 + i] = i < L ? float(std::cos(double(lv[i]))) : 1.0f;
          tab[32 + i] = i < L ? float(std::sin(double(lv[i]))) : 0.0f;
        }
      }
    }
    if (rc != 0) {
      delete h;
      return TQ_EUNSUPPORTED;
    }
  } catch (const std::bad_alloc&) {
    delete h;
    return TQ_ENOMEM;
  } catch (...) {
    delete h;
    return TQ_EUNSUPPORTED;
  }
  int rc = finish_init(h);
  if (rc == TQ_OK && h->hadamard) {
    // row 0 of H is all +1: Pi[0][j] = sigma_j c
    std::vector<float> sig(d);
    h->hscale = std::fabs(h->pi[0]);
    for (int j = 0; j < d; ++j) sig[j] = h->pi[j] < 0.0f ? -1.0f : 1.0f;
    if (hipMalloc(reinterpret_cast<void**>(&h->d_hsigma), sizeof(float) * d) != hipSuccess) {
      h->d_hsigma = nullptr;
      rc = TQ_ENOMEM;
    } else if (hipMemcpy(h->d_hsigma, sig.data(), sizeof(float) * d, hipMemcpyHostToDevice) != hipSuccess) {
      rc = TQ_EHIP;
    }
  }
  if (rc == TQ_OK && h->polar) {
    const size_t bytes = h->polar_tab.size() * sizeof(float);
    if (hipMalloc(reinterpret_cast<void**>(&h->d_polar_tab), bytes) != hipSuccess) {
      h->d_polar_tab = nullptr;
      rc = TQ_ENOMEM;
    } else if (hipMemcpy(h->d_polar_tab, h->polar_tab.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
      rc = TQ_EHIP;
    }
  }
  if (rc != TQ_OK) {
    free_device(h);
    delete h;
    return rc;
  }
  // the static scratch of the allocation-free entry points: its address on
  // this device, looked up once (a failure here is reported by those entry
  // points, not by init)
  (void)tqdev::noalloc_prepare(h->device);
  if (trace_enabled())
    std::fprintf(stderr, "[tq] init d=%d bits=%d device=%d\n", h->d, h->bits, h->device);
  *out = h;
  return TQ_OK;
}

int tq_init(int32_t d, int32_t bits, uint64_t seed, tq_handle* out) {
  return init_common(d, bits, nullptr, nullptr, seed, out);
}

int tq_init_split(int32_t d, int32_t bits, int32_t hi, uint64_t seed, tq_handle* out) {
  return init_common(d, bits, nullptr, nullptr, seed, out, kRotHaar, hi);
}

int tq_init_explicit(int32_t d, int32_t bits, const float* pi, const float* g, tq_handle* out) {
  if (!pi || !g) return TQ_EINVAL;
  return init_common(d, bits, pi, g, 0, out, kRotExplicit);
}

int tq_init_hadamard(int32_t d, int32_t bits, uint64_t seed, tq_handle* out) {
  if (d < 2 || d > 4096 || (d & (d - 1)) != 0) {
    if (out) *out = nullptr;
    return TQ_EINVAL;
  }
  return init_common(d, bits, nullptr, nullptr, seed, out, kRotHadamard);
}

int tq_init_polar(int32_t d, int32_t bits, uint64_t seed, tq_handle* out) {
  if (d < 2 || d > 4096 || (d & (d - 1)) != 0) {
    if (out) *out = nullptr;
    return TQ_EINVAL;
  }
  return init_common(d, bits, nullptr, nullptr, seed, out, kRotHaar, 0, true);
}

int tq_polar_codebook(int32_t d, int32_t bits, int32_t level, float* levels, float* thresholds) {
  try {
    const int rc = tqhost::polar_level_codebook(d, bits, level, levels, thresholds);
    return rc == 0 ? TQ_OK : rc == -1 ? TQ_EINVAL : TQ_EUNSUPPORTED;
  } catch (...) {
    return TQ_ENOMEM;
  }
}

int tq_hadamard_rotation(int32_t d, uint64_t seed, float* pi) {
  if (!pi || d < 2 || d > 4096 || (d & (d - 1)) != 0) return TQ_EINVAL;
  return tqhost::hadamard_rotation(d, seed, pi) == 0 ? TQ_OK : TQ_EINVAL;
}

int tq_destroy(tq_handle h) {
  if (!h) return TQ_OK;
  free_device(h);
  delete h;
  return TQ_OK;
}

int tq_get_layout(tq_handle h, tq_layout* out) {
  if (!h || !out) return TQ_EINVAL;
  out->d = h->d;
  out->bits = h->bits;
  out->code_bits = h->code_bits;
  out->levels = h->levels;
  out->words = h->words;
  out->format_version = TQ_FORMAT_VERSION;
  out->code_bytes = int64_t(4) * (int64_t(h->code_bits) * h->words + h->hi_words);
  out->sign_bytes = int64_t(4) * h->words;
  out->key_bytes = out->code_bytes + out->sign_bytes + 8;
  out->hi = h->hi;
  out->hi_words = h->hi_words;
  out->polar = h->polar;
  return TQ_OK;
}

uint64_t tq_params_hash(tq_handle h) {
  if (!h) return 0;
  uint64_t x = 0xcbf29ce484222325ull;
  auto eat = [&x](const std::vector<float>& v) {
    const unsigned char* p = reinterpret_cast<const unsigned char*>(v.data());
    for (size_t i = 0; i < v.size() * sizeof(float); ++i) {
      x ^= p[i];
      x *= 0x100000001b3ull;
    }
  };
  eat(h->pi);
  eat(h->g);
  eat(h->centroids);
  eat(h->centroids_hi);
  for (int i = 0; i < 4; ++i) {
    x ^= uint64_t(h->hi >> (8 * i)) & 0xFFu;
    x *= 0x100000001b3ull;
  }
  eat(h->polar_tab);
  return x;
}

int tq_quantize(tq_handle h, const void* keys, int32_t key_dtype, int64_t n, int64_t ldk, uint32_t* codes,
                uint32_t* signs, float* norms, float* rnorms, void* stream) {
  if (!h || n < 0) return TQ_EINVAL;
  if (key_dtype != TQ_F32 && key_dtype != TQ_BF16) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  if (!keys || !codes || !signs || !norms || !rnorms || ldk < h->d) return TQ_EINVAL;
  if (!aligned4(codes) || !aligned4(signs) || !aligned4(norms) || !aligned4(rnorms)) return TQ_EINVAL;
  if (check_device(h) != TQ_OK) return TQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // d = 128 with bf16 keys: the register-resident matrix-core kernel; other
  // d >= 16: the tiled matrix-core kernels; smaller d: float32 kernels
  hipError_t e;
  if (h->polar)
    e = tqdev::quantize_polar128_supported(h, keys, key_dtype, ldk)
            ? tqdev::launch_quantize_polar128(h, keys, key_dtype, n, ldk, codes, signs, norms, rnorms, s)
            : tqdev::launch_quantize_polar(h, keys, key_dtype, n, ldk, codes, signs, norms, rnorms, s);
  else if (tqdev::force_reference_kernels())
    e = tqdev::launch_quantize_v1(h, keys, key_dtype, n, ldk, codes, signs, norms, rnorms, s);
  else if (tqdev::quantize_mfma128_supported(h, keys, key_dtype, ldk, codes, signs, norms, rnorms))
    e = tqdev::launch_quantize_mfma128(h, keys, n, ldk, codes, signs, norms, rnorms, s);
  else if (tqdev::quantize_fused_supported(h, keys, key_dtype, ldk) && !tqdev::force_tiled_quantizer())
    e = tqdev::launch_quantize_fused(h, keys, key_dtype, n, ldk, codes, signs, norms, rnorms, s);
  else if (tqdev::quantize_gemm_supported(h))
    e = tqdev::launch_quantize_gemm(h, keys, key_dtype, n, ldk, codes, signs, norms, rnorms, s);
  else
    e = tqdev::launch_quantize_v1(h, keys, key_dtype, n, ldk, codes, signs, norms, rnorms, s);
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

size_t tq_logits_workspace_size(tq_handle h, int64_t groups, int64_t nq) {
  if (!h || groups < 0 || nq < 0) return 0;
  return tqdev::score_prep_bytes(h->d, groups, nq);
}

}  // extern "C"

namespace tqdev {

// scores [groups][nq][n] by the scorer pick_scorer chooses; workspace of
// tq_logits_workspace_size bytes (arguments already checked)
int run_logits(const tq_ctx* h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
               const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores,
               void* workspace, hipStream_t s) {
  hipError_t e;
  const Scorer sc = pick_scorer(h, nq);
  if (sc == Scorer::kLut) {
    // query transform fused into the scoring kernel; workspace unused
    e = tqdev::launch_logits_lut128(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, s);
  } else {
    float* vw = static_cast<float*>(workspace);
    e = tqdev::launch_query_prep(h, queries, groups * nq, vw, s);
    if (e != hipSuccess) return TQ_EHIP;
    e = sc == Scorer::kMfma    ? tqdev::launch_score_mfma(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, s)
        : sc == Scorer::kPolar
            ? (tqdev::logits_polar128_supported(h)
                   ? tqdev::launch_logits_polar128(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, s)
                   : tqdev::launch_logits_polar(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, s))
                               : tqdev::launch_logits_v1(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, s);
  }
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

// the checks tq_logits makes on everything but the workspace
int check_logits_args(const tq_ctx* h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
                      const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores) {
  if (!h || groups < 0 || nq < 0 || n < 0) return TQ_EINVAL;
  if (groups == 0 || nq == 0 || n == 0) return TQ_OK;
  if (!queries || !codes || !signs || !norms || !rnorms || !scores) return TQ_EINVAL;
  if (groups > 65535) return TQ_EUNSUPPORTED;
  if (check_device(h) != TQ_OK) return TQ_EINVAL;
  return TQ_OK;
}

}  // namespace tqdev

namespace {

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// workspace of tq_attention: scores, the query transform, the value pass's
// partial sums
struct AttnWorkspace {
  size_t scores, prep, partials, total;
};

AttnWorkspace attn_workspace(const tq_ctx* hk, const tq_ctx* hv, int64_t groups, int64_t nq, int64_t n) {
  AttnWorkspace w{};
  w.scores = tqdev::ws_align(size_t(groups) * size_t(nq) * size_t(n) * sizeof(float));
  w.prep = tqdev::ws_align(tqdev::score_prep_bytes(hk->d, groups, nq));
  w.partials = tqdev::attn_partial_bytes(hv, groups, nq, n);
  w.total = w.scores + w.prep + w.partials;
  return w;
}

}  // namespace

extern "C" {

int tq_logits(tq_handle h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
              const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores,
              void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = tqdev::check_logits_args(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores);
  if (rc != TQ_OK || groups == 0 || nq == 0 || n == 0) return rc;
  if (!workspace || workspace_bytes < tq_logits_workspace_size(h, groups, nq)) return TQ_EINVAL;
  if (!aligned256(workspace)) return TQ_EINVAL;
  return tqdev::run_logits(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, workspace,
                           static_cast<hipStream_t>(stream));
}

int tq_dequant_prod(tq_handle h, const uint32_t* codes, const uint32_t* signs, const float* norms,
                    const float* rnorms, int64_t n, float* ktilde, void* stream) {
  if (!h || n < 0) return TQ_EINVAL;
  if (h->polar) return TQ_EUNSUPPORTED;
  if (n == 0) return TQ_OK;
  if (!codes || !signs || !norms || !rnorms || !ktilde) return TQ_EINVAL;
  if (n > int64_t(0x7FFFFFFF) * 4) return TQ_EUNSUPPORTED;
  if (check_device(h) != TQ_OK) return TQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = (!tqdev::force_reference_kernels() && tqdev::dequant_mfma128_supported(h) && h->d_ds_frag &&
                        dequant_rows_aligned(h, codes) && (reinterpret_cast<uintptr_t>(signs) & 15u) == 0)
                           ? tqdev::launch_dequant_prod_mfma128(h, codes, signs, norms, rnorms, n, ktilde, s)
                           : tqdev::launch_dequant_prod_v1(h, codes, signs, norms, rnorms, n, ktilde, s);
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

int tq_dense_logits(const float* queries, int64_t groups, int64_t nq, const void* keys, int32_t key_dtype,
                    int64_t n, int32_t d, int64_t ldk, float* scores, void* stream) {
  if (groups < 0 || nq < 0 || n < 0 || d < 1 || d > 4096 || ldk < d) return TQ_EINVAL;
  if (key_dtype != TQ_F32 && key_dtype != TQ_BF16) return TQ_EINVAL;
  if (groups == 0 || nq == 0 || n == 0) return TQ_OK;
  if (!queries || !keys || !scores || !aligned4(queries) || !aligned4(scores)) return TQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(keys) & (key_dtype == TQ_BF16 ? 1u : 3u)) != 0) return TQ_EINVAL;
  if (groups > 65535 || (n + 3) / 4 > 0x7FFFFFFF) return TQ_EUNSUPPORTED;
  const hipError_t e = tqdev::launch_dense_logits(queries, groups, nq, keys, key_dtype, n, d, ldk, scores,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

int tq_pack_values(tq_handle h, const uint32_t* codes, int64_t groups, int64_t n, uint32_t* vcodes, void* stream) {
  if (!h || groups < 0 || n < 0) return TQ_EINVAL;
  if (h->hi != 0 || h->polar) return TQ_EUNSUPPORTED;  // stored values use one width of scalar codes
  if (groups == 0 || n == 0) return TQ_OK;
  if (!codes || !vcodes || !aligned4(codes) || (reinterpret_cast<uintptr_t>(vcodes) & 15u) != 0) return TQ_EINVAL;
  if (groups > 65535 || (n + 31) / 32 > 0x7FFFFFFF) return TQ_EUNSUPPORTED;
  if (check_device(h) != TQ_OK) return TQ_EINVAL;
  const hipError_t e = tqdev::launch_pack_values(h, codes, groups, n, vcodes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

size_t tq_attention_workspace_size(tq_handle hk, tq_handle hv, int64_t groups, int64_t nq, int64_t n) {
  if (!hk || !hv || groups < 0 || nq < 0 || n < 0) return 0;
  return attn_workspace(hk, hv, groups, nq, n).total;
}

int tq_attention(tq_handle hk, tq_handle hv, const float* queries, int64_t groups, int64_t nq,
                 const uint32_t* kcodes, const uint32_t* ksigns, const float* knorms, const float* krnorms,
                 const uint32_t* vcodes, const float* vnorms, int64_t n, float scale, float* out, float* lse,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!hk || !hv || groups < 0 || nq < 0 || n < 0) return TQ_EINVAL;
  if (hk->d != hv->d || hk->device != hv->device || !std::isfinite(scale)) return TQ_EINVAL;
  if (hv->hi != 0 || hv->polar || hk->polar) return TQ_EUNSUPPORTED;  // scalar codes, one width
  if (groups == 0 || nq == 0) return TQ_OK;
  if (!out || !aligned4(out) || (lse && !aligned4(lse))) return TQ_EINVAL;
  if (groups * ((nq + 15) / 16) > 65535) return TQ_EUNSUPPORTED;
  if (check_device(hk) != TQ_OK) return TQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n == 0) {  // no tokens: o = 0, lse = -inf
    hipError_t e = tqdev::launch_fill_u32(reinterpret_cast<unsigned int*>(out), groups * nq * hk->d, 0u, s);
    if (e == hipSuccess && lse) e = tqdev::launch_fill_u32(reinterpret_cast<unsigned int*>(lse), groups * nq, 0xFF800000u, s);
    return e == hipSuccess ? TQ_OK : TQ_EHIP;
  }
  if (!queries || !kcodes || !ksigns || !knorms || !krnorms || !vcodes || !vnorms || !workspace) return TQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(vcodes) & 15u) != 0 || !aligned4(vnorms) || !aligned256(workspace))
    return TQ_EINVAL;
  const AttnWorkspace w = attn_workspace(hk, hv, groups, nq, n);
  if (workspace_bytes < w.total) return TQ_EINVAL;
  char* base = static_cast<char*>(workspace);
  if (tqdev::attention_fused_supported(hk, hv) &&
      tqdev::attn_fused_partial_bytes(hk, groups, nq, n) <= w.partials) {
    // scores stay on chip; the partials take the two-kernel form's place
    const hipError_t e = tqdev::launch_attention_fused(hk, hv, queries, groups, nq, kcodes, ksigns, knorms, krnorms, n,
                                                       vcodes, vnorms, scale, base + w.scores + w.prep, out, lse, s);
    return e == hipSuccess ? TQ_OK : TQ_EHIP;
  }
  float* scores = reinterpret_cast<float*>(base);
  const int rc = tqdev::run_logits(hk, queries, groups, nq, kcodes, ksigns, knorms, krnorms, n, scores, base + w.scores, s);
  if (rc != TQ_OK) return rc;
  const hipError_t e = tqdev::launch_attention_values(hv, scores, groups, nq, n, vcodes, vnorms, scale,
                                                      base + w.scores + w.prep, out, lse, s);
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // extern "C"

namespace {

// Search entry point, two forms:
//  * fused: the matrix-core scorer keeps each query's k best keys per block
//    (no score matrix is written), then one merge pass combines the blocks'
//    lists.  Used whenever the matrix-core scorer is (many queries, any d)
//    and the lists fit in LDS.  The blocks that walk one query's keys share
//    the best k-th score any of them has found (a lower bound of the k-th
//    best overall), so that far fewer keys enter a list only to be pushed
//    out again.
//  * chunked: score a chunk of keys for all queries into the workspace, merge
//    it into running lists, repeat.
// TQ_TOPK_CHUNK=<keys> forces the chunked form with that chunk size (tests
// use it to cover many chunks).
bool topk_fused(const tq_ctx* h, int64_t groups, int64_t nq, int64_t n, int32_t k) {
  if (std::getenv("TQ_TOPK_CHUNK")) return false;
  return n > 0 && groups <= 65535 && pick_scorer(h, nq) == Scorer::kMfma && tqdev::score_topk_mfma_supported(h, n, k);
}

// Keys scored per chunk by the chunked form: scores of one chunk for all nq
// queries stay within 64 Mi floats (about the size of the MALL); the general
// scorer, which spreads only over keys, gets at least 65536 keys per chunk
// to fill the GPU.
int64_t topk_chunk(const tq_ctx* h, int64_t nq, int64_t n) {
  int64_t c = (int64_t(64) << 20) / (nq > 0 ? nq : 1);
  if (pick_scorer(h, nq) == Scorer::kGeneral && c < 65536) c = 65536;
  if (const char* v = std::getenv("TQ_TOPK_CHUNK")) c = std::atoll(v);
  c = c / 64 * 64;
  if (c < 64) c = 64;
  return c < n ? c : n;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// chunked: chunk [nq][c] scores, running lists [nq][k], vw of one group;
// fused: block lists [groups][nq][splits][k] (part_s, part_i), vw of all
// groups, shared bounds [groups][nq] (bound)
struct TopkWorkspace {
  bool fused;
  int64_t splits;
  size_t chunk, list_s, list_i, vw, bound, total;
};

TopkWorkspace topk_layout(const tq_ctx* h, int64_t groups, int64_t nq, int64_t n, int32_t k) {
  TopkWorkspace w{};
  w.fused = topk_fused(h, groups, nq, n, k);
  if (w.fused) {
    w.splits = tqdev::score_topk_mfma_splits(h, groups, nq, n);
    const size_t entries = size_t(groups) * size_t(nq) * size_t(w.splits) * size_t(k);
    w.chunk = 0;
    w.list_s = 0;
    w.list_i = align256(entries * sizeof(float));
    w.vw = w.list_i + align256(entries * sizeof(int64_t));
    w.bound = w.vw + tqdev::score_prep_bytes(h->d, groups, nq);
    w.total = w.bound + align256(size_t(groups) * size_t(nq) * sizeof(unsigned int));
    return w;
  }
  const int64_t c = topk_chunk(h, nq, n);
  w.chunk = 0;
  w.list_s = align256(size_t(nq) * size_t(c) * sizeof(float));
  w.list_i = w.list_s + align256(size_t(nq) * size_t(k) * sizeof(float));
  w.vw = w.list_i + align256(size_t(nq) * size_t(k) * sizeof(int64_t));
  w.total = w.vw + tqdev::score_prep_bytes(h->d, 1, nq);
  return w;
}

}  // namespace

extern "C" {

size_t tq_logits_topk_workspace_size(tq_handle h, int64_t groups, int64_t nq, int64_t n, int32_t k) {
  if (!h || groups < 0 || nq < 0 || n < 0 || k < 1 || k > tqdev::kTopkMax) return 0;
  return topk_layout(h, groups, nq, n, k).total;
}

int tq_logits_topk(tq_handle h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
                   const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, int32_t k,
                   int64_t* top_idx, float* top_scores, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h || groups < 0 || nq < 0 || n < 0) return TQ_EINVAL;
  if (h->polar) return TQ_EUNSUPPORTED;
  if (k < 1 || k > tqdev::kTopkMax) return TQ_EINVAL;
  if (groups == 0 || nq == 0) return TQ_OK;
  if (!queries || !top_idx || !top_scores || !workspace) return TQ_EINVAL;
  if (n > 0 && (!codes || !signs || !norms || !rnorms)) return TQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TQ_EINVAL;
  const TopkWorkspace lay = topk_layout(h, groups, nq, n, k);
  if (workspace_bytes < lay.total) return TQ_EINVAL;
  if (check_device(h) != TQ_OK) return TQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* list_s = reinterpret_cast<float*>(ws + lay.list_s);
  int64_t* list_i = reinterpret_cast<int64_t*>(ws + lay.list_i);
  float* vw = reinterpret_cast<float*>(ws + lay.vw);
  hipError_t e = hipSuccess;
  if (lay.fused) {
    // every group at once: query transform, bounds to -inf, per-block lists,
    // one merge
    unsigned int* bound = reinterpret_cast<unsigned int*>(ws + lay.bound);
    if ((e = tqdev::launch_query_prep(h, queries, groups * nq, vw, s)) != hipSuccess) return TQ_EHIP;
    if ((e = tqdev::launch_fill_u32(bound, groups * nq, tqdev::kBoundEmpty, s)) != hipSuccess) return TQ_EHIP;
    e = tqdev::launch_score_topk_mfma(h, vw, groups, nq, codes, signs, norms, rnorms, n, n, k, bound, list_s, list_i,
                                      s);
    if (e != hipSuccess) return TQ_EHIP;
    e = tqdev::launch_topk_merge(list_s, list_i, groups * nq, lay.splits * k, 0, k, nullptr, nullptr, true,
                                 top_scores, top_idx, s);
    return e == hipSuccess ? TQ_OK : TQ_EHIP;
  }
  float* chunk = reinterpret_cast<float*>(ws + lay.chunk);
  const Scorer sc = pick_scorer(h, nq);
  const int64_t c = topk_chunk(h, nq, n);
  const int64_t cw = int64_t(h->code_bits) * h->words + h->hi_words;  // code words per key
  for (int64_t g = 0; g < groups && e == hipSuccess; ++g) {
    const float* qg = queries + g * nq * h->d;
    float* og = top_scores + g * nq * k;
    int64_t* oi = top_idx + g * nq * k;
    if (n == 0) {  // no keys: every entry is empty
      e = tqdev::launch_topk_merge(chunk, nullptr, nq, 0, 0, k, list_s, list_i, true, og, oi, s);
      continue;
    }
    if (sc != Scorer::kLut && (e = tqdev::launch_query_prep(h, qg, nq, vw, s)) != hipSuccess) break;
    for (int64_t c0 = 0; c0 < n && e == hipSuccess; c0 += c) {
      const int64_t ce = n - c0 < c ? n - c0 : c;
      const int64_t key0 = g * n + c0;
      const uint32_t* cg = codes + key0 * cw;
      const uint32_t* sg = signs + key0 * h->words;
      switch (sc) {
        case Scorer::kLut:
          e = tqdev::launch_logits_lut128(h, qg, 1, nq, cg, sg, norms + key0, rnorms + key0, ce, chunk, s);
          break;
        case Scorer::kMfma:
          e = tqdev::launch_score_mfma(h, vw, 1, nq, cg, sg, norms + key0, rnorms + key0, ce, chunk, s);
          break;
        default:
          e = tqdev::launch_logits_v1(h, vw, 1, nq, cg, sg, norms + key0, rnorms + key0, ce, chunk, s);
      }
      if (e != hipSuccess) break;
      e = tqdev::launch_topk_merge(chunk, nullptr, nq, ce, c0, k, list_s, list_i, c0 + ce >= n, og, oi, s);
    }
  }
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

int tq_dequant_mse(tq_handle h, const uint32_t* codes, const float* norms, int64_t n, float* khat,
                   void* stream) {
  if (!h || n < 0) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  if (!codes || !norms || !khat) return TQ_EINVAL;
  if (check_device(h) != TQ_OK) return TQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = h->polar ? (tqdev::dequant_polar128_supported(h)
                                       ? tqdev::launch_dequant_polar128(h, codes, norms, n, khat, s)
                                       : tqdev::launch_dequant_polar(h, codes, norms, n, khat, s))
                       : (!tqdev::force_reference_kernels() && tqdev::dequant_mfma128_supported(h) &&
                          dequant_rows_aligned(h, codes))
                           ? tqdev::launch_dequant_mfma128(h, codes, norms, n, khat, s)
                           : tqdev::launch_dequant_v1(h, codes, norms, n, khat, s);
  return e == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // extern "C"
