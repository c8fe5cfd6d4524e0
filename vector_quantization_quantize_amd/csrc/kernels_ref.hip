// Straightforward gfx950 kernels for every stage of the path (fp32 VALU,
// any d in [2, 4096], any bits in [2, 5]).  They are the general fallback
// and the baseline the tuned kernels are checked against, and the kernels
// of fractional widths: the first `hi` rotated coordinates take their level
// from a second set `cbh` with one more index bit, stored as one extra
// plane of hi_words = ceil(hi / 32) words after the code_bits full planes
// (per-key code stride code_bits * words + hi_words; hi = 0 for a plain
// handle).
//
// Stages (web pages about TurboQuant, by title and section):
//   quantize  - "TurboQuant tutorial" (gitcode.csdn.net), PolarQuant and QJL
//               sections; "TurboQuant digest" (juejin.cn) section 2.
//   score     - "TurboQuant digest" section 2 and "TurboQuant deep review"
//               (freelamp.com), error-compensation section: high-precision
//               query against 1-bit residual signs, zero-bias estimate.
//   dequant   - "TurboQuant tutorial", polar part: codes and the kept length
//               map back to a vector (stage 1 only).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

constexpr int kThreads = 256;

// idx = #{ i : t_i <= z }  (a tie goes to the upper cell)
__device__ __forceinline__ int bucket(float z, const float* t, int levels) {
  int idx = 0;
  for (int i = 0; i + 1 < levels; ++i) idx += (t[i] <= z) ? 1 : 0;
  return idx;
}

// Register block of a matrix product over an LDS tile: for the 4 rows
// x_r = x + r ds (r < 4) and the output columns j0 .. j0+3 (those below d),
//   a[r][c] = sum_i m[i d + j0 + c] x_r[i],  i ascending, one fma per term.
// Four columns per thread cut the loads per fma from 5/4 to 1/2 (1/4 with
// 16-byte loads when d is a multiple of 4).
// The loop is unrolled by 8 with no branch in its body, so that the matrix
// loads of 8 rows (L2 hits, but hundreds of cycles each) are in flight
// together; columns past d read column d - 1 and are never stored.
template <bool kVec>
__device__ __forceinline__ void product4x4_body(const float* __restrict__ m, int d, const float* x, int ds, int j0,
                                                float (&a)[4][4]) {
  int jc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) jc[c] = j0 + c < d ? j0 + c : d - 1;
#pragma unroll 8
  for (int i = 0; i < d; ++i) {
    const float* row = m + size_t(i) * d;
    float w[4];
    if constexpr (kVec) {
      const float4 v = *reinterpret_cast<const float4*>(row + j0);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = row[jc[c]];
    }
    const float x0 = x[i], x1 = x[ds + i], x2 = x[2 * ds + i], x3 = x[3 * ds + i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[0][c] = fmaf(w[c], x0, a[0][c]);
      a[1][c] = fmaf(w[c], x1, a[1][c]);
      a[2][c] = fmaf(w[c], x2, a[2][c]);
      a[3][c] = fmaf(w[c], x3, a[3][c]);
    }
  }
}

__device__ __forceinline__ void product4x4(const float* __restrict__ m, int d, const float* x, int ds, int j0,
                                           float (&a)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) a[r][c] = 0.0f;
  if ((d & 3) == 0)
    product4x4_body<true>(m, d, x, ds, j0, a);
  else
    product4x4_body<false>(m, d, x, ds, j0, a);
}

// ---------------------------------------------------------------------------
// quantize: one block per tile of `tk` keys, two LDS buffers of tk x (d+1).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
quantize_ref_kernel(const void* __restrict__ keys, int key_dtype, int64_t n, int64_t ldk, int d,
                    int code_bits, int words, int tk, const float* __restrict__ piT,
                    const float* __restrict__ gT, Codebook cb, uint32_t* __restrict__ codes,
                    uint32_t* __restrict__ signs, float* __restrict__ norms,
                    float* __restrict__ rnorms, int hi, int hi_words, Codebook cbh) {
  extern __shared__ float smem[];
  const int ds = d + 1;  // padded row stride
  float* buf0 = smem;
  float* buf1 = smem + size_t(tk) * ds;
  float* nrm = buf1 + size_t(tk) * ds;
  float* lvl = nrm + tk;           // levels
  float* thr = lvl + kMaxLevels;   // thresholds
  float* lvlh = thr + kMaxLevels;  // the finer set (coordinates below hi)
  float* thrh = lvlh + kMaxLevels;
  const int tid = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * tk;
  const int64_t cw = int64_t(code_bits) * words + hi_words;  // code words per key
  if (tid < kMaxLevels) {
    lvl[tid] = cb.c[tid];
    thr[tid] = cb.t[tid];
    lvlh[tid] = cbh.c[tid];
    thrh[tid] = cbh.t[tid];
  }
  // keys -> buf0 (fp32): one loop per key type, loads from clamped rows and
  // no branch in the body, so the unrolled loads are all in flight at once
  auto stage = [&](auto load) {
#pragma unroll 8
    for (int p = tid; p < tk * d; p += kThreads) {
      const int k = p / d, i = p - k * d;
      const int64_t key = base + k;
      const float v = load((key < n ? key : n - 1) * ldk + i);
      buf0[k * ds + i] = key < n ? v : 0.0f;
    }
  };
  if (key_dtype == TQ_BF16)
    stage([&](int64_t off) { return __uint_as_float(uint32_t(static_cast<const uint16_t*>(keys)[off]) << 16); });
  else
    stage([&](int64_t off) { return static_cast<const float*>(keys)[off]; });
  __syncthreads();
  // norms
  for (int k = tid; k < tk; k += kThreads) {
    float s = 0.0f;
    for (int i = 0; i < d; ++i) s = fmaf(buf0[k * ds + i], buf0[k * ds + i], s);
    const float nk = sqrtf(s);
    nrm[k] = nk;
    if (base + k < n) norms[base + k] = nk;
  }
  __syncthreads();
  // z = (Pi k) / n, four keys x four output coordinates per thread
  const int groups = tk / 4, quads = (d + 3) / 4;
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, j0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(piT, d, buf0 + (4 * kg) * ds, ds, j0, a);
    for (int r = 0; r < 4; ++r) {
      const float nk = nrm[4 * kg + r];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < d) buf1[(4 * kg + r) * ds + j0 + c] = nk > 0.0f ? a[r][c] / nk : 0.0f;
    }
  }
  __syncthreads();
  // bucketize, residual in place, code planes
  for (int p = tid; p < tk * words; p += kThreads) {
    const int k = p / words, w = p - k * words;
    uint32_t plane[5] = {0u, 0u, 0u, 0u, 0u};
    for (int b = 0; b < 32; ++b) {
      const int j = 32 * w + b;
      if (j >= d) break;
      const float z = buf1[k * ds + j];
      const bool fine = j < hi;
      const int idx = bucket(z, fine ? thrh : thr, fine ? cbh.levels : cb.levels);
      buf1[k * ds + j] = z - (fine ? lvlh[idx] : lvl[idx]);
      for (int q = 0; q <= code_bits; ++q) plane[q] |= uint32_t((idx >> q) & 1) << b;
    }
    const int64_t key = base + k;
    if (key < n) {
      for (int q = 0; q < code_bits; ++q) codes[key * cw + int64_t(q) * words + w] = plane[q];
      if (w < hi_words) codes[key * cw + int64_t(code_bits) * words + w] = plane[code_bits];
    }
  }
  __syncthreads();
  for (int k = tid; k < tk; k += kThreads) {
    float s = 0.0f;
    for (int i = 0; i < d; ++i) s = fmaf(buf1[k * ds + i], buf1[k * ds + i], s);
    if (base + k < n) rnorms[base + k] = sqrtf(s);
  }
  // p = G r -> buf0
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, j0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(gT, d, buf1 + (4 * kg) * ds, ds, j0, a);
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < d) buf0[(4 * kg + r) * ds + j0 + c] = a[r][c];
  }
  __syncthreads();
  for (int p = tid; p < tk * words; p += kThreads) {
    const int k = p / words, w = p - k * words;
    uint32_t word = 0u;
    for (int b = 0; b < 32; ++b) {
      const int j = 32 * w + b;
      if (j >= d) break;
      word |= uint32_t(buf0[k * ds + j] > 0.0f) << b;
    }
    const int64_t key = base + k;
    if (key < n) signs[key * words + w] = word;
  }
}

// ---------------------------------------------------------------------------
// query prep: v = Pi q, w = G v, one block per query
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
query_prep_kernel(const float* __restrict__ queries, int d, const float* __restrict__ piT,
                  const float* __restrict__ gT, float* __restrict__ vw, int64_t stride, int64_t half) {
  extern __shared__ float smem[];
  float* qs = smem;
  float* vs = smem + d;
  const int64_t qi = blockIdx.x;
  for (int i = threadIdx.x; i < d; i += kThreads) qs[i] = queries[qi * d + i];
  __syncthreads();
  float* out = vw + qi * stride;
  for (int j = threadIdx.x; j < half; j += kThreads) {
    float a = 0.0f;
    if (j < d)
      for (int i = 0; i < d; ++i) a = fmaf(piT[size_t(i) * d + j], qs[i], a);
    if (j < d) vs[j] = a;
    out[j] = a;  // zero padding past d
  }
  __syncthreads();
  for (int j = threadIdx.x; j < half; j += kThreads) {
    float a = 0.0f;
    if (j < d)
      for (int i = 0; i < d; ++i) a = fmaf(gT[size_t(i) * d + j], vs[i], a);
    out[half + j] = a;
  }
}

// ---------------------------------------------------------------------------
// scores: one thread per key, queries of the group in chunks of 4
// ---------------------------------------------------------------------------
// NP = planes per coordinate at most (code_bits, plus one with fractional
// widths): a compile-time bound for the index loops.
template <int NP>
__global__ void __launch_bounds__(kThreads)
logits_ref_kernel(const float* __restrict__ vw, int64_t nq, int d, int code_bits, int words,
                  int64_t n, int64_t stride, int64_t half, const uint32_t* __restrict__ codes,
                  const uint32_t* __restrict__ signs, const float* __restrict__ norms,
                  const float* __restrict__ rnorms, float* __restrict__ scores, Codebook cb, int hi,
                  int hi_words, Codebook cbh) {
  extern __shared__ float smem[];
  float* lvl = smem;
  float* lvlh = smem + kMaxLevels;    // the finer set (coordinates below hi)
  // [d][8]: coordinate j's v for the 4 queries, then its w for them, so
  // that two 16-byte reads (the same address in every lane) serve all 8
  // products of one coordinate
  float* qv = smem + 2 * kMaxLevels;
  const int64_t g = blockIdx.y;
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t key = g * n + t;
  if (threadIdx.x < kMaxLevels) {
    lvl[threadIdx.x] = cb.c[threadIdx.x];
    lvlh[threadIdx.x] = cbh.c[threadIdx.x];
  }
  const int64_t cw = int64_t(code_bits) * words + hi_words;  // code words per key
  const float kappa = 1.2533141373155002512f / float(d);  // sqrt(pi/2) / d
  float nk = 0.f, rho = 0.f;
  if (t < n) {
    nk = norms[key];
    rho = rnorms[key];
  }
  for (int64_t q0 = 0; q0 < nq; q0 += 4) {
    const int qc = int(nq - q0 < 4 ? nq - q0 : 4);
    __syncthreads();
    for (int p = threadIdx.x; p < 4 * d; p += kThreads) {
      const int q = p / d, j = p - q * d;
      const float* src = vw + (g * nq + q0 + (q < qc ? q : 0)) * stride;
      qv[8 * j + q] = q < qc ? src[j] : 0.f;
      qv[8 * j + 4 + q] = q < qc ? src[half + j] : 0.f;
    }
    __syncthreads();
    if (t >= n) continue;
    float a1[4] = {0.f, 0.f, 0.f, 0.f}, a2[4] = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < words; ++w) {
      // planes past the key's own stay 0 and add nothing to the index, so
      // every plane loop below has the fixed trip count NP
      uint32_t plane[NP];
#pragma unroll
      for (int q = 0; q < NP; ++q) plane[q] = 0u;
#pragma unroll
      for (int q = 0; q < NP; ++q)
        if (q < code_bits) plane[q] = codes[key * cw + int64_t(q) * words + w];
#pragma unroll
      for (int q = 1; q < NP; ++q)
        if (q == code_bits && w < hi_words) plane[q] = codes[key * cw + int64_t(q) * words + w];
      const uint32_t sw = signs[key * words + w];
      auto step = [&](int b) {
        const int j = 32 * w + b;
        int idx = 0;
#pragma unroll
        for (int q = 0; q < NP; ++q) idx |= int((plane[q] >> b) & 1u) << q;
        const float cv = j < hi ? lvlh[idx] : lvl[idx];
        const float sg = ((sw >> b) & 1u) ? 1.0f : -1.0f;
        const float4 vv = *reinterpret_cast<const float4*>(qv + 8 * j);
        const float4 ww = *reinterpret_cast<const float4*>(qv + 8 * j + 4);
        a1[0] = fmaf(vv.x, cv, a1[0]);
        a1[1] = fmaf(vv.y, cv, a1[1]);
        a1[2] = fmaf(vv.z, cv, a1[2]);
        a1[3] = fmaf(vv.w, cv, a1[3]);
        a2[0] = fmaf(ww.x, sg, a2[0]);
        a2[1] = fmaf(ww.y, sg, a2[1]);
        a2[2] = fmaf(ww.z, sg, a2[2]);
        a2[3] = fmaf(ww.w, sg, a2[3]);
      };
      if (32 * w + 32 <= d) {
#pragma unroll
        for (int b = 0; b < 32; ++b) step(b);
      } else {
        for (int b = 0; b < d - 32 * w; ++b) step(b);
      }
    }
    const float corr = rho * kappa;
    for (int q = 0; q < qc; ++q)
      scores[(g * nq + q0 + q) * n + t] = nk * fmaf(corr, a2[q], a1[q]);
  }
}

// ---------------------------------------------------------------------------
// dequant: k_hat = n Pi^T c[idx]; block per tile of tk keys
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
dequant_ref_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms, int64_t n, int d,
                   int code_bits, int words, int tk, const float* __restrict__ pi, Codebook cb,
                   float* __restrict__ khat, int hi, int hi_words, Codebook cbh) {
  extern __shared__ float smem[];
  const int ds = d + 1;
  float* ch = smem;                    // [tk][ds] c[idx]
  float* lvl = smem + size_t(tk) * ds;
  float* lvlh = lvl + kMaxLevels;      // the finer set (coordinates below hi)
  const int tid = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * tk;
  const int64_t cw = int64_t(code_bits) * words + hi_words;  // code words per key
  if (tid < kMaxLevels) {
    lvl[tid] = cb.c[tid];
    lvlh[tid] = cbh.c[tid];
  }
  __syncthreads();
  for (int p = tid; p < tk * words; p += kThreads) {
    const int k = p / words, w = p - k * words;
    const int64_t key = base + k;
    uint32_t plane[5] = {0u, 0u, 0u, 0u, 0u};
    if (key < n) {
      for (int q = 0; q < code_bits; ++q) plane[q] = codes[key * cw + int64_t(q) * words + w];
      if (w < hi_words) plane[code_bits] = codes[key * cw + int64_t(code_bits) * words + w];
    }
    for (int b = 0; b < 32; ++b) {
      const int j = 32 * w + b;
      if (j >= d) break;
      int idx = 0;
      for (int q = 0; q <= code_bits; ++q) idx |= int((plane[q] >> b) & 1u) << q;
      ch[k * ds + j] = j < hi ? lvlh[idx] : lvl[idx];
    }
  }
  __syncthreads();
  // (Pi^T c)_j = sum_i Pi[i][j] c_i
  const int groups = tk / 4, quads = (d + 3) / 4;
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, j0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(pi, d, ch + (4 * kg) * ds, ds, j0, a);
    for (int r = 0; r < 4; ++r) {
      const int64_t key = base + 4 * kg + r;
      if (key >= n) continue;
      const float nk = norms[key];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < d) khat[key * d + j0 + c] = nk * a[r][c];
    }
  }
}

// ---------------------------------------------------------------------------
// reconstruction with the correction: k_tilde = n Pi^T (c[idx] + rho kappa
// G^T (2 beta - 1)), kappa = sqrt(pi/2) / d (the vector whose inner product
// with any query is the asymmetric score).  Block per tile of tk keys:
// t = c[idx] and the signs go to LDS; t += rho kappa G^T s; then Pi^T t.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
dequant_prod_ref_kernel(const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
                        const float* __restrict__ norms, const float* __restrict__ rnorms, int64_t n, int d,
                        int code_bits, int words, int tk, const float* __restrict__ pi,
                        const float* __restrict__ g, Codebook cb, float kappa, float* __restrict__ out, int hi,
                        int hi_words, Codebook cbh) {
  extern __shared__ float smem[];
  const int ds = d + 1;
  float* t = smem;                       // [tk][ds] c[idx], then c + rho kappa G^T s
  float* sg = smem + size_t(tk) * ds;    // [tk][ds] 2 beta - 1
  float* lvl = sg + size_t(tk) * ds;
  float* lvlh = lvl + kMaxLevels;        // the finer set (coordinates below hi)
  const int tid = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * tk;
  const int64_t cw = int64_t(code_bits) * words + hi_words;  // code words per key
  if (tid < kMaxLevels) {
    lvl[tid] = cb.c[tid];
    lvlh[tid] = cbh.c[tid];
  }
  __syncthreads();
  for (int p = tid; p < tk * words; p += kThreads) {
    const int k = p / words, w = p - k * words;
    const int64_t key = base + k;
    uint32_t plane[5] = {0u, 0u, 0u, 0u, 0u};
    uint32_t sw = 0u;
    if (key < n) {
      for (int q = 0; q < code_bits; ++q) plane[q] = codes[key * cw + int64_t(q) * words + w];
      if (w < hi_words) plane[code_bits] = codes[key * cw + int64_t(code_bits) * words + w];
      sw = signs[key * words + w];
    }
    for (int b = 0; b < 32; ++b) {
      const int j = 32 * w + b;
      if (j >= d) break;
      int idx = 0;
      for (int q = 0; q <= code_bits; ++q) idx |= int((plane[q] >> b) & 1u) << q;
      t[k * ds + j] = j < hi ? lvlh[idx] : lvl[idx];
      sg[k * ds + j] = (sw >> b) & 1u ? 1.0f : -1.0f;
    }
  }
  __syncthreads();
  const int groups = tk / 4, quads = (d + 3) / 4;
  // (G^T s)_i = sum_j G[j][i] s_j; each (key, i) of t is written by one thread
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, i0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(g, d, sg + (4 * kg) * ds, ds, i0, a);
    for (int r = 0; r < 4; ++r) {
      const int64_t key = base + 4 * kg + r;
      const float rk = (key < n ? rnorms[key] : 0.0f) * kappa;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (i0 + c < d) t[(4 * kg + r) * ds + i0 + c] = fmaf(rk, a[r][c], t[(4 * kg + r) * ds + i0 + c]);
    }
  }
  __syncthreads();
  // (Pi^T t)_j = sum_i Pi[i][j] t_i
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, j0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(pi, d, t + (4 * kg) * ds, ds, j0, a);
    for (int r = 0; r < 4; ++r) {
      const int64_t key = base + 4 * kg + r;
      if (key >= n) continue;
      const float nk = norms[key];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < d) out[key * d + j0 + c] = nk * a[r][c];
    }
  }
}

// keys per tile so that `buffers` LDS arrays of tk x (d+1) floats fit in
// `budget` bytes; a multiple of 4, at least 4
// ---------------------------------------------------------------------------
// Polar stage 1 (tq_init_polar): angles of the recursive polar transform of
// z = Pi u, quantized per level, and z_hat composed back from the levels
// ("TurboQuant tutorial", Cartesian-to-polar section; "TurboQuant deep
// review", breakthrough section).  Level l's d / 2^l angles sit in slots
// d - d / 2^(l-1) .. of a key's slot array; per level, the table holds 16
// thresholds (+inf past L - 1), then cos and sin of the 16 levels.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int polar_off(int d, int l) { return d - (d >> (l - 1)); }

// #{t <= a} over a level's thresholds (+inf padding never counts)
__device__ __forceinline__ int polar_code(float a, const float* t, int levels) {
  int c = 0;
  for (int i = 0; i + 1 < levels; ++i) c += a >= t[i] ? 1 : 0;
  return c;
}

// z_hat_j from the key's slot codes, top level first (radius 1 times the
// cos / sin of the level value on the path down to coordinate j)
__device__ __forceinline__ float polar_zhat(const uint8_t* slot, int d, int nl, int j, const float* tab) {
  float v = 1.0f;
  for (int l = nl; l >= 1; --l) {
    const int code = slot[polar_off(d, l) + (j >> l)];
    v *= ((j >> (l - 1)) & 1) ? tab[(l - 1) * kPolarTab + 32 + code] : tab[(l - 1) * kPolarTab + 16 + code];
  }
  return v;
}

// unpack tk keys' codes (slot order in the bit planes) into slot bytes
__device__ __forceinline__ void polar_unpack(const uint32_t* __restrict__ codes, int64_t base, int64_t n, int d,
                                             int code_bits, int words, int tk, uint8_t* slots) {
  for (int p = threadIdx.x; p < tk * words; p += kThreads) {
    const int k = p / words, w = p - k * words;
    const int64_t key = base + k < n ? base + k : n - 1;
    uint32_t plane[5] = {0u, 0u, 0u, 0u, 0u};
    for (int q = 0; q < code_bits; ++q) plane[q] = codes[key * int64_t(code_bits) * words + int64_t(q) * words + w];
    for (int b = 0; b < 32 && 32 * w + b < d; ++b) {
      int c = 0;
      for (int q = 0; q < code_bits; ++q) c |= int((plane[q] >> b) & 1u) << q;
      slots[k * d + 32 * w + b] = uint8_t(c);
    }
  }
}

__global__ void __launch_bounds__(kThreads)
quantize_polar_kernel(const void* __restrict__ keys, int key_dtype, int64_t n, int64_t ldk, int d, int code_bits,
                      int words, int tk, int nl, const float* __restrict__ piT, const float* __restrict__ gT,
                      const float* __restrict__ ptab, uint32_t* __restrict__ codes, uint32_t* __restrict__ signs,
                      float* __restrict__ norms, float* __restrict__ rnorms) {
  extern __shared__ float smem[];
  const int ds = d + 1;
  float* buf0 = smem;                                  // keys, then the radii, then p = G r
  float* buf1 = smem + size_t(tk) * ds;                // z, then r = z - z_hat
  float* nrm = buf1 + size_t(tk) * ds;
  float* tab = nrm + tk;                               // [nl][kPolarTab]
  uint8_t* slots = reinterpret_cast<uint8_t*>(tab + nl * kPolarTab);  // [tk][d]
  const int tid = threadIdx.x;
  const int levels = 1 << code_bits;
  const int64_t base = int64_t(blockIdx.x) * tk;
  for (int i = tid; i < nl * kPolarTab; i += kThreads) tab[i] = ptab[i];
  auto stage = [&](auto load) {
#pragma unroll 8
    for (int p = tid; p < tk * d; p += kThreads) {
      const int k = p / d, i = p - k * d;
      const int64_t key = base + k;
      const float v = load((key < n ? key : n - 1) * ldk + i);
      buf0[k * ds + i] = key < n ? v : 0.0f;
    }
  };
  if (key_dtype == TQ_BF16)
    stage([&](int64_t off) { return __uint_as_float(uint32_t(static_cast<const uint16_t*>(keys)[off]) << 16); });
  else
    stage([&](int64_t off) { return static_cast<const float*>(keys)[off]; });
  __syncthreads();
  for (int k = tid; k < tk; k += kThreads) {
    float s = 0.0f;
    for (int i = 0; i < d; ++i) s = fmaf(buf0[k * ds + i], buf0[k * ds + i], s);
    const float nk = sqrtf(s);
    nrm[k] = nk;
    if (base + k < n) norms[base + k] = nk;
  }
  __syncthreads();
  const int groups = tk / 4, quads = (d + 3) / 4;
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, j0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(piT, d, buf0 + (4 * kg) * ds, ds, j0, a);
    for (int r = 0; r < 4; ++r) {
      const float nk = nrm[4 * kg + r];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < d) buf1[(4 * kg + r) * ds + j0 + c] = nk > 0.0f ? a[r][c] / nk : 0.0f;
    }
  }
  __syncthreads();
  // level 1: pairs of coordinates -> angle in [0, 2 pi) and radius
  const int h1 = d >> 1;
  for (int p = tid; p < tk * h1; p += kThreads) {
    const int k = p / h1, i = p - k * h1;
    const float x = buf1[k * ds + 2 * i], y = buf1[k * ds + 2 * i + 1];
    float a = atan2f(y, x);
    a = a < 0.0f ? a + 6.2831853071795865f : a;
    slots[k * d + i] = uint8_t(polar_code(a, tab, levels));
    buf0[k * ds + i] = sqrtf(fmaf(x, x, y * y));
  }
  if (tid < tk) slots[tid * d + d - 1] = 0;
  // levels 2 .. nl: pairs of radii -> angle in [0, pi/2] and radius
  for (int l = 2; l <= nl; ++l) {
    __syncthreads();
    const int cnt = d >> l, src = polar_off(d, l - 1), dst = polar_off(d, l);
    for (int p = tid; p < tk * cnt; p += kThreads) {
      const int k = p / cnt, i = p - k * cnt;
      const float x = buf0[k * ds + src + 2 * i], y = buf0[k * ds + src + 2 * i + 1];
      slots[k * d + dst + i] = uint8_t(polar_code(atan2f(y, x), tab + (l - 1) * kPolarTab, levels));
      buf0[k * ds + dst + i] = sqrtf(fmaf(x, x, y * y));
    }
  }
  __syncthreads();
  // r = z - z_hat in place
  for (int p = tid; p < tk * d; p += kThreads) {
    const int k = p / d, j = p - k * d;
    buf1[k * ds + j] -= polar_zhat(slots + k * d, d, nl, j, tab);
  }
  __syncthreads();
  for (int p = tid; p < tk * words; p += kThreads) {
    const int k = p / words, w = p - k * words;
    uint32_t plane[5] = {0u, 0u, 0u, 0u, 0u};
    for (int b = 0; b < 32 && 32 * w + b < d; ++b) {
      const int c = slots[k * d + 32 * w + b];
      for (int q = 0; q < code_bits; ++q) plane[q] |= uint32_t((c >> q) & 1) << b;
    }
    const int64_t key = base + k;
    if (key < n)
      for (int q = 0; q < code_bits; ++q) codes[key * int64_t(code_bits) * words + int64_t(q) * words + w] = plane[q];
  }
  for (int k = tid; k < tk; k += kThreads) {
    float s = 0.0f;
    for (int i = 0; i < d; ++i) s = fmaf(buf1[k * ds + i], buf1[k * ds + i], s);
    if (base + k < n) rnorms[base + k] = sqrtf(s);
  }
  __syncthreads();  // buf0 (radii) is overwritten by p = G r below
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, j0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(gT, d, buf1 + (4 * kg) * ds, ds, j0, a);
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < d) buf0[(4 * kg + r) * ds + j0 + c] = a[r][c];
  }
  __syncthreads();
  for (int p = tid; p < tk * words; p += kThreads) {
    const int k = p / words, w = p - k * words;
    uint32_t word = 0u;
    for (int b = 0; b < 32 && 32 * w + b < d; ++b) word |= uint32_t(buf0[k * ds + 32 * w + b] > 0.0f) << b;
    const int64_t key = base + k;
    if (key < n) signs[key * words + w] = word;
  }
}

// scores of polar keys: per block tk keys of one group, z_hat composed into
// LDS once, then one thread per key and 4 queries at a time
__global__ void __launch_bounds__(kThreads)
logits_polar_kernel(const float* __restrict__ vw, int64_t nq, int d, int code_bits, int words, int tk, int nl,
                    int64_t n, int64_t stride, int64_t half, const uint32_t* __restrict__ codes,
                    const uint32_t* __restrict__ signs, const float* __restrict__ norms,
                    const float* __restrict__ rnorms, const float* __restrict__ ptab, float* __restrict__ scores) {
  extern __shared__ float smem[];
  const int ds = d + 1;
  float* zh = smem;                       // [tk][ds]
  float* qv = zh + size_t(tk) * ds;       // [d][8]: v then w of 4 queries
  float* tab = qv + size_t(8) * d;
  uint8_t* slots = reinterpret_cast<uint8_t*>(tab + nl * kPolarTab);
  const int64_t g = blockIdx.y;
  const int64_t base = int64_t(blockIdx.x) * tk;  // within the group
  for (int i = threadIdx.x; i < nl * kPolarTab; i += kThreads) tab[i] = ptab[i];
  polar_unpack(codes + g * n * int64_t(code_bits) * words, base, n, d, code_bits, words, tk, slots);
  __syncthreads();
  for (int p = threadIdx.x; p < tk * d; p += kThreads) {
    const int k = p / d, j = p - k * d;
    zh[k * ds + j] = polar_zhat(slots + k * d, d, nl, j, tab);
  }
  const float kappa = 1.2533141373155002512f / float(d);
  const int k = threadIdx.x;
  const int64_t t = base + k;
  const int64_t key = g * n + (t < n ? t : n - 1);
  const float nk = norms[key], rho = rnorms[key];
  for (int64_t q0 = 0; q0 < nq; q0 += 4) {
    const int qc = int(nq - q0 < 4 ? nq - q0 : 4);
    __syncthreads();
    for (int p = threadIdx.x; p < 4 * d; p += kThreads) {
      const int q = p / d, j = p - q * d;
      const float* src = vw + (g * nq + q0 + (q < qc ? q : 0)) * stride;
      qv[8 * j + q] = q < qc ? src[j] : 0.f;
      qv[8 * j + 4 + q] = q < qc ? src[half + j] : 0.f;
    }
    __syncthreads();
    if (k >= tk || t >= n) continue;
    float a1[4] = {0.f, 0.f, 0.f, 0.f}, a2[4] = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < words; ++w) {
      const uint32_t sw = signs[key * words + w];
      for (int b = 0; b < 32 && 32 * w + b < d; ++b) {
        const int j = 32 * w + b;
        const float cv = zh[k * ds + j];
        const float sg = ((sw >> b) & 1u) ? 1.0f : -1.0f;
        const float4 vv = *reinterpret_cast<const float4*>(qv + 8 * j);
        const float4 ww = *reinterpret_cast<const float4*>(qv + 8 * j + 4);
        a1[0] = fmaf(vv.x, cv, a1[0]);
        a1[1] = fmaf(vv.y, cv, a1[1]);
        a1[2] = fmaf(vv.z, cv, a1[2]);
        a1[3] = fmaf(vv.w, cv, a1[3]);
        a2[0] = fmaf(ww.x, sg, a2[0]);
        a2[1] = fmaf(ww.y, sg, a2[1]);
        a2[2] = fmaf(ww.z, sg, a2[2]);
        a2[3] = fmaf(ww.w, sg, a2[3]);
      }
    }
    const float corr = rho * kappa;
    for (int q = 0; q < qc; ++q) scores[(g * nq + q0 + q) * n + t] = nk * fmaf(corr, a2[q], a1[q]);
  }
}

// stage-1 reconstruction of polar keys: n Pi^T z_hat
__global__ void __launch_bounds__(kThreads)
dequant_polar_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms, int64_t n, int d,
                     int code_bits, int words, int tk, int nl, const float* __restrict__ pi,
                     const float* __restrict__ ptab, float* __restrict__ khat) {
  extern __shared__ float smem[];
  const int ds = d + 1;
  float* zh = smem;
  float* tab = zh + size_t(tk) * ds;
  uint8_t* slots = reinterpret_cast<uint8_t*>(tab + nl * kPolarTab);
  const int tid = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * tk;
  for (int i = tid; i < nl * kPolarTab; i += kThreads) tab[i] = ptab[i];
  polar_unpack(codes, base, n, d, code_bits, words, tk, slots);
  __syncthreads();
  for (int p = tid; p < tk * d; p += kThreads) {
    const int k = p / d, j = p - k * d;
    zh[k * ds + j] = polar_zhat(slots + k * d, d, nl, j, tab);
  }
  __syncthreads();
  const int groups = tk / 4, quads = (d + 3) / 4;
  for (int p = tid; p < groups * quads; p += kThreads) {
    const int kg = p / quads, j0 = 4 * (p - kg * quads);
    float a[4][4];
    product4x4(pi, d, zh + (4 * kg) * ds, ds, j0, a);
    for (int r = 0; r < 4; ++r) {
      const int64_t key = base + 4 * kg + r;
      if (key >= n) continue;
      const float nk = norms[key];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < d) khat[key * d + j0 + c] = nk * a[r][c];
    }
  }
}

int tile_keys(int d, int buffers, size_t budget, int cap) {
  size_t per = size_t(buffers) * (d + 1) * sizeof(float);
  int tk = int(budget / per);
  tk = tk / 4 * 4;
  if (tk > cap) tk = cap;
  if (tk < 4) tk = 4;
  return tk;
}

template <class K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

}  // namespace

hipError_t launch_quantize_v1(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                              uint32_t* codes, uint32_t* signs, float* norms, float* rnorms,
                              hipStream_t stream) {
  const int d = h->d;
  const int tk = tile_keys(d, 2, 64 * 1024, 64);
  const size_t lds = (size_t(2) * tk * (d + 1) + tk + 4 * kMaxLevels) * sizeof(float);
  hipError_t e = allow_lds(quantize_ref_kernel, lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (n + tk - 1) / tk;
  hipLaunchKernelGGL(quantize_ref_kernel, dim3(unsigned(blocks)), dim3(kThreads), lds, stream, keys,
                     key_dtype, n, ldk, d, h->code_bits, h->words, tk, h->d_piT, h->d_gT, h->cb, codes,
                     signs, norms, rnorms, h->hi, h->hi_words, h->cbh);
  return hipGetLastError();
}

hipError_t launch_query_prep(const tq_ctx* h, const float* queries, int64_t count, float* vw,
                             hipStream_t stream) {
  const int d = h->d;
  const size_t lds = size_t(2) * d * sizeof(float);
  hipLaunchKernelGGL(query_prep_kernel, dim3(unsigned(count)), dim3(kThreads), lds, stream, queries, d,
                     h->d_piT, h->d_gT, vw, vw_stride(d), vw_half(d));
  return hipGetLastError();
}

hipError_t launch_logits_v1(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq,
                            const uint32_t* codes, const uint32_t* signs, const float* norms,
                            const float* rnorms, int64_t n, float* scores, hipStream_t stream) {
  const int d = h->d;
  const size_t lds = (2 * kMaxLevels + size_t(8) * d) * sizeof(float);
  const dim3 grid(static_cast<uint32_t>((n + kThreads - 1) / kThreads), static_cast<uint32_t>(groups));
  auto launch = [&](auto kernel) {
    hipError_t e = allow_lds(kernel, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, stream, vw, nq, d, h->code_bits, h->words, n,
                       vw_stride(d), vw_half(d), codes, signs, norms, rnorms, scores, h->cb, h->hi, h->hi_words,
                       h->cbh);
    return hipGetLastError();
  };
  switch (h->code_bits + (h->hi > 0 ? 1 : 0)) {
    case 1: return launch(logits_ref_kernel<1>);
    case 2: return launch(logits_ref_kernel<2>);
    case 3: return launch(logits_ref_kernel<3>);
    case 4: return launch(logits_ref_kernel<4>);
    case 5: return launch(logits_ref_kernel<5>);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequant_v1(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n,
                             float* khat, hipStream_t stream) {
  const int d = h->d;
  const int tk = tile_keys(d, 1, 64 * 1024, 64);
  const size_t lds = (size_t(tk) * (d + 1) + 2 * kMaxLevels) * sizeof(float);
  hipError_t e = allow_lds(dequant_ref_kernel, lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (n + tk - 1) / tk;
  hipLaunchKernelGGL(dequant_ref_kernel, dim3(unsigned(blocks)), dim3(kThreads), lds, stream, codes, norms,
                     n, d, h->code_bits, h->words, tk, h->d_pi, h->cb, khat, h->hi, h->hi_words, h->cbh);
  return hipGetLastError();
}

hipError_t launch_dequant_prod_v1(const tq_ctx* h, const uint32_t* codes, const uint32_t* signs,
                                  const float* norms, const float* rnorms, int64_t n, float* out,
                                  hipStream_t stream) {
  const int d = h->d;
  const int tk = tile_keys(d, 2, 64 * 1024, 64);
  const size_t lds = (size_t(2) * tk * (d + 1) + 2 * kMaxLevels) * sizeof(float);
  hipError_t e = allow_lds(dequant_prod_ref_kernel, lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (n + tk - 1) / tk;
  const float kappa = float(1.2533141373155002512 / double(d));  // sqrt(pi/2) / d
  hipLaunchKernelGGL(dequant_prod_ref_kernel, dim3(unsigned(blocks)), dim3(kThreads), lds, stream, codes, signs,
                     norms, rnorms, n, d, h->code_bits, h->words, tk, h->d_pi, h->d_g, h->cb, kappa, out, h->hi,
                     h->hi_words, h->cbh);
  return hipGetLastError();
}

// LDS bytes of a polar tile: float buffers plus the level table and the
// slot bytes (rounded to 4)
static size_t polar_lds(int d, int tk, int fbufs, int nl, size_t extra_floats) {
  return (size_t(fbufs) * tk * (d + 1) + extra_floats + size_t(nl) * kPolarTab) * sizeof(float) +
         (size_t(tk) * d + 3) / 4 * 4;
}

hipError_t launch_quantize_polar(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                                 uint32_t* codes, uint32_t* signs, float* norms, float* rnorms, hipStream_t stream) {
  const int d = h->d;
  const int tk = tile_keys(d, 2, 60 * 1024, 64);
  const size_t lds = polar_lds(d, tk, 2, h->polar_levels, tk);
  hipError_t e = allow_lds(quantize_polar_kernel, lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (n + tk - 1) / tk;
  hipLaunchKernelGGL(quantize_polar_kernel, dim3(unsigned(blocks)), dim3(kThreads), lds, stream, keys, key_dtype, n,
                     ldk, d, h->code_bits, h->words, tk, h->polar_levels, h->d_piT, h->d_gT, h->d_polar_tab, codes,
                     signs, norms, rnorms);
  return hipGetLastError();
}

hipError_t launch_logits_polar(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                               const uint32_t* signs, const float* norms, const float* rnorms, int64_t n,
                               float* scores, hipStream_t stream) {
  const int d = h->d;
  // keys per block: z_hat rows and slot bytes within about 140 KB beside
  // the query rows (8 d floats) and the level table
  const int64_t room = int64_t(140) * 1024 - int64_t(8) * d * 4 - int64_t(h->polar_levels) * kPolarTab * 4;
  int64_t tk64 = room / (int64_t(d + 1) * 4 + d);
  tk64 = tk64 > kThreads ? kThreads : (tk64 < 1 ? 1 : tk64);
  const int tk = int(tk64);
  const size_t lds = polar_lds(d, tk, 1, h->polar_levels, size_t(8) * d);
  hipError_t e = allow_lds(logits_polar_kernel, lds);
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<uint32_t>((n + tk - 1) / tk), static_cast<uint32_t>(groups));
  hipLaunchKernelGGL(logits_polar_kernel, grid, dim3(kThreads), lds, stream, vw, nq, d, h->code_bits, h->words, tk,
                     h->polar_levels, n, vw_stride(d), vw_half(d), codes, signs, norms, rnorms, h->d_polar_tab,
                     scores);
  return hipGetLastError();
}

hipError_t launch_dequant_polar(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n, float* khat,
                                hipStream_t stream) {
  const int d = h->d;
  const int tk = tile_keys(d, 1, 56 * 1024, 64);
  const size_t lds = polar_lds(d, tk, 1, h->polar_levels, 0);
  hipError_t e = allow_lds(dequant_polar_kernel, lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (n + tk - 1) / tk;
  hipLaunchKernelGGL(dequant_polar_kernel, dim3(unsigned(blocks)), dim3(kThreads), lds, stream, codes, norms, n, d,
                     h->code_bits, h->words, tk, h->polar_levels, h->d_pi, h->d_polar_tab, khat);
  return hipGetLastError();
}

}  // namespace tqdev
