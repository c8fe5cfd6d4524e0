// Matrix-core scorer for many queries against packed keys, d <= 256.
//
// Method ("TurboQuant digest" section 2; "TurboQuant deep review",
// error-compensation section): the score of query q against a packed key is
//     n * ( <v, c[idx]> + rho * sqrt(pi/2) / d * <w, 2 beta - 1> ),
// v = Pi q, w = G v.  With many queries per key set (search), both inner
// products are dense contractions over the coordinates: scores = n (V C^T +
// kappa rho W Sgn^T) for the query rows V, W and the keys' level values C
// and signs Sgn.  They run on the matrix cores, 32 x 32 x 16 f16 tiles:
//   * C: two float16 pieces of 2^10 c[level] (22 bits, no denormals);
//   * Sgn: +-1, exact;
//   * V, W: one float16 piece each, every query row scaled by a power of two
//     so that its norm lies in [2^9, 2^10).  Rounding each element to 11
//     bits moves <v, c> by at most 2^-12 ||v|| ||c|| (Cauchy-Schwarz, and
//     ||c[idx]|| is about 1) and the sign term by at most 2^-12 ||w||_1
//     sqrt(pi/2) rho / d: together about half of the 1e-3 ||q|| n bound in
//     the worst case, far less for random data.
// Three passes per K step: V C_hi, V C_lo (one accumulator), W Sgn (another).
//
// Work split: a block of 4 waves takes 128 queries (wave w: rows 32w ..
// 32w + 31, A operands loaded once into registers) and walks 32-key tiles.
// Per tile, thread (key, word) unpacks 32 coordinates of one key from its
// bit planes into LDS rows of f16 values (hi, lo) and signs, through small
// LDS tables indexed by packed index bits; the next tile's words are loaded
// while the current tile is multiplied.  Rows past nq and keys past the end
// repeat the last one and store the same value there, so stores carry no
// branch.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kTileKeys = 32;                     // MFMA N
constexpr int kMaxSteps = 16;                     // K = d padded to 16, d <= 256
constexpr int kRowHalves = kMaxSteps * 16 + 8;    // staged row, padded: 132 dwords, conflict-free b128 reads
constexpr float kCScale = 1024.0f;                // on the level values

// coordinates per value-table lookup, by B: the index bits of E coordinates
// of every plane address one entry of E hi and E lo halves
template <int B>
struct Unpack {
  static constexpr int E = B == 1 ? 8 : B == 2 ? 4 : 2;
  static constexpr int kEntries = 1 << (E * B);
  static constexpr int kHalves = 2 * E;
};

__device__ __forceinline__ f16x8 to_f16x8(const float4& a, const float4& b, float s) {
  f16x8 h;
  h[0] = static_cast<_Float16>(a.x * s);
  h[1] = static_cast<_Float16>(a.y * s);
  h[2] = static_cast<_Float16>(a.z * s);
  h[3] = static_cast<_Float16>(a.w * s);
  h[4] = static_cast<_Float16>(b.x * s);
  h[5] = static_cast<_Float16>(b.y * s);
  h[6] = static_cast<_Float16>(b.z * s);
  h[7] = static_cast<_Float16>(b.w * s);
  return h;
}

template <int B>
__global__ void __launch_bounds__(kThreads, 2)
score_mfma_kernel(const float* __restrict__ vw, int64_t vw_stride, int64_t vw_half, int64_t nq, int ksteps,
                  const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
                  const float* __restrict__ norms, const float* __restrict__ rnorms, int words, int64_t nkeys,
                  float* __restrict__ scores, int64_t sstride, Codebook cb, float kappa, int64_t tiles_per_block) {
  using U = Unpack<B>;
  constexpr int E = U::E;
  __shared__ uint4 chi4[kTileKeys * kRowHalves / 8];
  __shared__ uint4 clo4[kTileKeys * kRowHalves / 8];
  __shared__ uint4 sg4[kTileKeys * kRowHalves / 8];
  __shared__ _Float16 vtab[U::kEntries * U::kHalves];
  __shared__ uint4 stab[256];  // byte -> 8 halves of +-1
  __shared__ float inv_s[2][128];
  _Float16* chi = reinterpret_cast<_Float16*>(chi4);
  _Float16* clo = reinterpret_cast<_Float16*>(clo4);
  _Float16* sgv = reinterpret_cast<_Float16*>(sg4);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kl = lane & 31, g = lane >> 5;
  const int64_t grp = blockIdx.z;
  vw += grp * nq * vw_stride;
  codes += grp * nkeys * B * words;
  signs += grp * nkeys * words;
  norms += grp * nkeys;
  rnorms += grp * nkeys;
  scores += grp * nq * sstride;

  // tables: value entries (hi then lo halves of 2^10 c[level] for E
  // coordinates) and sign bytes
  for (int idx = tid; idx < U::kEntries; idx += kThreads) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int level = 0;
#pragma unroll
      for (int p = 0; p < B; ++p) level |= ((idx >> (p * E + e)) & 1) << p;
      const float x = cb.c[level] * kCScale;
      const _Float16 hi = static_cast<_Float16>(x);
      vtab[idx * U::kHalves + e] = hi;
      vtab[idx * U::kHalves + E + e] = static_cast<_Float16>(x - static_cast<float>(hi));
    }
  }
  {
    _Float16 h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = ((tid >> e) & 1) ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(-1.0f);
    stab[tid] = __builtin_bit_cast(uint4, f16x8{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]});
  }

  // A operands of this wave's 32 query rows (rows past nq repeat the last)
  const int64_t qrow = blockIdx.x * 128 + 32 * w + kl;
  const float* vrow = vw + (qrow < nq ? qrow : nq - 1) * vw_stride + 8 * g;
  // pass 1: norms of the row's v and w (the row's two halves sit in lanes
  // l and l ^ 32); pass 2 reloads them (from cache) scaled into float16
  float ssv = 0.0f, ssw = 0.0f;
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    if (s < ksteps) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 a = *reinterpret_cast<const float4*>(vrow + 16 * s + 4 * h);
        const float4 b = *reinterpret_cast<const float4*>(vrow + vw_half + 16 * s + 4 * h);
        ssv += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
        ssw += b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
      }
    }
  }
  ssv += __shfl_xor(ssv, 32);
  ssw += __shfl_xor(ssw, 32);
  auto pow2_scale = [](float ss) {
    if (!(ss > 0.0f)) return 1.0f;
    int e = 0;
    (void)frexpf(sqrtf(ss), &e);
    return ldexpf(1.0f, 10 - e);  // norm * scale in [2^9, 2^10)
  };
  const float sv = pow2_scale(ssv), sw = pow2_scale(ssw);
  f16x8 av[kMaxSteps], aw[kMaxSteps];
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    if (s < ksteps) {
      av[s] = to_f16x8(*reinterpret_cast<const float4*>(vrow + 16 * s),
                       *reinterpret_cast<const float4*>(vrow + 16 * s + 4), sv);
      aw[s] = to_f16x8(*reinterpret_cast<const float4*>(vrow + vw_half + 16 * s),
                       *reinterpret_cast<const float4*>(vrow + vw_half + 16 * s + 4), sw);
    } else {
      av[s] = aw[s] = f16x8{};
    }
  }
  if (g == 0) {
    inv_s[0][32 * w + kl] = 1.0f / (sv * kCScale);
    inv_s[1][32 * w + kl] = kappa / sw;
  }

  // staging role: thread (key kk, word wi) of the tile, 32 coordinates
  const int kk = tid / words, wi = tid % words;
  const bool stager = tid < kTileKeys * words;
  const int64_t ntiles = (nkeys + kTileKeys - 1) / kTileKeys;
  const int64_t t0 = blockIdx.y * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < ntiles ? t0 + tiles_per_block : ntiles;
  auto fetch = [&](int64_t tile, uint32_t (&pw)[B + 1]) {
    int64_t key = tile * kTileKeys + kk;
    key = key < nkeys ? key : nkeys - 1;
#pragma unroll
    for (int p = 0; p < B; ++p) pw[p] = stager ? codes[(key * B + p) * words + wi] : 0u;
    pw[B] = stager ? signs[key * words + wi] : 0u;
  };
  uint32_t nw[B + 1];
  if (t0 < t1) fetch(t0, nw);

  for (int64_t tile = t0; tile < t1; ++tile) {
    uint32_t pw[B + 1];
#pragma unroll
    for (int p = 0; p <= B; ++p) pw[p] = nw[p];
    __syncthreads();  // the previous tile's rows are no longer read
    if (stager) {
      _Float16* rh = chi + kk * kRowHalves + 32 * wi;
      _Float16* rl = clo + kk * kRowHalves + 32 * wi;
      _Float16* rs = sgv + kk * kRowHalves + 32 * wi;
#pragma unroll
      for (int e0 = 0; e0 < 32; e0 += 8) {
        _Float16 hv[8], lv[8];
#pragma unroll
        for (int k = 0; k < 8 / E; ++k) {
          uint32_t idx = 0;
#pragma unroll
          for (int p = 0; p < B; ++p) idx |= __builtin_amdgcn_ubfe(pw[p], e0 + k * E, E) << (p * E);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            hv[k * E + e] = vtab[idx * U::kHalves + e];
            lv[k * E + e] = vtab[idx * U::kHalves + E + e];
          }
        }
        *reinterpret_cast<f16x8*>(rh + e0) = f16x8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
        *reinterpret_cast<f16x8*>(rl + e0) = f16x8{lv[0], lv[1], lv[2], lv[3], lv[4], lv[5], lv[6], lv[7]};
        *reinterpret_cast<uint4*>(rs + e0) = stab[__builtin_amdgcn_ubfe(pw[B], e0, 8)];
      }
    }
    __syncthreads();
    if (tile + 1 < t1) fetch(tile + 1, nw);
    // norm and rho of this lane's key column (keys past the end repeat the last)
    int64_t key = tile * kTileKeys + kl;
    key = key < nkeys ? key : nkeys - 1;
    const float nk = norms[key], rk = rnorms[key];
    f32x16 acc1 = {}, acc2 = {};
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
      if (s < ksteps) {
        const int off = kl * kRowHalves + 16 * s + 8 * g;
        const f16x8 bh = *reinterpret_cast<const f16x8*>(chi + off);
        const f16x8 bl = *reinterpret_cast<const f16x8*>(clo + off);
        const f16x8 bs = *reinterpret_cast<const f16x8*>(sgv + off);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s], bh, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s], bl, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(aw[s], bs, acc2, 0, 0, 0);
      }
    }
    // element r of the lane: query row 8(r/4) + 4g + r%4 of the wave, key kl
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lrow = 32 * w + 8 * (r >> 2) + 4 * g + (r & 3);
      int64_t q = blockIdx.x * 128 + lrow;
      q = q < nq ? q : nq - 1;
      scores[q * sstride + key] = nk * fmaf(rk * inv_s[1][lrow], acc2[r], acc1[r] * inv_s[0][lrow]);
    }
  }
}

template <int B>
hipError_t launch_b(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                    const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores,
                    hipStream_t stream) {
  const int64_t qtiles = (nq + 127) / 128;
  const int64_t ntiles = (n + kTileKeys - 1) / kTileKeys;
  // about four blocks per CU in all (two resident), whole tiles per block
  const int64_t want = 4 * static_cast<int64_t>(h->cus);
  int64_t splits = (want + qtiles * groups - 1) / (qtiles * groups);
  splits = splits < 1 ? 1 : splits > ntiles ? ntiles : splits;
  const int64_t tpb = (ntiles + splits - 1) / splits;
  splits = (ntiles + tpb - 1) / tpb;
  if (qtiles > 0x7FFFFFFF || splits > 65535 || groups > 65535) return hipErrorInvalidConfiguration;
  const float kappa = 1.2533141373155002512f / float(h->d);
  hipLaunchKernelGGL(score_mfma_kernel<B>, dim3(static_cast<uint32_t>(qtiles), static_cast<uint32_t>(splits),
                                                static_cast<uint32_t>(groups)),
                     dim3(kThreads), 0, stream, vw, vw_stride(h->d), vw_half(h->d), nq, (h->d + 15) / 16, codes,
                     signs, norms, rnorms, h->words, n, scores, n, h->cb, kappa, tpb);
  return hipGetLastError();
}

}  // namespace

bool score_mfma_supported(const tq_ctx* h) { return h->d <= 256 && h->code_bits >= 1 && h->code_bits <= 4; }

hipError_t launch_score_mfma(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                             const uint32_t* signs, const float* norms, const float* rnorms, int64_t n,
                             float* scores, hipStream_t stream) {
  if (n <= 0 || nq <= 0 || groups <= 0) return hipSuccess;
  switch (h->code_bits) {
    case 1: return launch_b<1>(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    case 2: return launch_b<2>(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    case 3: return launch_b<3>(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    case 4: return launch_b<4>(h, vw, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqdev
