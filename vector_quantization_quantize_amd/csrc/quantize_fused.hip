// One-kernel matrix-core quantizer for 16 <= d <= 208 (d a multiple of 8),
// float32 or bf16 keys, plain handles with a seeded (float16-exact) G.
//
// Stages ("TurboQuant tutorial" (gitcode.csdn.net), PolarQuant and QJL
// sections; "TurboQuant digest" (juejin.cn) section 2):
//   n = ||k||, z = Pi k / n, idx_j = #{t_i <= z_j}, r = z - c[idx],
//   rho = ||r||, beta = [G r > 0], packed into bit planes.
// A block holds W = ceil(d / 32) multiplying waves (and at least 4 waves,
// which all stage), wave w owning bit word w (output coordinates
// 32 w .. 32 w + 31) of both products; its rows of 2^12 Pi (two
// float16 pieces) and of 2^10 G (one piece) stay in registers for the whole
// run (at d <= 208 the fragments of both fit the 256 registers of a wave;
// larger d take the tiled general quantizer).  The block walks tiles of 32
// keys:
//   1. stage: 8 threads per key load its row in 8-element chunks
//      (coalesced), sum the squares (per-thread runs, then a 3-level tree)
//      and store their chunks as float16 pieces hi = f16(2^s k), lo =
//      f16(2^s k - hi) with 2^s n in [2^13, 2^14) (bf16 keys: one exact
//      piece);
//   2. rotate: 32 x 32 x 16 MFMA, hi hi + hi lo + lo hi per K step (bf16:
//      2 passes), each run of 8 K steps in fresh accumulators added into
//      float32 running sums; then per element z = acc / (2^12 2^s n),
//      bucketize against the thresholds (the middle one, then the half
//      that z falls in), code bits (16 per lane, the other
//      16 of the word from lane l ^ 32), r = z - c[idx] and its rho^2
//      share, r to LDS as float16 pieces of 2^12 r;
//   3. project: p = (2^10 G) r_hi + (2^10 G) r_lo, sign bits per word;
//      rho from the waves' shares in a fixed order.
// The operand tiles (rows permuted so that accumulator element e of lane l
// is coordinate 16 (l / 32) + e of the wave's 32), the piece split, the
// pass order and the chunked accumulation are the tiled general quantizer's,
// so its error analysis holds here.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTK = 32;                 // keys per tile
constexpr int kMaxW = 7;                // words (waves) at d <= 208
constexpr int kRowH = 32 * kMaxW + 8;   // halves per staged row (padding spreads the rows over the LDS banks)
constexpr int kChunkSteps = 8;          // K steps per fresh accumulator

__device__ __forceinline__ float key_scale_f(float nk) {
  if (!(nk > 0.0f)) return 1.0f;
  int e = 0;
  (void)frexpf(nk, &e);
  return ldexpf(1.0f, 14 - e);
}

// KS: K steps of the rotation (ceil(d / 16)); the projection takes
// KS2 = 2 W = 2 ceil(KS / 2) over the 32 W padded coordinates.
template <int KT, int KS>
__global__ void __launch_bounds__(64 * kMaxW, 1)
quantize_fused_kernel(const void* __restrict__ keys, int64_t n, int64_t ldk, int d, int W, int B,
                      const uint16_t* __restrict__ pi_tiles, const uint16_t* __restrict__ g_tiles, Codebook cb,
                      uint32_t* __restrict__ codes, uint32_t* __restrict__ signs, float* __restrict__ norms,
                      float* __restrict__ rnorms) {
  constexpr int kPieces = KT == TQ_F32 ? 2 : 1;
  constexpr int KS2 = 2 * ((KS + 1) / 2);
  __shared__ __align__(16) _Float16 sK[kPieces][kTK][kRowH];  // key pieces
  __shared__ __align__(16) _Float16 sR[2][kTK][kRowH];     // residual pieces
  __shared__ float sRho[kMaxW][kTK];                       // rho^2 share of each wave
  __shared__ float sInv[kTK];
  __shared__ float sC[kMaxLevels], sT[kMaxLevels];  // levels; thresholds (+inf past L - 2)
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kl = lane & 31, g = lane >> 5;
  if (tid < kMaxLevels) {
    sC[tid] = cb.c[tid];
    sT[tid] = cb.t[tid];
  }
  const int half = cb.levels / 2;  // M: levels per half of the sorted set

  // this wave's operand rows: coordinate tile w / 4, rows 32 (w % 4) + l % 32
  const int ct = w >> 2, row = 32 * (w & 3) + kl;
  f16x8 pa_h[KS], pa_l[KS], ga[KS2];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int64_t off = ((int64_t(ct) * KS + s) * 128 + row) * 32 + 8 * g;
    pa_h[s] = *reinterpret_cast<const f16x8*>(pi_tiles + off);
    pa_l[s] = *reinterpret_cast<const f16x8*>(pi_tiles + off + 16);
  }
#pragma unroll
  for (int s = 0; s < KS2; ++s) {
    const int64_t off = ((int64_t(ct) * KS2 + s) * 128 + row) * 32 + 8 * g;
    ga[s] = *reinterpret_cast<const f16x8*>(g_tiles + off);
  }
  __syncthreads();

  const int64_t tiles = (n + kTK - 1) / kTK;
  const int chunks = d >> 3;                   // 8-element chunks per row
  const int sk = tid >> 3, st = tid & 7;       // staging (threads < 256): key sk, chunks st, st + 8, ...
  const bool stager = tid < 8 * kTK;
  constexpr int kEl = KT == TQ_F32 ? 4 : 2;

  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t k0 = tile * kTK;
    // ---- 1. stage: norms, then the key pieces (zeros past d up to the K steps) ----
    if (stager) {
      const int64_t key = k0 + sk < n ? k0 + sk : n - 1;  // rows past n repeat row n - 1
      const char* rowp = static_cast<const char*>(keys) + key * ldk * kEl;
      float x[4][8];
      float ss = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int c = st + 8 * m;
        if (c < chunks) {
          if constexpr (KT == TQ_F32) {
            const float4 a = reinterpret_cast<const float4*>(rowp)[2 * c];
            const float4 b = reinterpret_cast<const float4*>(rowp)[2 * c + 1];
            x[m][0] = a.x; x[m][1] = a.y; x[m][2] = a.z; x[m][3] = a.w;
            x[m][4] = b.x; x[m][5] = b.y; x[m][6] = b.z; x[m][7] = b.w;
          } else {
            const uint4 u = reinterpret_cast<const uint4*>(rowp)[c];
            const uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[m][2 * i] = __uint_as_float(v[i] << 16);
              x[m][2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[m][e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[m][e], x[m][e], ss);
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      const float nk = sqrtf(ss);
      const float sc = key_scale_f(nk);
      if (st == 0) {
        sInv[sk] = nk > 0.0f ? 1.0f / (4096.0f * sc * nk) : 0.0f;
        if (k0 + sk < n) norms[k0 + sk] = nk;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int c = st + 8 * m;
        if (c < 2 * KS) {
          f16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = x[m][e] * sc;
            const _Float16 h = static_cast<_Float16>(v);
            hi[e] = h;
            lo[e] = static_cast<_Float16>(v - static_cast<float>(h));
          }
          *reinterpret_cast<f16x8*>(&sK[0][sk][8 * c]) = hi;
          if constexpr (kPieces == 2) *reinterpret_cast<f16x8*>(&sK[kPieces - 1][sk][8 * c]) = lo;
        }
      }
    }
    __syncthreads();
    // ---- 2. rotate: element e of lane l is coordinate 32 w + 16 g + e of key kl ----
    const bool mult = w < W;  // (wave-uniform) waves past the words only stage
    if (mult) {
      f32x16 acc = {}, run = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const f16x8 bh = *reinterpret_cast<const f16x8*>(&sK[0][kl][16 * s + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa_h[s], bh, acc, 0, 0, 0);
        if constexpr (kPieces == 2) {
          const f16x8 bl = *reinterpret_cast<const f16x8*>(&sK[kPieces - 1][kl][16 * s + 8 * g]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa_h[s], bl, acc, 0, 0, 0);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa_l[s], bh, acc, 0, 0, 0);
        if ((s + 1) % kChunkSteps == 0 || s + 1 == KS) {
          run += acc;
          acc = f32x16{};
        }
      }
      const float inv = sInv[kl];
      const int c0 = 32 * w + 16 * g;
      uint32_t hw[4] = {0u, 0u, 0u, 0u};
      float rho2 = 0.0f;
      f16x8 rh[2], rl[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool valid = c0 + e < d;
        const float z = run[e] * inv;
        // idx = #{t_i <= z} over the sorted thresholds, split at the middle
        // one: z >= t[M - 1] lies at or above t[0 .. M - 1] and only
        // t[M .. L - 2] remain to count, else below t[M - 1 ..] and only
        // t[0 .. M - 2] do (M - 1 compares instead of L - 1, same result)
        const bool upper = z >= sT[half - 1];
        int idx = upper ? half : 0;
#pragma unroll
        for (int q = 0; q < kMaxLevels / 2 - 1; ++q) {
          if (q >= half - 1) break;  // (uniform)
          idx += z >= (upper ? sT[half + q] : sT[q]) ? 1 : 0;
        }
        const float r = valid ? z - sC[idx] : 0.0f;
        idx = valid ? idx : 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) hw[p] |= uint32_t((idx >> p) & 1) << e;
        rho2 = fmaf(r, r, rho2);
        const float r2 = r * 4096.0f;
        const _Float16 h = static_cast<_Float16>(r2);
        rh[e >> 3][e & 7] = h;
        rl[e >> 3][e & 7] = static_cast<_Float16>(r2 - static_cast<float>(h));
      }
      *reinterpret_cast<f16x8*>(&sR[0][kl][c0]) = rh[0];
      *reinterpret_cast<f16x8*>(&sR[0][kl][c0 + 8]) = rh[1];
      *reinterpret_cast<f16x8*>(&sR[1][kl][c0]) = rl[0];
      *reinterpret_cast<f16x8*>(&sR[1][kl][c0 + 8]) = rl[1];
      rho2 += __shfl_xor(rho2, 32);
      if (g == 0) sRho[w][kl] = rho2;
      // the other 16 bits of each code word are in lane l ^ 32
      uint32_t full[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) full[p] = hw[p] | (__shfl_xor(hw[p], 32) << 16);
      const int64_t key = k0 + kl;
      if (g == 0 && key < n) {
        uint32_t* crow = codes + key * int64_t(B) * W;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (p < B) crow[p * W + w] = full[p];
      }
    }
    __syncthreads();
    // ---- 3. project ----
    if (mult) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < KS2; ++s) {
        const f16x8 bh = *reinterpret_cast<const f16x8*>(&sR[0][kl][16 * s + 8 * g]);
        const f16x8 bl = *reinterpret_cast<const f16x8*>(&sR[1][kl][16 * s + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ga[s], bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ga[s], bl, acc, 0, 0, 0);
      }
      const int c0 = 32 * w + 16 * g;
      uint32_t hw = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) hw |= uint32_t(c0 + e < d && acc[e] > 0.0f) << e;
      const uint32_t full = hw | (__shfl_xor(hw, 32) << 16);
      const int64_t key = k0 + kl;
      if (g == 0 && key < n) signs[key * W + w] = full;
      if (w == 0 && g == 0 && key < n) {
        float s2 = 0.0f;
        for (int v = 0; v < W; ++v) s2 += sRho[v][kl];
        rnorms[key] = sqrtf(s2);
      }
    }
  }
}

template <int KS>
hipError_t launch_ks(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk, uint32_t* codes,
                     uint32_t* signs, float* norms, float* rnorms, hipStream_t stream) {
  const int64_t tiles = (n + kTK - 1) / kTK;
  // 4 waves and 60 KB of LDS (d <= 128): two blocks share a CU
  const int64_t slots = static_cast<int64_t>(h->cus) * (h->words <= 4 ? 2 : 1);
  const dim3 grid{static_cast<uint32_t>(tiles < slots ? tiles : slots)};
  const dim3 block{static_cast<uint32_t>(64 * (h->words > 4 ? h->words : 4))};
  if (key_dtype == TQ_F32)
    hipLaunchKernelGGL((quantize_fused_kernel<TQ_F32, KS>), grid, block, 0, stream, keys, n, ldk, h->d, h->words,
                       h->code_bits, h->d_qpi_tiles, h->d_qg_tiles, h->cb, codes, signs, norms, rnorms);
  else
    hipLaunchKernelGGL((quantize_fused_kernel<TQ_BF16, KS>), grid, block, 0, stream, keys, n, ldk, h->d, h->words,
                       h->code_bits, h->d_qpi_tiles, h->d_qg_tiles, h->cb, codes, signs, norms, rnorms);
  return hipGetLastError();
}

}  // namespace

bool quantize_fused_supported(const tq_ctx* h, const void* keys, int key_dtype, int64_t ldk) {
  const int elem = key_dtype == TQ_F32 ? 4 : 2;
  return !h->polar && !h->hadamard && h->hi == 0 && h->g_f16 && h->d >= 16 && h->d <= 208 && h->d % 8 == 0 &&
         h->d_qpi_tiles && h->d_qg_tiles && h->code_bits >= 1 && h->code_bits <= 4 && !force_reference_kernels() &&
         (key_dtype == TQ_F32 || key_dtype == TQ_BF16) && (reinterpret_cast<uintptr_t>(keys) & 15u) == 0 &&
         (ldk * elem) % 16 == 0;
}

hipError_t launch_quantize_fused(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                                 uint32_t* codes, uint32_t* signs, float* norms, float* rnorms, hipStream_t stream) {
  switch ((h->d + 15) / 16) {
#define TQ_QF(KS) \
  case KS: return launch_ks<KS>(h, keys, key_dtype, n, ldk, codes, signs, norms, rnorms, stream);
    TQ_QF(1)
    TQ_QF(2)
    TQ_QF(3)
    TQ_QF(4)
    TQ_QF(5)
    TQ_QF(6)
    TQ_QF(7)
    TQ_QF(8)
    TQ_QF(9)
    TQ_QF(10)
    TQ_QF(11)
    TQ_QF(12)
    TQ_QF(13)
#undef TQ_QF
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqdev
