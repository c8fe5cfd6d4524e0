// Matrix-core quantize kernel for d = 128 and bf16 keys (gfx950 MFMA).
//
// Stages ("TurboQuant tutorial" (gitcode.csdn.net), PolarQuant and QJL
// sections; "TurboQuant digest" (juejin.cn) section 2):
//   n = ||k||, z = Pi k / n, idx_j = #{t_i <= z_j}, r = z - c[idx],
//   rho = ||r||, beta = [G r > 0], packed into bit planes.
//
// Both projections are dense contractions and run on the matrix cores, with
// operands split so that the float32 result is as good as a float32 dot
// product:
//   * z' = Pi k: Pi = P_hi + P_mid + P_lo exactly (three bfloat16 pieces of
//     each float32 entry) and a bf16 key is exact, so every product is exact
//     and only the float32 accumulation rounds (3 MFMA passes).
//   * p = G r: G * 2^10 and r * 2^12 are each split into two float16 pieces
//     (22 bits); hi*hi + hi*lo + lo*hi (3 passes) leaves an error below
//     2^-21 sum_j |G_mj r_j|, under 1e-6 of the JL-normalised value p/sqrt(d).
//     The power-of-two scales do not change signs.
//   * n = ||Pi k|| = ||k|| (Pi orthogonal), from the float32 z'.
//
// Work split: a block of 4 waves takes 32 keys at a time (one 32 x 32 x 16
// MFMA tile in N); wave w owns output coordinates [32w, 32w + 32), i.e. bit
// word w of every plane, and keeps its slices of Pi (3 bf16 pieces) and G (2
// f16 pieces) in registers for the whole run.  Lane l holds, for key l % 32,
// the 16 coordinates 8(r/4) + 4(l/32) + (r%4), r = 0..15, of its word.  The
// residual goes through LDS to every wave as the B operand of p = G r; the
// host orders G's columns so that the K-slots of each MFMA step match the
// coordinates a lane already holds (no register shuffles).  Two barriers
// per tile: one to sum ||z'||^2 over the 4 words, one to publish r.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQThreads = 256;
constexpr int kSteps = 8;            // K = 128 in steps of 16
constexpr float kResidualScale = 4096.0f;

// Binary descent over the ascending thresholds held in LDS: at level p the
// candidate index is idx + 2^p and its lower threshold t[idx + 2^p - 1]
// (a tie goes to the upper cell), so idx = #{ i : t_i <= z } after B
// levels.  Per-lane LDS reads keep the descent free of selects, which the
// compiler would otherwise turn into divergent branches; the 31 table
// entries sit in distinct banks.
template <int B>
__device__ __forceinline__ int descend(float z, const float* tt) {
  int idx = 0;
#pragma unroll
  for (int p = B - 1; p >= 0; --p) idx += (z >= tt[idx + (1 << p) - 1]) ? (1 << p) : 0;
  return idx;
}

// Lane bits are gathered in accumulator order (element r at bit r); element
// r sits at row 8(r/4) + 4g + r%4 of the word, so nibble j moves to bits
// [8j + 4g, 8j + 4g + 4).  The partner lane (g ^ 1) fills the other nibbles.
__device__ __forceinline__ uint32_t spread_nibbles(uint32_t x, int g) {
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  return x << (4 * g);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int B>
__global__ void __launch_bounds__(kQThreads, 2)
quantize_mfma128_kernel(const uint16_t* __restrict__ keys, int64_t n, int64_t ldk,
                        const uint4* __restrict__ pi_frag, const uint4* __restrict__ g_frag, Codebook cb,
                        uint32_t* __restrict__ codes, uint32_t* __restrict__ signs, float* __restrict__ norms,
                        float* __restrict__ rnorms, int64_t tiles) {
  // residual exchange [buf][piece][step][lane group][key] (8 halves each)
  __shared__ uint4 xb[2][2][kSteps][2][32];
  __shared__ float zsq[2][4][32];
  __shared__ float rsq[2][4][32];
  // key tiles, double buffered: 32 rows of 128 bf16, row stride 272 bytes so
  // that the 8 lanes of one LDS pass (8 consecutive keys) hit distinct banks
  __shared__ uint4 ktile[2][32][17];
  __shared__ float tabc[kMaxLevels], tabt[kMaxLevels];

  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kl = lane & 31;
  const int g = lane >> 5;

  bf16x8 api[kSteps][3];
  f16x8 ag[kSteps][2];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
#pragma unroll
    for (int q = 0; q < 3; ++q) api[s][q] = __builtin_bit_cast(bf16x8, pi_frag[((w * kSteps + s) * 3 + q) * 64 + lane]);
#pragma unroll
    for (int q = 0; q < 2; ++q) ag[s][q] = __builtin_bit_cast(f16x8, g_frag[((w * kSteps + s) * 2 + q) * 64 + lane]);
  }

  if (threadIdx.x < kMaxLevels) {
    tabc[threadIdx.x] = cb.c[threadIdx.x];
    tabt[threadIdx.x] = cb.t[threadIdx.x];
  }
  // thread t stages bytes [32 (t % 8), +32) of key t / 8 of a tile
  const int sk = threadIdx.x >> 3, sc = threadIdx.x & 7;
  auto fetch = [&](int64_t tile, uint4& a, uint4& b) {
    const int64_t k = tile * 32 + sk;
    if (tile < tiles && k < n) {
      const uint4* row = reinterpret_cast<const uint4*>(keys + k * ldk);
      a = row[2 * sc];
      b = row[2 * sc + 1];
    } else {
      a = b = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  {
    uint4 a, b;
    fetch(blockIdx.x, a, b);
    ktile[0][sk][2 * sc] = a;
    ktile[0][sk][2 * sc + 1] = b;
  }
  __syncthreads();

  int buf = 0;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t key = tile * 32 + kl;
    const bool valid = key < n;
    // B operand of z' = Pi k: lane supplies k[16 s + 8 g .. + 7] of its key
    bf16x8 kf[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) kf[s] = __builtin_bit_cast(bf16x8, ktile[buf][kl][2 * s + g]);
    // next tile's keys: in flight during this tile's work, stored to LDS
    // before the second barrier
    uint4 na, nb;
    fetch(tile + gridDim.x, na, nb);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(api[s][0], kf[s], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(api[s][1], kf[s], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(api[s][2], kf[s], acc, 0, 0, 0);
    }
    // ||z'||^2 over this word, then over the 4 words
    float ss = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ss = fmaf(acc[r], acc[r], ss);
    ss += __shfl_xor(ss, 32);
    if (g == 0) zsq[buf][w][kl] = ss;
    __syncthreads();
    const float nk = sqrtf((zsq[buf][0][kl] + zsq[buf][1][kl]) + (zsq[buf][2][kl] + zsq[buf][3][kl]));
    const float inv = nk > 0.0f ? 1.0f / nk : 0.0f;

    uint32_t cw[B];
#pragma unroll
    for (int p = 0; p < B; ++p) cw[p] = 0u;
    float rr = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float rs[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 8 * h + e + u;
          const float z = acc[r] * inv;
          const int idx = descend<B>(z, tabt);
          const float res = z - tabc[idx];
#pragma unroll
          for (int p = 0; p < B; ++p) cw[p] |= uint32_t((idx >> p) & 1) << r;
          rr = fmaf(res, res, rr);
          rs[u] = res * kResidualScale;
        }
        const f16x2 h2 = {(_Float16)rs[0], (_Float16)rs[1]};
        hi[e >> 1] = __builtin_bit_cast(uint32_t, h2);
        lo[e >> 1] = pack_f16x2(rs[0] - float(h2[0]), rs[1] - float(h2[1]));
      }
      xb[buf][0][2 * w + h][g][kl] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      xb[buf][1][2 * w + h][g][kl] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
#pragma unroll
    for (int p = 0; p < B; ++p) {
      cw[p] = spread_nibbles(cw[p], g);
      cw[p] |= __shfl_xor(cw[p], 32);
    }
    rr += __shfl_xor(rr, 32);
    if (g == 0) {
      rsq[buf][w][kl] = rr;
      if (valid)
#pragma unroll
        for (int p = 0; p < B; ++p) codes[(key * B + p) * 4 + w] = cw[p];
    }
    ktile[buf ^ 1][sk][2 * sc] = na;
    ktile[buf ^ 1][sk][2 * sc + 1] = nb;
    __syncthreads();
    if (w == 0 && g == 0 && valid) {
      norms[key] = nk;
      rnorms[key] = sqrtf((rsq[buf][0][kl] + rsq[buf][1][kl]) + (rsq[buf][2][kl] + rsq[buf][3][kl]));
    }
    // p = G r for this wave's 32 output coordinates
    f32x16 acc2 = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const f16x8 rh = __builtin_bit_cast(f16x8, xb[buf][0][s][g][kl]);
      const f16x8 rl = __builtin_bit_cast(f16x8, xb[buf][1][s][g][kl]);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ag[s][1], rh, acc2, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ag[s][0], rl, acc2, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ag[s][0], rh, acc2, 0, 0, 0);
    }
    uint32_t sw = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) sw |= uint32_t(acc2[r] > 0.0f) << r;
    sw = spread_nibbles(sw, g);
    sw |= __shfl_xor(sw, 32);
    if (g == 0 && valid) signs[key * 4 + w] = sw;
    buf ^= 1;
  }
}

template <int B>
hipError_t launch_b(const tq_ctx* h, const void* keys, int64_t n, int64_t ldk, uint32_t* codes, uint32_t* signs,
                    float* norms, float* rnorms, hipStream_t stream) {
  const int64_t tiles = (n + 31) / 32;
  int64_t blocks = tiles < 512 ? tiles : 512;  // two resident blocks on each of 256 CUs
  hipLaunchKernelGGL(quantize_mfma128_kernel<B>, dim3(static_cast<uint32_t>(blocks)), dim3(kQThreads), 0, stream,
                     static_cast<const uint16_t*>(keys), n, ldk, reinterpret_cast<const uint4*>(h->d_pi_frag),
                     reinterpret_cast<const uint4*>(h->d_g_frag), h->cb, codes, signs, norms, rnorms, tiles);
  return hipGetLastError();
}

}  // namespace

bool quantize_mfma128_supported(const tq_ctx* h, const void* keys, int key_dtype, int64_t ldk) {
  return h->d == 128 && key_dtype == TQ_BF16 && h->d_pi_frag && h->d_g_frag && (ldk % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(keys) & 15u) == 0 && h->code_bits >= 1 && h->code_bits <= 4;
}

hipError_t launch_quantize_mfma128(const tq_ctx* h, const void* keys, int64_t n, int64_t ldk, uint32_t* codes,
                                   uint32_t* signs, float* norms, float* rnorms, hipStream_t stream) {
  switch (h->code_bits) {
    case 1: return launch_b<1>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    case 2: return launch_b<2>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    case 3: return launch_b<3>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    case 4: return launch_b<4>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqdev
