// General matrix-core quantizer: any d >= 16, float32 or bfloat16 keys,
// plain or fractional-width handles (gfx950 MFMA).
//
// Stages ("TurboQuant tutorial" (gitcode.csdn.net), PolarQuant and QJL
// sections; "TurboQuant digest" (juejin.cn) section 2):
//   n = ||k||, z = Pi k / n, idx_j = #{t_i <= z_j}, r = z - c[idx],
//   rho = ||r||, beta = [G r > 0], packed into bit planes.
// Both projections are dense contractions over all keys, so they run as
// tiled matrix products on the matrix cores:
//   1. prep: n = ||k|| in float32 and the keys as float16 pieces of 2^s k
//      (below), in the operand layout of step 2.
//   2. rotate: Z = (2^12 Pi) (2^s K) for tiles of 128 output coordinates x
//      128 keys, then per element: bucketize, the code bits, r = z - c[idx]
//      and rho^2 (partial sums per coordinate tile).  r goes to a scratch
//      buffer as two float16 pieces of 2^12 r, in the operand layout of
//      step 3.
//   3. project: P = (2^10 G) (2^12 R), then beta = [p > 0]; the blocks of
//      coordinate tile 0 also add up the rho^2 partials of their keys.
// Operands are split so that the float32 result is as good as a float32
// dot product:
//   * a key is scaled by the power of two 2^s that puts 2^s n in
//     [2^13, 2^14) and split into float16 hi = f16(2^s k) and
//     lo = f16(2^s k - hi) (22 significant bits; elements far below n lose
//     bits only under 2^-38 n);
//   * 2^12 Pi, 2^10 G and 2^12 r are split the same way; hi*hi + hi*lo +
//     lo*hi (3 passes of 32 x 32 x 16 f16 MFMA) leave a representation error
//     near 2^-22 of the terms' magnitudes, and the power-of-two scales keep
//     every decision's sign and threshold; a seeded G has float16-exact
//     entries, whose lo piece is zero: its projection runs 2 passes;
//   * the rotation accumulates each run of 8 K steps (128 input coordinates)
//     in fresh matrix-core accumulators and adds it into float32 running
//     sums: float32 accumulation over d = 1536 terms in one chain would move
//     z by about 2^-24 sqrt(d / 16) |z|, and G amplifies an error in r by
//     about sqrt(d) in p, more than the 1e-6 decision window on p.
//
// Work split of a block (8 waves, tiles of 128 coordinates x 128 keys):
// waves 0-3 multiply (wave (wm, wn): 64 x 64, 2 x 2 tiles of 32 x 32),
// waves 4-7 load and stage K steps into a ring of three LDS buffers (loads
// issued eight steps ahead in six named register slots); one block per CU
// walks a run of tiles.  The operand tiles
// of Pi and G are built once by tq_init with their rows permuted inside each
// 32-row tile so that accumulator element e of lane l is output coordinate
// 16 (l / 32) + e of the tile: a lane's 16 decisions of one bit word are
// contiguous, and one exchange with lane l ^ 32 completes the word.
// Keys are processed in chunks whose key and residual pieces fit the
// handle's scratch (at most 256 MB): prep, rotate, project per chunk.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;          // output coordinates per block tile
constexpr int kBN = 128;          // keys per block tile
// Staged operand of one K step: two planes (hi, lo pieces) of 128 rows x 16
// halves; a row's two 16-byte units are swapped in rows 4-7 of every 8
// (XOR with bit 2 of the row), and plane 1 starts 64 bytes past a multiple
// of 128 bytes.  Then the 8 lanes that share an LDS cycle hit 8 distinct
// 16-byte bank groups both when the multiplying waves read 8 consecutive
// rows of one unit and when the staging waves write 2 rows x 2 units x 2
// planes (2-way conflicts with the padded layout this replaced).
constexpr int kPlaneH = kBM * 16 + 32;  // halves per plane (4096 + 64 bytes)
constexpr int kThreads = 512;     // 4 multiplying + 4 staging waves
constexpr int kChunkSteps = 8;    // K steps per fresh accumulator (rotation)
constexpr int kStepHalves = kBM * 2 * 16;  // one K step of an operand tile: [row][piece][16]
constexpr size_t kScratchBudget = size_t(256) << 20;
constexpr int kMaxCoordTiles = 4096 / kBM;  // d <= 4096

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }

// the power of two 2^s with 2^s n in [2^13, 2^14) (1 for n = 0)
__device__ __forceinline__ float key_scale(float nk) {
  if (!(nk > 0.0f)) return 1.0f;
  int e = 0;
  (void)frexpf(nk, &e);
  return ldexpf(1.0f, 14 - e);
}

// ---------------------------------------------------------------------------
// 1. prep: for d > 256 two launches (1a then 1b), else 1b alone in its
// fused form.
// 1a. norms: one wave per key; lane l sums the squares of its elements
// 4 l + 256 i .. + 3 (float32) or 8 l + 512 i .. + 7 (bfloat16) in
// sequence, then a butterfly over the 64 lanes, all in float32.
// ---------------------------------------------------------------------------
template <int KT>
__global__ void __launch_bounds__(256)
qg_norm_kernel(const void* __restrict__ keys, int64_t nkeys, int64_t ldk, int d, int vec_ok,
               float* __restrict__ norms) {
  constexpr int kE = KT == TQ_F32 ? 4 : 8;  // elements per lane and round
  const int lane = threadIdx.x & 63;
  const int64_t key = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (key >= nkeys) return;  // (whole waves)
  float ss = 0.0f;
  for (int e0 = kE * lane; e0 < d; e0 += 64 * kE) {
    float x[kE];
    if constexpr (KT == TQ_F32) {
      const float* row = static_cast<const float*>(keys) + key * ldk;
      if (vec_ok && e0 + 4 <= d) {
        const float4 v = *reinterpret_cast<const float4*>(row + e0);
        x[0] = v.x;
        x[1] = v.y;
        x[2] = v.z;
        x[3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = e0 + e < d ? row[e0 + e] : 0.0f;
      }
    } else {
      const uint16_t* row = static_cast<const uint16_t*>(keys) + key * ldk;
      if (vec_ok && e0 + 8 <= d) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + e0);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_to_f32(uint16_t(w[e] & 0xFFFFu));
          x[2 * e + 1] = bf16_to_f32(uint16_t(w[e] >> 16));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = e0 + e < d ? bf16_to_f32(row[e0 + e]) : 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) ss = fmaf(x[e], x[e], ss);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) norms[key] = sqrtf(ss);
}

// ---------------------------------------------------------------------------
// 1b. pieces: the keys scaled by 2^s and split into two float16 pieces,
// written in the rotation's operand layout [key tile][K step][key 128]
// [piece 2][16].  A block takes one key tile and a group of 8 K steps;
// thread t takes K step t % 8 of the group for keys t / 8 + 32 p (p < 4):
// the 8 lanes of a key read 512 contiguous bytes (float32) of its row, and
// a wave writes 8 runs of 8 keys x 64 bytes.  Rows past the end of the
// keys repeat the last key (their results are never stored).
// ---------------------------------------------------------------------------
constexpr int kPieceSteps = 8;  // K steps per pieces block

// elements k0 .. k0 + 15 of a key as float32 (zero past d)
template <int KT>
__device__ __forceinline__ void load16(const void* __restrict__ keys, int64_t key, int64_t ldk, int k0, int d,
                                       int vec_ok, float (&x)[16]) {
  if constexpr (KT == TQ_F32) {
    const float* row = static_cast<const float*>(keys) + key * ldk + k0;
    if (vec_ok && k0 + 16 <= d) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = reinterpret_cast<const float4*>(row)[q];
        x[4 * q] = v.x;
        x[4 * q + 1] = v.y;
        x[4 * q + 2] = v.z;
        x[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = k0 + e < d ? row[e] : 0.0f;
    }
  } else {
    const uint16_t* row = static_cast<const uint16_t*>(keys) + key * ldk + k0;
    if (vec_ok && k0 + 16 <= d) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 v = reinterpret_cast<const uint4*>(row)[q];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * q + 2 * e] = bf16_to_f32(uint16_t(w[e] & 0xFFFFu));
          x[8 * q + 2 * e + 1] = bf16_to_f32(uint16_t(w[e] >> 16));
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = k0 + e < d ? bf16_to_f32(row[e]) : 0.0f;
    }
  }
}

// the two float16 pieces of 2^s x for K step s of key kl of key tile kt
__device__ __forceinline__ void put_pieces(uint16_t* __restrict__ kpc, int64_t kt, int ks, int s, int kl,
                                           const float (&x)[16], float scale) {
  f16x8 hi[2], lo[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float v = x[e] * scale;
    const _Float16 h = static_cast<_Float16>(v);
    hi[e >> 3][e & 7] = h;
    lo[e >> 3][e & 7] = static_cast<_Float16>(v - static_cast<float>(h));
  }
  f16x8* dst = reinterpret_cast<f16x8*>(kpc + ((kt * ks + s) * kBN + kl) * 32);
  dst[0] = hi[0];
  dst[1] = hi[1];
  dst[2] = lo[0];
  dst[3] = lo[1];
}

// FUSED (at most 16 K steps, d <= 256): one block per key tile; thread t
// takes K steps t % 8 and t % 8 + 8, and the 8 lanes of a key also form
// its norm (each lane's squares in sequence, then a butterfly over the 8
// lanes), so the keys are read once.
template <int KT, bool FUSED>
__global__ void __launch_bounds__(256)
qg_pieces_kernel(const void* __restrict__ keys, int64_t nkeys, int64_t ldk, int d, int ks, int vec_ok,
                 float* __restrict__ norms, uint16_t* __restrict__ kpc) {
  if constexpr (FUSED) {
    const int64_t kt = blockIdx.x;
    const int s0 = threadIdx.x & 7, s1 = s0 + 8;
#pragma unroll 1
    for (int j = 0; j < 4; ++j) {
      const int kl = (threadIdx.x >> 3) + 32 * j;
      const int64_t k = kt * kBN + kl;
      const int64_t key = k < nkeys ? k : nkeys - 1;
      float x0[16], x1[16];
      if (s0 < ks) {
        load16<KT>(keys, key, ldk, 16 * s0, d, vec_ok, x0);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x0[e] = 0.0f;
      }
      if (s1 < ks) {
        load16<KT>(keys, key, ldk, 16 * s1, d, vec_ok, x1);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x1[e] = 0.0f;
      }
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) ss = fmaf(x0[e], x0[e], ss);
#pragma unroll
      for (int e = 0; e < 16; ++e) ss = fmaf(x1[e], x1[e], ss);
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) ss += __shfl_xor(ss, o);
      const float nk = sqrtf(ss);
      if (s0 == 0 && k < nkeys) norms[key] = nk;
      const float scale = key_scale(nk);
      if (s0 < ks) put_pieces(kpc, kt, ks, s0, kl, x0, scale);
      if (s1 < ks) put_pieces(kpc, kt, ks, s1, kl, x1, scale);
    }
  } else {
    const int groups = (ks + kPieceSteps - 1) / kPieceSteps;
    const int64_t kt = blockIdx.x / groups;
    const int sg = int(blockIdx.x - kt * groups);
    const int s = sg * kPieceSteps + (threadIdx.x & 7);
    if (s >= ks) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kl = (threadIdx.x >> 3) + 32 * j;
      int64_t key = kt * kBN + kl;
      key = key < nkeys ? key : nkeys - 1;
      float x[16];
      load16<KT>(keys, key, ldk, 16 * s, d, vec_ok, x);
      put_pieces(kpc, kt, ks, s, kl, x, key_scale(norms[key]));
    }
  }
}


// two float16 pieces of 8 floats: hi = f16(x), lo = f16(x - hi)
__device__ __forceinline__ void split8(const float (&x)[8], f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const _Float16 h = static_cast<_Float16>(x[e]);
    hi[e] = h;
    lo[e] = static_cast<_Float16>(x[e] - static_cast<float>(h));
  }
}

// a staging thread's loads for one K step: two 16-byte chunks of the A tile
// and the B operand (rotation: 8 raw key elements; projection: two 16-byte
// chunks of the residual pieces)
struct Slot {
  uint4 a0, a1, b0, b1;
};

// halves offset of 16-byte unit u (0, 1) of row r within a plane
__device__ __forceinline__ int unit_off(int r, int u) { return 16 * r + 8 * (u ^ ((r >> 2) & 1)); }

struct Levels {
  float t[kMaxLevels];   // thresholds, ascending (L - 1 used)
  float c[kMaxLevels];   // levels, ascending
  int bits;              // log2 L
};

// ---------------------------------------------------------------------------
// Randomized Hadamard rotation (tq_init_hadamard handles, d a power of two):
// Pi = H diag(sigma) c with H the Sylvester matrix and c = float32(1/sqrt(d)),
// so z = c H (sigma * k) / n, a fast Walsh-Hadamard transform: d log2 d
// additions instead of the d^2 products of the dense rotation.  A block
// takes 4 consecutive keys, one wave each; lane l holds elements
// l M .. l M + M - 1 (M = d / 64, or one element per lane below d = 64):
// log2 M butterfly stages inside the lane, the rest across lanes by
// exchanges with lane l ^ 2^b.  Then, per element, the rotation's
// epilogue: bucketize, code bits, r = z - c[idx] as residual pieces for the
// projection, and rho^2.  The pieces go through LDS so that the block writes
// each K step of its 4 keys as one contiguous 256-byte run of the
// projection's operand layout (a wave writing its own key directly would
// scatter 64-byte pieces d / 16 steps apart).
// ---------------------------------------------------------------------------
template <int KT, int LGD>
__global__ void __launch_bounds__(256)
qg_wht_kernel(const void* __restrict__ keys, int64_t nkeys, int64_t ldk, int vec_ok,
              const float* __restrict__ sigma, float c, Levels lv, int B, int W, int code_row,
              uint32_t* __restrict__ codes, float* __restrict__ norms, uint16_t* __restrict__ rp,
              float* __restrict__ part, int nct) {
  constexpr int D = 1 << LGD;
  constexpr int LGM = LGD > 6 ? LGD - 6 : 0;
  constexpr int M = 1 << LGM;
  constexpr int DPM = D < 32 ? 32 : D;  // coordinates padded to whole code words
  constexpr int KS2 = DPM / 16;         // K steps of the projection
  constexpr int ROWH = 4 * 32 + 8;      // halves per staged K step (4 keys x 2 pieces x 16) + 16 bytes
  __shared__ __align__(16) _Float16 stage[KS2 * ROWH];
  __shared__ float lc[kMaxLevels];
  if (threadIdx.x < kMaxLevels) lc[threadIdx.x] = lv.c[threadIdx.x];

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t key0 = int64_t(blockIdx.x) * 4, key = key0 + w;
  const bool kin = key < nkeys;
  const int j0 = lane * M;
  const bool active = kin && j0 < D;
  float x[M];
  if constexpr (KT == TQ_F32) {
    const float* row = static_cast<const float*>(keys) + (kin ? key : 0) * ldk;
    if (M >= 4 && vec_ok) {
#pragma unroll
      for (int q = 0; q < M / 4; ++q) {
        const float4 v = active ? *reinterpret_cast<const float4*>(row + j0 + 4 * q) : float4{0.f, 0.f, 0.f, 0.f};
        x[4 * q] = v.x;
        x[4 * q + 1] = v.y;
        x[4 * q + 2] = v.z;
        x[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < M; ++e) x[e] = active ? row[j0 + e] : 0.0f;
    }
  } else {
    const uint16_t* row = static_cast<const uint16_t*>(keys) + (kin ? key : 0) * ldk;
    if (M >= 8 && vec_ok) {
#pragma unroll
      for (int q = 0; q < M / 8; ++q) {
        const uint4 v = active ? *reinterpret_cast<const uint4*>(row + j0 + 8 * q) : uint4{0u, 0u, 0u, 0u};
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[8 * q + 2 * t] = bf16_to_f32(uint16_t(u[t] & 0xFFFFu));
          x[8 * q + 2 * t + 1] = bf16_to_f32(uint16_t(u[t] >> 16));
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < M; ++e) x[e] = active ? bf16_to_f32(row[j0 + e]) : 0.0f;
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < M; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float nk = sqrtf(ss);
  if (M >= 4) {
#pragma unroll
    for (int q = 0; q < M / 4; ++q) {
      const float4 sg = active ? *reinterpret_cast<const float4*>(sigma + j0 + 4 * q) : float4{0.f, 0.f, 0.f, 0.f};
      x[4 * q] *= sg.x;
      x[4 * q + 1] *= sg.y;
      x[4 * q + 2] *= sg.z;
      x[4 * q + 3] *= sg.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) x[e] *= active ? sigma[j0 + e] : 0.0f;
  }
  // butterflies (a, b) -> (a + b, a - b) over each index bit: inside the
  // lane for the low log2 M bits, then across lanes
#pragma unroll
  for (int b = 0; b < LGM; ++b)
#pragma unroll
    for (int e = 0; e < M; ++e)
      if (!(e & (1 << b))) {
        const float a0 = x[e], a1 = x[e | (1 << b)];
        x[e] = a0 + a1;
        x[e | (1 << b)] = a0 - a1;
      }
#pragma unroll
  for (int b = 0; b < LGD - LGM; ++b) {
    const bool upper = (lane >> b) & 1;
#pragma unroll
    for (int e = 0; e < M; ++e) {
      const float y = __shfl_xor(x[e], 1 << b);
      x[e] = upper ? y - x[e] : x[e] + y;
    }
  }
  __syncthreads();  // lc
  const float zs = nk > 0.0f ? c / nk : 0.0f;
  float rho2 = 0.0f;
  uint32_t bits[4] = {0u, 0u, 0u, 0u};  // code bits per plane of this lane's (part of a) word
  constexpr int G = M < 8 ? M : 8;        // elements per LDS store
#pragma unroll
  for (int q = 0; q < M / G; ++q) {
    _Float16 ph[G], pl[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int e = q * G + t;
      const float z = x[e] * zs;
      // idx = #{thresholds <= z}; unused thresholds are +inf
      int idx = 0;
#pragma unroll
      for (int u = 0; u + 1 < kMaxLevels; ++u) idx += z >= lv.t[u] ? 1 : 0;
      const float r = active ? z - lc[idx] : 0.0f;
      idx = active ? idx : 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) bits[p] |= uint32_t((idx >> p) & 1) << ((j0 + e) & 31);
      rho2 = fmaf(r, r, rho2);
      const float r2 = r * 4096.0f;
      ph[t] = static_cast<_Float16>(r2);
      pl[t] = static_cast<_Float16>(r2 - static_cast<float>(ph[t]));
    }
    const int j = j0 + q * G;
    if (j < DPM) {
      _Float16* at = stage + (j >> 4) * ROWH + w * 32 + (j & 15);
      if constexpr (G == 8) {
        f16x8 vh, vl;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          vh[t] = ph[t];
          vl[t] = pl[t];
        }
        *reinterpret_cast<f16x8*>(at) = vh;
        *reinterpret_cast<f16x8*>(at + 16) = vl;
      } else {
#pragma unroll
        for (int t = 0; t < G; ++t) {
          at[t] = ph[t];
          at[16 + t] = pl[t];
        }
      }
    }
    if constexpr (M >= 32) {
      if (((q + 1) * G) % 32 == 0) {  // a whole word of this lane is done
        const int word = (j0 + q * G) >> 5;
        if (kin)
          for (int p = 0; p < B; ++p) codes[key * code_row + p * W + word] = bits[p];
#pragma unroll
        for (int p = 0; p < 4; ++p) bits[p] = 0u;
      }
    }
  }
  if constexpr (M < 32) {
    // a word spans 32 / M lanes: OR their bits together
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int o = 1; o < 32 / M; o <<= 1) bits[p] |= __shfl_xor(bits[p], o);
    if (kin && (j0 & 31) == 0 && j0 < D) {
      const int word = j0 >> 5;
      for (int p = 0; p < B; ++p) codes[key * code_row + p * W + word] = bits[p];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) rho2 += __shfl_xor(rho2, o);
  if (kin) {
    if (lane == 0) norms[key] = nk;
    if (lane < 2 * nct) part[key * 2 * nct + lane] = lane == 0 ? rho2 : 0.0f;
  }
  __syncthreads();
  // K step s of the 4 keys: 256 contiguous bytes at key tile kt, step s,
  // keys tkey0 .. tkey0 + 3 (keys past the chunk get zero pieces)
  const int64_t kt = key0 / kBN, tkey0 = key0 - kt * kBN;
  for (int i = threadIdx.x; i < KS2 * 16; i += 256) {
    const int st = i >> 4, u = i & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + st * ROWH + 8 * u);
    *reinterpret_cast<uint4*>(rp + ((kt * KS2 + st) * kBN + tkey0) * 32 + 8 * u) = v;
  }
}

// ---------------------------------------------------------------------------
// 2. / 3. the tiled products.  MODE 0: rotate + bucketize (B operand: the
// key pieces); MODE 1: project + signs (B operand: the residual pieces);
// MODE 2: MODE 1 for a G whose entries are exact in float16 (its lo piece
// is zero, so the lo x hi pass is skipped).
// ---------------------------------------------------------------------------
struct QArgs {
  const uint16_t* atiles;  // operand tiles of this matrix
  int ks;                  // K steps of this product
  const uint16_t* bsrc;    // B operand pieces [key tile][K step][key 128][piece 2][16]
  int d, dpm, nct, ks2;    // dimension, coordinates padded to 32, coordinate tiles, residual K steps
  const float* norms;      // the chunk's norms
  int64_t nkeys;           // keys in the chunk
  uint16_t* rp;            // residual pieces [key tile][step ks2][key 128][piece 2][16]
  float* part;             // rho^2 partials [key][nct][row half]
  int64_t items, tiles;    // (key tile, coordinate tile) items of the launch; key tiles
  uint32_t* codes;         // the chunk's code rows
  int code_row, B, W, hi, hi_words;
  uint32_t* signs;         // the chunk's sign rows
  float* rnorms;           // the chunk's rho
  Levels base, fine;       // level sets (fine: coordinates below hi)
};

// Work items are (key tile, coordinate tile) pairs, coordinate tile
// fastest.  Workgroups go to the 8 XCDs in turn (block b to XCD b % 8), so
// block b takes the items v, v + B, v + 2B, ... (B blocks) with
// v = (b % 8) (B / 8) + b / 8: at any time the blocks of one XCD work on a
// run of consecutive items, i.e. on all coordinate tiles of a few key
// tiles, and each key tile's operand rows are fetched into that XCD's L2
// once for all its coordinate tiles (and each coordinate tile's once for
// the few key tiles) instead of every block streaming its own key tile
// from the MALL.  Any dispatch order gives the same results.  A step is one
// K step of one item; the block's steps run back to back, so the staging
// waves load the next item's operands while the multiplying waves finish
// the current one.  LDS holds three staged steps: at iteration it the
// multiplying waves read step it + 1's fragments from LDS while the matrix
// cores work on step it, and the staging waves fill step it + 2; one barrier
// per step.
// NB: code bits of the handle (rotation; 0 for the projection)
template <int MODE, int NB>
__global__ void __launch_bounds__(kThreads, 1) qgemm_kernel(QArgs a) {
  __shared__ __align__(16) _Float16 sA[3][2 * kPlaneH];  // [buf][piece plane][row][16], swizzled
  __shared__ __align__(16) _Float16 sB[3][2 * kPlaneH];  // [buf][piece plane][key][16], swizzled
  __shared__ float lv_c[2][kMaxLevels];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kl = lane & 31, g = lane >> 5;
  const bool producer = w >= 4;
  const int wm = w & 1, wn = (w >> 1) & 1, pt = tid - 256;
  const int ks = a.ks;
  // this block's items: vb + j * gridDim.x, j < my_items
  const int64_t nb = gridDim.x;
  const int64_t vb = nb % 8 == 0 ? int64_t(blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : int64_t(blockIdx.x);
  const int64_t my_items = a.items > vb ? (a.items - vb + nb - 1) / nb : 0;
  const int64_t steps = my_items * ks;
  if (tid < kMaxLevels) {
    lv_c[0][tid] = a.base.c[tid];
    lv_c[1][tid] = a.fine.c[tid];
  }

  if (my_items == 0) return;  // (the whole block)

  if (producer) {
    // chunk c in {pt, pt + 256} of a step's 512 16-byte chunks (of either
    // operand) is (row c / 4, piece (c / 2) % 2, half c % 2)
    // The step to fetch next: item vb + f_j nb (key tile f_kt, coordinate
    // tile f_ct, advanced incrementally), K step f_s, and its operand rows.
    const int64_t kt_step = nb / a.nct;
    const int ct_step = int(nb - kt_step * a.nct);
    int64_t f_j = 0, f_kt = vb / a.nct;
    int f_s = 0, f_ct = int(vb - f_kt * a.nct);
    const uint16_t* f_a = a.atiles + int64_t(f_ct) * ks * kStepHalves;
    const uint16_t* f_b = a.bsrc + f_kt * ks * kStepHalves;
    // Every call issues its four loads: a fixed number of loads per step
    // lets the compiler wait for exactly the slot being staged, not for
    // loads issued after it.  Past the block's last step the last step is
    // loaded again (valid addresses, unused data).
    auto fetch = [&]() __attribute__((always_inline)) {
      Slot sl;
      const uint4* ap = reinterpret_cast<const uint4*>(f_a);
      const uint4* bp = reinterpret_cast<const uint4*>(f_b);
      sl.a0 = ap[pt];
      sl.a1 = ap[pt + 256];
      sl.b0 = bp[pt];
      sl.b1 = bp[pt + 256];
      if (f_s + 1 < ks) {
        ++f_s;
        f_a += kStepHalves;
        f_b += kStepHalves;
      } else if (f_j + 1 < my_items) {
        f_s = 0;
        ++f_j;
        f_kt += kt_step;
        f_ct += ct_step;
        if (f_ct >= a.nct) {
          f_ct -= a.nct;
          ++f_kt;
        }
        f_a = a.atiles + int64_t(f_ct) * ks * kStepHalves;
        f_b = a.bsrc + f_kt * ks * kStepHalves;
      }
      return sl;
    };
    auto stage = [&](int buf, const Slot& sl) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = pt + 256 * i, row = c >> 2, piece = (c >> 1) & 1, half = c & 1;
        const int off = piece * kPlaneH + unit_off(row, half);
        *reinterpret_cast<uint4*>(&sA[buf][off]) = i == 0 ? sl.a0 : sl.a1;
        *reinterpret_cast<uint4*>(&sB[buf][off]) = i == 0 ? sl.b0 : sl.b1;
      }
    };
    Slot pa0 = fetch(), pa1 = fetch(), pa2 = fetch(), pa3 = fetch(), pa4 = fetch(), pa5 = fetch();
    stage(0, pa0);
    pa0 = fetch();  // step 6
    stage(1, pa1);
    pa1 = fetch();  // step 7
    __syncthreads();
    // iteration it stages step it + 2 (slot (it + 2) % 6) into buffer
    // (it + 2) % 3, then fetches step it + 8 into that slot; it0 is a
    // multiple of 6, so the buffer is (D + 2) % 3.  Full rounds of six run
    // without conditions, then the last steps one by one.
#define TQ_QG_STEP(D, SLOT)   \
  stage(((D) + 2) % 3, SLOT); \
  SLOT = fetch();             \
  __syncthreads();
    int64_t it0 = 0;
    for (; it0 + 6 <= steps; it0 += 6) {
      TQ_QG_STEP(0, pa2)
      TQ_QG_STEP(1, pa3)
      TQ_QG_STEP(2, pa4)
      TQ_QG_STEP(3, pa5)
      TQ_QG_STEP(4, pa0)
      TQ_QG_STEP(5, pa1)
    }
    const int64_t left = steps - it0;
    if (left > 0) { TQ_QG_STEP(0, pa2) }
    if (left > 1) { TQ_QG_STEP(1, pa3) }
    if (left > 2) { TQ_QG_STEP(2, pa4) }
    if (left > 3) { TQ_QG_STEP(3, pa5) }
    if (left > 4) { TQ_QG_STEP(4, pa0) }
#undef TQ_QG_STEP
    return;
  }

  // ---- multiplying waves ----
  f32x16 acc[2][2], run[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = run[i][j] = f32x16{};
  struct Frags {
    f16x8 ah[2], al[2], bh[2], bl[2];
  };
  auto read_frags = [&](int buf) __attribute__((always_inline)) {
    Frags f;
    const _Float16* sa = sA[buf];
    const _Float16* sb = sB[buf];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int off = unit_off(64 * wm + 32 * i + kl, g);
      f.ah[i] = *reinterpret_cast<const f16x8*>(sa + off);
      f.al[i] = *reinterpret_cast<const f16x8*>(sa + kPlaneH + off);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int off = unit_off(64 * wn + 32 * j + kl, g);
      f.bh[j] = *reinterpret_cast<const f16x8*>(sb + off);
      f.bl[j] = *reinterpret_cast<const f16x8*>(sb + kPlaneH + off);
    }
    return f;
  };
  __syncthreads();
  Frags cur = read_frags(0);
  int64_t m_item = vb;
  int m_s = 0;
  // A step multiplies the fragments in use and reads the next step's into
  // load; steps run in pairs that swap the roles (no register copies).  The
  // item's epilogue follows its last step's barrier.
  int nbuf = 1;      // buffer of step it + 1
  int64_t it = 0;    // the block's step
  auto step = [&](const Frags& cur, Frags& load) __attribute__((always_inline)) {
    if (it + 1 < steps) load = read_frags(nbuf);
    nbuf = nbuf == 2 ? 0 : nbuf + 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.ah[i], cur.bh[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.ah[i], cur.bl[j], acc[i][j], 0, 0, 0);
        if constexpr (MODE != 2)  // MODE 2: A exact in one float16 piece
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.al[i], cur.bh[j], acc[i][j], 0, 0, 0);
      }
    ++m_s;
    if constexpr (MODE == 0) {
      if (m_s % kChunkSteps == 0 || m_s == ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            run[i][j] += acc[i][j];
            acc[i][j] = f32x16{};
          }
      }
    }
    ++it;
    __syncthreads();
  };
  auto epilogue = [&]() __attribute__((always_inline)) {
    {
      // the item's epilogue: element e of tile (i, j) is coordinate
      // c0(i) + 16 g + e, key 64 wn + 32 j + kl of the key tile
      const int64_t kt = m_item / a.nct;
      const int ct = int(m_item - kt * a.nct);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tkey = 64 * wn + 32 * j + kl;
        int64_t key = kt * kBN + tkey;
        const bool kin = key < a.nkeys;
        key = kin ? key : a.nkeys - 1;
        float rho2 = 0.0f;
        float inv = 0.0f;
        if constexpr (MODE == 0) {
          const float nk = a.norms[key];
          inv = nk > 0.0f ? 1.0f / (4096.0f * key_scale(nk) * nk) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int c0 = ct * kBM + 64 * wm + 32 * i;
          if (c0 >= a.dpm) continue;  // padding rows of the last coordinate tile (wave-uniform)
          const int word = c0 >> 5;
          uint32_t hw[6] = {0u, 0u, 0u, 0u, 0u, 0u};  // bit planes 0..B of the index (B + 1 <= 5), or the signs
          if constexpr (MODE == 0) {
            const f32x16 tot = run[i][j];
            const bool fine_here = c0 < a.hi;
            f16x8 rh[2], rl[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int coord = c0 + 16 * g + e;
              const bool valid = coord < a.d;
              const float z = tot[e] * inv;
              // idx = #{t_i <= z}: compares against the thresholds (kernel
              // arguments, uniform), no dependent lookups
              int idx = 0;
#pragma unroll
              for (int q = 0; q + 1 < (1 << NB); ++q) idx += z >= a.base.t[q] ? 1 : 0;
              int set = 0;
              if constexpr (NB < 4) {  // fractional widths take B <= 3
                if (fine_here) {       // the word has coordinates below hi (wave-uniform)
                  int idf = 0;
#pragma unroll
                  for (int q = 0; q + 1 < (2 << NB); ++q) idf += z >= a.fine.t[q] ? 1 : 0;
                  set = coord < a.hi ? 1 : 0;
                  idx = set ? idf : idx;
                }
              }
              const float r = valid ? z - lv_c[set][idx] : 0.0f;
              idx = valid ? idx : 0;
#pragma unroll
              for (int p = 0; p < 6; ++p) hw[p] |= uint32_t((idx >> p) & 1) << e;
              rho2 = fmaf(r, r, rho2);
              const float r2 = r * 4096.0f;
              const _Float16 h = static_cast<_Float16>(r2);
              rh[e >> 3][e & 7] = h;
              rl[e >> 3][e & 7] = static_cast<_Float16>(r2 - static_cast<float>(h));
            }
            // residual pieces: step (c0 + 16 g) / 16 of the projection's K
            const int s2 = (c0 + 16 * g) >> 4;
            _Float16* dst = reinterpret_cast<_Float16*>(a.rp) + ((kt * a.ks2 + s2) * kBN + tkey) * 32;
            *reinterpret_cast<f16x8*>(dst) = rh[0];
            *reinterpret_cast<f16x8*>(dst + 8) = rh[1];
            *reinterpret_cast<f16x8*>(dst + 16) = rl[0];
            *reinterpret_cast<f16x8*>(dst + 24) = rl[1];
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int coord = c0 + 16 * g + e;
              hw[0] |= uint32_t(coord < a.d && acc[i][j][e] > 0.0f) << e;
            }
          }
          // the other 16 decisions of the word are in lane l ^ 32
          uint32_t full[6];
#pragma unroll
          for (int p = 0; p < 6; ++p) {
            const uint32_t other = __shfl_xor(hw[p], 32);
            full[p] = g == 0 ? (hw[p] | (other << 16)) : 0u;
          }
          if (g == 0 && kin && word < a.W) {
            if constexpr (MODE == 0) {
              uint32_t* crow = a.codes + key * a.code_row;
              for (int p = 0; p < a.B; ++p) crow[p * a.W + word] = full[p];
              if (a.hi > 0 && word < a.hi_words) crow[a.B * a.W + word] = full[a.B];
            } else {
              a.signs[key * a.W + word] = full[0];
            }
          }
        }
        if constexpr (MODE == 0) {
          rho2 += __shfl_xor(rho2, 32);
          // this wave's half of the item's rows
          if (g == 0 && kin) a.part[(key * a.nct + ct) * 2 + wm] = rho2;
        } else {
          // rho from the partials (fixed order), once per key
          if (ct == 0 && wm == 0 && g == 0 && kin) {
            // all loads first (one round trip), then the sum in order
            const float* pp = a.part + key * 2 * a.nct;
            float v[2 * kMaxCoordTiles];
#pragma unroll
            for (int c = 0; c < 2 * kMaxCoordTiles; ++c) v[c] = c < 2 * a.nct ? pp[c] : 0.0f;
            float s2 = 0.0f;
#pragma unroll
            for (int c = 0; c < 2 * kMaxCoordTiles; ++c) s2 += v[c];
            a.rnorms[key] = sqrtf(s2);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = run[i][j] = f32x16{};
      m_s = 0;
      m_item += nb;
    }
  };
  Frags other;
  for (int64_t j = 0; j < my_items; ++j) {
    int s = 0;
    for (; s + 2 <= ks; s += 2) {
      step(cur, other);
      step(other, cur);
    }
    if (s < ks) {
      step(cur, other);
      cur = other;
    }
    epilogue();
  }
}

int perm_row(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

uint16_t f16_bits_h(float x) {
  const _Float16 h = static_cast<_Float16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

float f16_value_h(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }

// tiles [ct][step][row 128][piece 2][16] of scale * M[coord][k], rows
// permuted within each 32-row tile, zero past d (rows and K)
std::vector<uint16_t> operand_tiles(const std::vector<float>& m, int d, int nct, int ks, float scale) {
  std::vector<uint16_t> out(size_t(nct) * ks * kStepHalves, 0);
  for (int ct = 0; ct < nct; ++ct)
    for (int s = 0; s < ks; ++s)
      for (int r = 0; r < kBM; ++r) {
        const int coord = ct * kBM + 32 * (r >> 5) + perm_row(r & 31);
        for (int e = 0; e < 16; ++e) {
          const int k = 16 * s + e;
          const float x = coord < d && k < d ? m[size_t(coord) * d + k] * scale : 0.0f;
          const uint16_t hi = f16_bits_h(x);
          const size_t at = ((size_t(ct) * ks + s) * kBM + r) * 32 + e;
          out[at] = hi;
          out[at + 16] = f16_bits_h(x - f16_value_h(hi));
        }
      }
  return out;
}

struct Shape {
  int dpm, nct, kp, ks, ks2;
};

Shape shape_of(const tq_ctx* h) {
  Shape s;
  s.dpm = 32 * h->words;
  s.nct = (s.dpm + kBM - 1) / kBM;
  s.kp = (h->d + 15) / 16 * 16;
  s.ks = s.kp / 16;
  s.ks2 = s.dpm / 16;
  return s;
}

Levels levels_of(const Codebook& cb) {
  Levels l{};
  for (int i = 0; i < kMaxLevels; ++i) {
    l.t[i] = cb.t[i];
    l.c[i] = cb.c[i];
  }
  int b = 0;
  while ((1 << b) < cb.levels) ++b;
  l.bits = b;
  return l;
}

hipError_t launch_wht(const tq_ctx* h, const void* keys, int key_dtype, int64_t nc, int64_t ldk, bool vec_ok,
                      uint32_t* codes, float* norms, uint16_t* rp, float* part, const Shape& s, hipStream_t stream) {
  int lgd = 0;
  while ((1 << lgd) < h->d) ++lgd;
  const int code_row = h->code_bits * h->words;
  const Levels lv = levels_of(h->cb);
  const dim3 grid{static_cast<uint32_t>((nc + 3) / 4)};
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, keys, nc, ldk, vec_ok ? 1 : 0, h->d_hsigma, h->hscale,
                       lv, h->code_bits, h->words, code_row, codes, norms, rp, part, s.nct);
    return hipGetLastError();
  };
#define TQ_WHT_CASE(L) \
  case L:              \
    return key_dtype == TQ_F32 ? go(qg_wht_kernel<TQ_F32, L>) : go(qg_wht_kernel<TQ_BF16, L>);
  switch (lgd) {
    TQ_WHT_CASE(4)
    TQ_WHT_CASE(5)
    TQ_WHT_CASE(6)
    TQ_WHT_CASE(7)
    TQ_WHT_CASE(8)
    TQ_WHT_CASE(9)
    TQ_WHT_CASE(10)
    TQ_WHT_CASE(11)
    TQ_WHT_CASE(12)
    default: return hipErrorInvalidValue;
  }
#undef TQ_WHT_CASE
}

template <typename K>
hipError_t launch_pair(const QArgs& a0, K k0, const QArgs& a1, K k1, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL(k0, grid, dim3(kThreads), 0, stream, a0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k1, grid, dim3(kThreads), 0, stream, a1);
  return hipGetLastError();
}

}  // namespace

bool quantize_gemm_supported(const tq_ctx* h) {
  return h->d >= kQGemmMinD && h->d_qpi_tiles && h->d_qg_tiles && h->code_bits >= 1 && h->code_bits <= 4;
}

int build_quantize_gemm_tiles(tq_ctx* h) {
  if (h->d < kQGemmMinD) return TQ_OK;
  const Shape s = shape_of(h);
  const std::vector<uint16_t> pt = operand_tiles(h->pi, h->d, s.nct, s.ks, 4096.0f);
  const std::vector<uint16_t> gt = operand_tiles(h->g, h->d, s.nct, s.ks2, 1024.0f);
  auto up = [](uint16_t** dst, const std::vector<uint16_t>& v) {
    if (hipMalloc(reinterpret_cast<void**>(dst), v.size() * 2) != hipSuccess) {
      *dst = nullptr;
      return TQ_ENOMEM;
    }
    return hipMemcpy(*dst, v.data(), v.size() * 2, hipMemcpyHostToDevice) == hipSuccess ? TQ_OK : TQ_EHIP;
  };
  int rc = up(&h->d_qpi_tiles, pt);
  if (rc != TQ_OK) return rc;
  return up(&h->d_qg_tiles, gt);
}

void free_quantize_gemm(tq_ctx* h) {
  if (h->qscratch_used && h->qscratch_done) (void)hipEventSynchronize(h->qscratch_done);
  uint16_t** ptrs[] = {&h->d_qpi_tiles, &h->d_qg_tiles};
  for (uint16_t** p : ptrs) {
    if (*p) (void)hipFree(*p);
    *p = nullptr;
  }
  if (h->qscratch) (void)hipFree(h->qscratch);
  h->qscratch = nullptr;
  h->qscratch_bytes = 0;
  if (h->qscratch_done) (void)hipEventDestroy(h->qscratch_done);
  h->qscratch_done = nullptr;
  h->qscratch_used = false;
}

hipError_t launch_quantize_gemm(tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk, uint32_t* codes,
                                uint32_t* signs, float* norms, float* rnorms, hipStream_t stream) {
  const Shape s = shape_of(h);
  const int d = h->d;
  // the chunk of keys whose key pieces, residual pieces and rho^2 partials
  // fit the scratch
  const size_t per_key = size_t(s.kp) * 4 + size_t(s.dpm) * 4 + size_t(s.nct) * 8;
  int64_t max_chunk = int64_t(kScratchBudget / per_key) / kBN * kBN;
  max_chunk = std::max<int64_t>(max_chunk, kBN);
  const int64_t chunk = std::min<int64_t>(max_chunk, (n + kBN - 1) / kBN * kBN);
  const size_t kp_bytes = (size_t(chunk) * s.kp * 4 + 255) / 256 * 256;
  const size_t rp_bytes = (size_t(chunk) * s.dpm * 4 + 255) / 256 * 256;
  const size_t need = kp_bytes + rp_bytes + size_t(chunk) * s.nct * 8;

  std::lock_guard<std::mutex> lock(h->qscratch_mu);
  if (!h->qscratch_done && hipEventCreateWithFlags(&h->qscratch_done, hipEventDisableTiming) != hipSuccess) {
    h->qscratch_done = nullptr;
    return hipErrorOutOfMemory;
  }
  if (h->qscratch_bytes < need) {
    if (h->qscratch) {
      if (h->qscratch_used) (void)hipEventSynchronize(h->qscratch_done);
      (void)hipFree(h->qscratch);
      h->qscratch = nullptr;
      h->qscratch_bytes = 0;
      h->qscratch_used = false;
    }
    if (hipMalloc(&h->qscratch, need) != hipSuccess) {
      h->qscratch = nullptr;
      return hipErrorOutOfMemory;
    }
    h->qscratch_bytes = need;
  }
  if (h->qscratch_used && h->qscratch_stream != stream) {
    const hipError_t e = hipStreamWaitEvent(stream, h->qscratch_done, 0);
    if (e != hipSuccess) return e;
  }
  uint16_t* kpc = static_cast<uint16_t*>(h->qscratch);
  uint16_t* rp = reinterpret_cast<uint16_t*>(static_cast<char*>(h->qscratch) + kp_bytes);
  float* part = reinterpret_cast<float*>(static_cast<char*>(h->qscratch) + kp_bytes + rp_bytes);

  const int elem = key_dtype == TQ_F32 ? 4 : 2;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(keys) & 15u) == 0 && (ldk * elem) % 16 == 0;
  const int code_row = h->code_bits * h->words + (h->hi ? h->hi_words : 0);
  QArgs base{};
  base.d = d;
  base.dpm = s.dpm;
  base.nct = s.nct;
  base.ks2 = s.ks2;
  base.rp = rp;
  base.part = part;
  base.code_row = code_row;
  base.B = h->code_bits;
  base.W = h->words;
  base.hi = h->hi;
  base.hi_words = h->hi ? h->hi_words : 0;
  base.base = levels_of(h->cb);
  base.fine = h->hi ? levels_of(h->cbh) : base.base;
  hipError_t e = hipSuccess;
  for (int64_t c0 = 0; c0 < n && e == hipSuccess; c0 += chunk) {
    const int64_t nc = std::min<int64_t>(chunk, n - c0);
    const int64_t tiles = (nc + kBN - 1) / kBN;
    const void* ck = static_cast<const char*>(keys) + size_t(c0) * size_t(ldk) * elem;
    if (h->hadamard && !h->hi) {
      // rotation by the fast transform, straight into the residual pieces
      e = launch_wht(h, ck, key_dtype, nc, ldk, vec_ok, codes + c0 * code_row, norms + c0, rp, part, s, stream);
      if (e != hipSuccess) break;
      QArgs pro = base;
      pro.atiles = h->d_qg_tiles;
      pro.bsrc = rp;
      pro.ks = s.ks2;
      pro.norms = norms + c0;
      pro.nkeys = nc;
      pro.signs = signs + c0 * h->words;
      pro.rnorms = rnorms + c0;
      const int64_t items = tiles * s.nct;
      pro.items = items;
      pro.tiles = tiles;
      const dim3 grid{static_cast<uint32_t>(std::min<int64_t>(items, h->cus))};
      if (h->g_f16)
        hipLaunchKernelGGL((qgemm_kernel<2, 0>), grid, dim3(kThreads), 0, stream, pro);
      else
        hipLaunchKernelGGL((qgemm_kernel<1, 0>), grid, dim3(kThreads), 0, stream, pro);
      e = hipGetLastError();
      continue;
    }
    // norms and key pieces of the chunk
    if (s.ks <= 2 * kPieceSteps) {
      // norms and pieces in one pass
      if (key_dtype == TQ_F32)
        hipLaunchKernelGGL((qg_pieces_kernel<TQ_F32, true>), dim3(uint32_t(tiles)), dim3(256), 0, stream, ck, nc,
                           ldk, d, s.ks, vec_ok ? 1 : 0, norms + c0, kpc);
      else
        hipLaunchKernelGGL((qg_pieces_kernel<TQ_BF16, true>), dim3(uint32_t(tiles)), dim3(256), 0, stream, ck, nc,
                           ldk, d, s.ks, vec_ok ? 1 : 0, norms + c0, kpc);
    } else {
      const uint32_t nblocks = uint32_t((nc + 3) / 4);
      const uint32_t pblocks = uint32_t(tiles * ((s.ks + kPieceSteps - 1) / kPieceSteps));
      if (key_dtype == TQ_F32) {
        hipLaunchKernelGGL(qg_norm_kernel<TQ_F32>, dim3(nblocks), dim3(256), 0, stream, ck, nc, ldk, d,
                           vec_ok ? 1 : 0, norms + c0);
        hipLaunchKernelGGL((qg_pieces_kernel<TQ_F32, false>), dim3(pblocks), dim3(256), 0, stream, ck, nc, ldk, d,
                           s.ks, vec_ok ? 1 : 0, norms + c0, kpc);
      } else {
        hipLaunchKernelGGL(qg_norm_kernel<TQ_BF16>, dim3(nblocks), dim3(256), 0, stream, ck, nc, ldk, d,
                           vec_ok ? 1 : 0, norms + c0);
        hipLaunchKernelGGL((qg_pieces_kernel<TQ_BF16, false>), dim3(pblocks), dim3(256), 0, stream, ck, nc, ldk, d,
                           s.ks, vec_ok ? 1 : 0, norms + c0, kpc);
      }
    }
    e = hipGetLastError();
    if (e != hipSuccess) break;
    QArgs rot = base, pro = base;
    rot.atiles = h->d_qpi_tiles;
    rot.bsrc = kpc;
    rot.ks = s.ks;
    rot.norms = norms + c0;
    rot.nkeys = nc;
    rot.codes = codes + c0 * code_row;
    pro.atiles = h->d_qg_tiles;
    pro.bsrc = rp;
    pro.ks = s.ks2;
    pro.norms = norms + c0;
    pro.nkeys = nc;
    pro.signs = signs + c0 * h->words;
    pro.rnorms = rnorms + c0;
    // persistent blocks, one per CU, on strided items
    const int64_t items = tiles * s.nct;
    const int64_t blocks = std::min<int64_t>(items, h->cus);
    rot.items = pro.items = items;
    rot.tiles = pro.tiles = tiles;
    const dim3 grid{static_cast<uint32_t>(blocks)};
    auto project = h->g_f16 ? qgemm_kernel<2, 0> : qgemm_kernel<1, 0>;
    switch (h->code_bits) {
      case 1: e = launch_pair(rot, qgemm_kernel<0, 1>, pro, project, grid, stream); break;
      case 2: e = launch_pair(rot, qgemm_kernel<0, 2>, pro, project, grid, stream); break;
      case 3: e = launch_pair(rot, qgemm_kernel<0, 3>, pro, project, grid, stream); break;
      default: e = launch_pair(rot, qgemm_kernel<0, 4>, pro, project, grid, stream); break;
    }
  }
  if (e != hipSuccess) return e;
  e = hipEventRecord(h->qscratch_done, stream);
  if (e != hipSuccess) return e;
  h->qscratch_stream = stream;
  h->qscratch_used = true;
  return hipSuccess;
}

}  // namespace tqdev
