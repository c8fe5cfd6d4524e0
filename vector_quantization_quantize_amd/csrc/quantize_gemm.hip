// General matrix-core quantizer: any d >= 16, float32 or bfloat16 keys,
// plain or fractional-width handles (gfx950 MFMA).
//
// Stages ("TurboQuant tutorial" (gitcode.csdn.net), PolarQuant and QJL
// sections; "TurboQuant digest" (juejin.cn) section 2):
//   n = ||k||, z = Pi k / n, idx_j = #{t_i <= z_j}, r = z - c[idx],
//   rho = ||r||, beta = [G r > 0], packed into bit planes.
// Both projections are dense contractions over all keys, so they run as
// tiled matrix products on the matrix cores:
//   1. norms: n = ||k|| in float32, one wave per key (tree sum of squares).
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
//     every decision's sign and threshold;
//   * the rotation accumulates each run of 8 K steps (128 input coordinates)
//     in fresh matrix-core accumulators and adds it into float32 running
//     sums: float32 accumulation over d = 1536 terms in one chain would move
//     z by about 2^-24 sqrt(d / 16) |z|, and G amplifies an error in r by
//     about sqrt(d) in p, more than the 1e-6 decision window on p.
//
// Work split of a block (8 waves, one tile of 128 coordinates x 128 keys):
// waves 0-3 multiply (wave (wm, wn): 64 x 64, 2 x 2 tiles of 32 x 32),
// waves 4-7 load and stage the next K step into LDS (double-buffered, loads
// issued six steps ahead in six named register slots).  The operand tiles
// of Pi and G are built once by tq_init with their rows permuted inside each
// 32-row tile so that accumulator element e of lane l is output coordinate
// 16 (l / 32) + e of the tile: a lane's 16 decisions of one bit word are
// contiguous, and one exchange with lane l ^ 32 completes the word.
// Keys are processed in chunks whose residual pieces fit the handle's
// scratch (at most 256 MB).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;          // output coordinates per block tile
constexpr int kBN = 128;          // keys per block tile
constexpr int kRow = 24;          // staged row: 16 halves + 8 pad (conflict-free 16-byte reads)
constexpr int kThreads = 512;     // 4 multiplying + 4 staging waves
constexpr int kChunkSteps = 8;    // K steps per fresh accumulator (rotation)
constexpr int kStepHalves = kBM * 2 * 16;  // one K step of an operand tile: [row][piece][16]
constexpr size_t kScratchBudget = size_t(256) << 20;

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }

// ---------------------------------------------------------------------------
// 1. norms
// ---------------------------------------------------------------------------
template <int KT>
__global__ void __launch_bounds__(256)
qg_norm_kernel(const void* __restrict__ keys, int64_t n, int64_t ldk, int d, float* __restrict__ norms) {
  const int64_t key = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (key >= n) return;
  float ss = 0.0f;
  if constexpr (KT == TQ_F32) {
    const float* row = static_cast<const float*>(keys) + key * ldk;
    for (int i = lane; i < d; i += 64) ss = fmaf(row[i], row[i], ss);
  } else {
    const uint16_t* row = static_cast<const uint16_t*>(keys) + key * ldk;
    for (int i = lane; i < d; i += 64) {
      const float x = bf16_to_f32(row[i]);
      ss = fmaf(x, x, ss);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) norms[key] = sqrtf(ss);
}

// the power of two 2^s with 2^s n in [2^13, 2^14) (1 for n = 0)
__device__ __forceinline__ float key_scale(float nk) {
  if (!(nk > 0.0f)) return 1.0f;
  int e = 0;
  (void)frexpf(nk, &e);
  return ldexpf(1.0f, 14 - e);
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

struct Levels {
  float t[kMaxLevels];   // thresholds, ascending (L - 1 used)
  float c[kMaxLevels];   // levels, ascending
  int bits;              // log2 L
};

// ---------------------------------------------------------------------------
// 2. / 3. the tiled products.  MODE 0: rotate + bucketize; MODE 1: project +
// signs.  KT: key type (rotation only).
// ---------------------------------------------------------------------------
struct QArgs {
  const uint16_t* atiles;  // operand tiles of this matrix
  int ks;                  // K steps of this product
  const void* keys;        // rotation: the chunk's keys
  int64_t ldk;
  int vec_ok;              // rotation: rows 16-byte aligned (whole 8-element loads allowed)
  int d, dpm, nct, ks2;    // dimension, coordinates padded to 32, coordinate tiles, residual K steps
  const float* norms;      // the chunk's norms
  int64_t nkeys;           // keys in the chunk
  uint16_t* rp;            // residual pieces [key tile][step ks2][key 128][piece 2][16]
  float* part;             // rho^2 partials [key][nct]
  uint32_t* codes;         // the chunk's code rows
  int code_row, B, W, hi, hi_words;
  uint32_t* signs;         // the chunk's sign rows
  float* rnorms;           // the chunk's rho
  Levels base, fine;       // level sets (fine: coordinates below hi)
};

template <int MODE, int KT>
__global__ void __launch_bounds__(kThreads, 1) qgemm_kernel(QArgs a) {
  __shared__ __align__(16) _Float16 sA[2][2 * kBM * kRow];  // [buf][piece][row][kRow]
  __shared__ __align__(16) _Float16 sB[2][2 * kBN * kRow];  // [buf][piece][key][kRow]
  __shared__ float red[2][kBN];                               // rho^2 of each multiplying row half
  __shared__ float lv_t[2][kMaxLevels], lv_c[2][kMaxLevels];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kl = lane & 31, g = lane >> 5;
  const bool producer = w >= 4;
  const int wm = w & 1, wn = (w >> 1) & 1, pt = tid - 256;
  const int64_t kt = blockIdx.x;
  const int ct = blockIdx.y;
  const int ks = a.ks;
  if (tid < kMaxLevels) {
    lv_t[0][tid] = a.base.t[tid];
    lv_c[0][tid] = a.base.c[tid];
    lv_t[1][tid] = a.fine.t[tid];
    lv_c[1][tid] = a.fine.c[tid];
  }

  const uint16_t* atile = a.atiles + int64_t(ct) * ks * kStepHalves;
  const uint16_t* btile = a.rp + kt * int64_t(a.ks2) * kStepHalves;  // projection's B operand

  // ---- staging role ----
  // A (and the projection's B): chunk c in {pt, pt + 256} of a step's 512
  // 16-byte chunks is (row c / 4, piece (c / 2) % 2, half c % 2).
  // The rotation's B: thread pt takes key pt % 128, elements 8 (pt / 128)
  // .. + 7 of the step.
  const int skey = pt & (kBN - 1), sh8 = pt >> 7;
  int64_t gkey = kt * kBN + skey;
  gkey = gkey < a.nkeys ? gkey : a.nkeys - 1;
  float kscale = 1.0f;
  if (MODE == 0 && producer) kscale = key_scale(a.norms[gkey]);
  int f_s = 0;  // next step to fetch
  auto fetch = [&]() __attribute__((always_inline)) {
    const int s = f_s < ks ? f_s : ks - 1;  // past the last step: a valid address, unused data
    ++f_s;
    Slot sl;
    const uint4* ap = reinterpret_cast<const uint4*>(atile + int64_t(s) * kStepHalves);
    sl.a0 = ap[pt];
    sl.a1 = ap[pt + 256];
    if constexpr (MODE == 1) {
      const uint4* bp = reinterpret_cast<const uint4*>(btile + int64_t(s) * kStepHalves);
      sl.b0 = bp[pt];
      sl.b1 = bp[pt + 256];
    } else {
      const int k0 = 16 * s + 8 * sh8;
      if constexpr (KT == TQ_F32) {
        const float* row = static_cast<const float*>(a.keys) + gkey * a.ldk;
        if (a.vec_ok && k0 + 8 <= a.d) {
          sl.b0 = *reinterpret_cast<const uint4*>(row + k0);
          sl.b1 = *reinterpret_cast<const uint4*>(row + k0 + 4);
        } else {
          uint32_t v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = k0 + e < a.d ? __float_as_uint(row[k0 + e]) : 0u;
          sl.b0 = uint4{v[0], v[1], v[2], v[3]};
          sl.b1 = uint4{v[4], v[5], v[6], v[7]};
        }
      } else {
        const uint16_t* row = static_cast<const uint16_t*>(a.keys) + gkey * a.ldk;
        if (a.vec_ok && k0 + 8 <= a.d) {
          sl.b0 = *reinterpret_cast<const uint4*>(row + k0);
        } else {
          uint32_t v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = k0 + 2 * e < a.d ? row[k0 + 2 * e] : 0u;
            const uint32_t hi = k0 + 2 * e + 1 < a.d ? row[k0 + 2 * e + 1] : 0u;
            v[e] = lo | (hi << 16);
          }
          sl.b0 = uint4{v[0], v[1], v[2], v[3]};
        }
        sl.b1 = uint4{0u, 0u, 0u, 0u};
      }
    }
    return sl;
  };
  auto stage = [&](int buf, const Slot& sl) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = pt + 256 * i, row = c >> 2, piece = (c >> 1) & 1, half = c & 1;
      const int off = piece * kBM * kRow + row * kRow + 8 * half;
      *reinterpret_cast<uint4*>(&sA[buf][off]) = i == 0 ? sl.a0 : sl.a1;
      if constexpr (MODE == 1) *reinterpret_cast<uint4*>(&sB[buf][off]) = i == 0 ? sl.b0 : sl.b1;
    }
    if constexpr (MODE == 0) {
      float x[8];
      if constexpr (KT == TQ_F32) {
        const uint32_t v[8] = {sl.b0.x, sl.b0.y, sl.b0.z, sl.b0.w, sl.b1.x, sl.b1.y, sl.b1.z, sl.b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(v[e]) * kscale;
      } else {
        const uint32_t v[4] = {sl.b0.x, sl.b0.y, sl.b0.z, sl.b0.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_to_f32(uint16_t(v[e] & 0xFFFFu)) * kscale;
          x[2 * e + 1] = bf16_to_f32(uint16_t(v[e] >> 16)) * kscale;
        }
      }
      f16x8 hi, lo;
      split8(x, hi, lo);
      const int off = skey * kRow + 8 * sh8;
      *reinterpret_cast<f16x8*>(&sB[buf][off]) = hi;
      *reinterpret_cast<f16x8*>(&sB[buf][kBN * kRow + off]) = lo;
    }
  };

  // ---- multiplying role ----
  f32x16 acc[2][2], run[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = run[i][j] = f32x16{};

  if (producer) {
    Slot pa0 = fetch(), pa1 = fetch(), pa2 = fetch(), pa3 = fetch(), pa4 = fetch(), pa5 = fetch();
    stage(0, pa0);
    pa0 = fetch();
    __syncthreads();
    // iteration it stages step it + 1 (slot (it + 1) % 6) into buffer
    // (it + 1) % 2, then fetches step it + 7 into that slot
#define TQ_QG_STEP(D, PAR, SLOT) \
  if (it0 + (D) < ks) {          \
    stage(PAR, SLOT);            \
    SLOT = fetch();              \
    __syncthreads();             \
  }
    for (int it0 = 0; it0 < ks; it0 += 6) {
      TQ_QG_STEP(0, 1, pa1)
      TQ_QG_STEP(1, 0, pa2)
      TQ_QG_STEP(2, 1, pa3)
      TQ_QG_STEP(3, 0, pa4)
      TQ_QG_STEP(4, 1, pa5)
      TQ_QG_STEP(5, 0, pa0)
    }
#undef TQ_QG_STEP
  } else {
    __syncthreads();
    for (int it = 0; it < ks; ++it) {
      const _Float16* sa = sA[it & 1];
      const _Float16* sb = sB[it & 1];
      f16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int off = (64 * wm + 32 * i + kl) * kRow + 8 * g;
        ah[i] = *reinterpret_cast<const f16x8*>(sa + off);
        al[i] = *reinterpret_cast<const f16x8*>(sa + kBM * kRow + off);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int off = (64 * wn + 32 * j + kl) * kRow + 8 * g;
        bh[j] = *reinterpret_cast<const f16x8*>(sb + off);
        bl[j] = *reinterpret_cast<const f16x8*>(sb + kBN * kRow + off);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bh[j], acc[i][j], 0, 0, 0);
        }
      if constexpr (MODE == 0) {
        if ((it + 1) % kChunkSteps == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              run[i][j] += acc[i][j];
              acc[i][j] = f32x16{};
            }
        }
      }
      __syncthreads();
    }
  }

  // ---- epilogue (multiplying waves; every thread meets the barriers) ----
  // element e of tile (i, j): coordinate c0(i) + 16 g + e, key 64 wn + 32 j + kl
  if (!producer) {
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
          const f32x16 tot = run[i][j] + acc[i][j];
          f16x8 rh[2], rl[2];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int coord = c0 + 16 * g + e;
            const bool valid = coord < a.d;
            const int set = coord < a.hi ? 1 : 0;
            const int bits = set ? a.fine.bits : a.base.bits;
            const float z = tot[e] * inv;
            int idx = 0;
            for (int st = (1 << bits) >> 1; st > 0; st >>= 1) idx += z >= lv_t[set][idx + st - 1] ? st : 0;
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
        if (g == 0) red[wm][tkey] = rho2;
      }
    }
  }
  if constexpr (MODE == 0) {
    __syncthreads();
    if (tid < kBN) {
      const int64_t key = kt * kBN + tid;
      if (key < a.nkeys) a.part[key * a.nct + ct] = red[0][tid] + red[1][tid];
    }
  } else {
    if (ct == 0 && tid < kBN) {
      const int64_t key = kt * kBN + tid;
      if (key < a.nkeys) {
        float s = 0.0f;
        for (int c = 0; c < a.nct; ++c) s += a.part[key * a.nct + c];
        a.rnorms[key] = sqrtf(s);
      }
    }
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
  // norms of every key
  {
    const int64_t blocks = (n + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (key_dtype == TQ_F32)
      hipLaunchKernelGGL(qg_norm_kernel<TQ_F32>, dim3(uint32_t(blocks)), dim3(256), 0, stream, keys, n, ldk, d, norms);
    else
      hipLaunchKernelGGL(qg_norm_kernel<TQ_BF16>, dim3(uint32_t(blocks)), dim3(256), 0, stream, keys, n, ldk, d, norms);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the chunk of keys whose residual pieces and partials fit the scratch
  const size_t per_key = size_t(s.dpm) * 4 + size_t(s.nct) * 4;
  int64_t max_chunk = int64_t(kScratchBudget / per_key) / kBN * kBN;
  max_chunk = std::max<int64_t>(max_chunk, kBN);
  const int64_t chunk = std::min<int64_t>(max_chunk, (n + kBN - 1) / kBN * kBN);
  const size_t rp_bytes = (size_t(chunk) * s.dpm * 4 + 255) / 256 * 256;
  const size_t need = rp_bytes + size_t(chunk) * s.nct * 4;

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
  uint16_t* rp = static_cast<uint16_t*>(h->qscratch);
  float* part = reinterpret_cast<float*>(static_cast<char*>(h->qscratch) + rp_bytes);

  const int elem = key_dtype == TQ_F32 ? 4 : 2;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(keys) & 15u) == 0 && (ldk * elem) % 16 == 0;
  const int code_row = h->code_bits * h->words + (h->hi ? h->hi_words : 0);
  QArgs base{};
  base.ldk = ldk;
  base.vec_ok = vec_ok ? 1 : 0;
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
    QArgs rot = base, pro = base;
    rot.atiles = h->d_qpi_tiles;
    rot.ks = s.ks;
    rot.keys = static_cast<const char*>(keys) + size_t(c0) * size_t(ldk) * elem;
    rot.norms = norms + c0;
    rot.nkeys = nc;
    rot.codes = codes + c0 * code_row;
    pro.atiles = h->d_qg_tiles;
    pro.ks = s.ks2;
    pro.norms = norms + c0;
    pro.nkeys = nc;
    pro.signs = signs + c0 * h->words;
    pro.rnorms = rnorms + c0;
    const dim3 grid(uint32_t(tiles), uint32_t(s.nct));
    if (key_dtype == TQ_F32)
      e = launch_pair(rot, qgemm_kernel<0, TQ_F32>, pro, qgemm_kernel<1, TQ_F32>, grid, stream);
    else
      e = launch_pair(rot, qgemm_kernel<0, TQ_BF16>, pro, qgemm_kernel<1, TQ_F32>, grid, stream);
  }
  if (e != hipSuccess) return e;
  e = hipEventRecord(h->qscratch_done, stream);
  if (e != hipSuccess) return e;
  h->qscratch_stream = stream;
  h->qscratch_used = true;
  return hipSuccess;
}

}  // namespace tqdev
