// Matrix-core quantizer for recursive polar-angle handles (tq_init_polar) at
// d = 128.
//
// Stages ("TurboQuant tutorial" (gitcode.csdn.net), Cartesian-to-polar and
// QJL sections; "TurboQuant deep review" (freelamp.com), recursive polar
// algorithm):
//   n = ||k||, z = Pi k / n;
//   level 1 turns each pair (z_2i, z_2i+1) into a radius and an angle in
//   [0, 2 pi); level l >= 2 turns each pair of level l - 1 radii into a
//   radius and an angle in [0, pi / 2]; an angle's index is #{t <= angle}
//   over its level's thresholds;
//   z_hat is composed back from radius 1 and the levels' cos / sin, r =
//   z - z_hat, rho = ||r||, beta = [G r > 0].
// A block of 4 waves walks tiles of 32 keys:
//   1. stage: 8 threads per key load its 128 elements (coalesced), sum the
//      squares (16-term runs, then a 3-level tree) and store the key as two
//      float16 pieces hi = f16(2^s k), lo = f16(2^s k - hi) with 2^s n in
//      [2^13, 2^14);
//   2. rotate: wave w computes output coordinates 32 w .. 32 w + 31 of the
//      tile from 2^12 Pi (two float16 pieces, in registers for the whole
//      run) and the key pieces, hi hi + hi lo + lo hi per K step of a
//      32 x 32 x 16 MFMA (bf16 keys have no lo piece: 2 passes); z = acc /
//      (2^12 2^s n) goes to LDS;
//   3. encode: 8 lanes per key, lane t owning coordinates 16 t .. 16 t + 15
//      (levels 1 - 4 inside the lane, levels 5 - 7 across the key's lanes by
//      shuffles); z_hat top-down, each coordinate's product taken in the
//      order top level first; code rows by OR-reductions over the key's
//      lanes; r to LDS as two float16 pieces of 2^12 r;
//   4. project: 2^10 G (exact in float16 for a seeded G: one piece, in
//      registers) times the residual pieces, 2 passes; the sign bits of a
//      word are completed by one exchange with lane l ^ 32.
// The operand tiles, the piece split, the pass order and the scaling are
// the general matrix-core quantizer's, so the float32 errors of z and p are
// those of that kernel, far inside the decision windows.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kTK = 32;          // keys per tile
constexpr int kPT = 256;         // threads per block (4 waves)
constexpr int kKP = kD + 8;      // halves per staged row (spreads the rows over the LDS banks)
constexpr int kZP = kD + 4;      // floats per z row
constexpr int kLevels = 7;       // log2 d

__device__ __forceinline__ float key_scale128(float nk) {
  if (!(nk > 0.0f)) return 1.0f;
  int e = 0;
  (void)frexpf(nk, &e);
  return ldexpf(1.0f, 14 - e);
}

// An angle's index #{t_i <= psi}, psi = atan2(y, x), needs no atan2.
// Levels 2 .. 7: x, y >= 0, so psi and t_i lie in [0, pi / 2], where tan
// increases: t_i <= psi iff tan t_i <= y / x.  u = y rcp(x) is within
// 2^-22 of y / x relative, which moves the angle by at most 2^-23
// sin(2 psi), inside the 1e-6 decision window.  x = 0 < y gives u = +inf
// (psi = pi / 2, above every threshold); x = y = 0 gives NaN, below every
// threshold like atan2(0, 0) = 0.
// The count over the sorted tangents splits at the middle one (u >= tt[M -
// 1] is at or above tt[0 .. M - 1]), so M - 1 more compares finish it.
template <int B>
__device__ __forceinline__ int code_quarter(float x, float y, const float* tt) {
  constexpr int M = 1 << (B - 1);
  const float u = y * __builtin_amdgcn_rcpf(x);
  const bool up = u >= tt[M - 1];
  int k = up ? M : 0;
#pragma unroll
  for (int i = 0; i + 1 < M; ++i) k += u >= (up ? tt[M + i] : tt[i]) ? 1 : 0;
  return k;
}

// Level 1: psi in [0, 2 pi).  The sign of sin(psi - t_i) is that of
// y cos t_i - x sin t_i (off only within about 2^-22 rad of t_i).  psi lies
// in [pi, 2 pi) (the upper half) when y < 0 or y = 0 > x; a threshold in
// the other half than psi is below it iff psi is in the upper half, one in
// the same half is decided by the sign (the difference of two angles of one
// half is in (-pi, pi)).  atan2(0, 0) = 0 lies below every threshold.
template <int B>
__device__ __forceinline__ int code_circle(float x, float y, const float* ct, const float* st, const int* th) {
  const bool hp = y < 0.0f || (y == 0.0f && x < 0.0f);
  int k = 0;
#pragma unroll
  for (int i = 0; i + 1 < (1 << B); ++i) {
    const bool ge = fmaf(y, ct[i], -(x * st[i])) >= 0.0f;
    k += (hp == (th[i] != 0) ? ge : hp) ? 1 : 0;
  }
  return x == 0.0f && y == 0.0f ? 0 : k;
}

// bit q of each code, placed at consecutive bits from 0
template <int N>
__device__ __forceinline__ uint32_t plane_bits(const int (&c)[N], int q) {
  uint32_t b = 0;
#pragma unroll
  for (int m = 0; m < N; ++m) b |= uint32_t((c[m] >> q) & 1) << m;
  return b;
}

template <int KT, int B>
__global__ void __launch_bounds__(kPT, 2)
quantize_polar128_kernel(const void* __restrict__ keys, int64_t n, int64_t ldk,
                         const uint16_t* __restrict__ pi_tiles, const uint16_t* __restrict__ g_tiles,
                         const float* __restrict__ ptab, uint32_t* __restrict__ codes,
                         uint32_t* __restrict__ signs, float* __restrict__ norms, float* __restrict__ rnorms) {
  __shared__ __align__(16) _Float16 sK[2][kTK][kKP];  // key pieces [piece][key][coordinate]
  __shared__ __align__(16) _Float16 sR[2][kTK][kKP];  // residual pieces
  __shared__ __align__(16) float sZ[kTK][kZP];
  __shared__ float sTab[kLevels * kPolarTab];          // per level: thresholds, cos, sin (16 each)
  __shared__ float sCT[16], sST[16];                    // level 1: cos and sin of each threshold
  __shared__ int sTH[16];                               // level 1: threshold in [pi, 2 pi)
  __shared__ float sTT[kLevels][16];                    // levels 2 .. 7: tan of each threshold
  __shared__ float sInv[kTK];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kl = lane & 31, g = lane >> 5;
  for (int i = tid; i < kLevels * kPolarTab; i += kPT) sTab[i] = ptab[i];
  if (tid < kLevels * 16) {
    const int l = tid >> 4, i = tid & 15;
    const float t = ptab[l * kPolarTab + i];  // +inf past the level's L - 1 thresholds (never used)
    if (l == 0) {
      float sn = 0.0f, cs = 0.0f;
      if (t < 8.0f) sincosf(t, &sn, &cs);
      sCT[i] = cs;
      sST[i] = sn;
      sTH[i] = t >= 3.14159265358979f ? 1 : 0;
    } else {
      sTT[l][i] = t < 8.0f ? tanf(t) : INFINITY;
    }
  }

  // operand fragments of this wave's 32 output rows: K step s, lane l holds
  // row l % 32, halves 8 (l / 32) .. + 7 of the step's 16, per piece
  f16x8 pa_h[8], pa_l[8], ga[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int64_t off = (int64_t(s) * kD + 32 * w + kl) * 32 + 8 * g;
    pa_h[s] = *reinterpret_cast<const f16x8*>(pi_tiles + off);
    pa_l[s] = *reinterpret_cast<const f16x8*>(pi_tiles + off + 16);
    ga[s] = *reinterpret_cast<const f16x8*>(g_tiles + off);
  }
  __syncthreads();

  const int64_t tiles = (n + kTK - 1) / kTK;
  const int sk = tid >> 3, st = tid & 7;        // staging: key sk, elements 16 st ..
  const int eb = lane & 7, et = lane >> 3;      // encode: key 8 w + eb, coordinates 16 et ..
  const int ek = 8 * w + eb;
  auto sh = [&](float v, int t) { return __shfl(v, eb + 8 * (t & 7)); };
  auto shi = [&](int v, int t) { return __shfl(v, eb + 8 * (t & 7)); };

  // this thread's 16 elements of its key row in tile t (rows past n repeat
  // row n - 1), as loaded: the next tile's are in flight while this one is
  // processed
  constexpr int kRaw = KT == TQ_F32 ? 4 : 2;
  struct Raw {
    uint4 v[kRaw];
  };
  auto fetch = [&](int64_t t) {
    const int64_t key = t * kTK + sk < n ? t * kTK + sk : n - 1;
    const char* row = static_cast<const char*>(keys) + (key * ldk + 16 * st) * (KT == TQ_F32 ? 4 : 2);
    Raw r;
#pragma unroll
    for (int q = 0; q < kRaw; ++q) r.v[q] = reinterpret_cast<const uint4*>(row)[q];
    return r;
  };
  Raw cur = fetch(blockIdx.x < tiles ? blockIdx.x : 0);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t k0 = tile * kTK;
    const Raw nxt = fetch(tile + gridDim.x < tiles ? tile + gridDim.x : tile);
    // ---- 1. stage ----
    {
      float x[16];
      if constexpr (KT == TQ_F32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[4 * q] = __uint_as_float(cur.v[q].x);
          x[4 * q + 1] = __uint_as_float(cur.v[q].y);
          x[4 * q + 2] = __uint_as_float(cur.v[q].z);
          x[4 * q + 3] = __uint_as_float(cur.v[q].w);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint4 v = cur.v[q];
          const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[8 * q + 2 * i] = __uint_as_float(u[i] << 16);
            x[8 * q + 2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
          }
        }
      }
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) ss = fmaf(x[e], x[e], ss);
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      const float nk = sqrtf(ss);
      const float sc = key_scale128(nk);
      if (st == 0) {
        sInv[sk] = nk > 0.0f ? 1.0f / (4096.0f * sc * nk) : 0.0f;
        if (k0 + sk < n) norms[k0 + sk] = nk;
      }
      // a bf16 element times 2^s is a float16 number unless below 2^-38 n
      // (float16 subnormals): its lo piece is zero and is not kept
      f16x8 hi[2], lo[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = x[e] * sc;
        const _Float16 h = static_cast<_Float16>(v);
        hi[e >> 3][e & 7] = h;
        if constexpr (KT == TQ_F32) lo[e >> 3][e & 7] = static_cast<_Float16>(v - static_cast<float>(h));
      }
      *reinterpret_cast<f16x8*>(&sK[0][sk][16 * st]) = hi[0];
      *reinterpret_cast<f16x8*>(&sK[0][sk][16 * st + 8]) = hi[1];
      if constexpr (KT == TQ_F32) {
        *reinterpret_cast<f16x8*>(&sK[1][sk][16 * st]) = lo[0];
        *reinterpret_cast<f16x8*>(&sK[1][sk][16 * st + 8]) = lo[1];
      }
    }
    __syncthreads();
    // ---- 2. rotate: element e of lane l is coordinate 32 w + 16 g + e of key kl ----
    {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f16x8 bh = *reinterpret_cast<const f16x8*>(&sK[0][kl][16 * s + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa_h[s], bh, acc, 0, 0, 0);
        if constexpr (KT == TQ_F32) {
          const f16x8 bl = *reinterpret_cast<const f16x8*>(&sK[1][kl][16 * s + 8 * g]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa_h[s], bl, acc, 0, 0, 0);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa_l[s], bh, acc, 0, 0, 0);
      }
      const float inv = sInv[kl];
      float* zr = &sZ[kl][32 * w + 16 * g];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(zr + 4 * q) =
            make_float4(acc[4 * q] * inv, acc[4 * q + 1] * inv, acc[4 * q + 2] * inv, acc[4 * q + 3] * inv);
    }
    __syncthreads();
    // ---- 3. encode key ek, coordinates 16 et .. 16 et + 15 ----
    {
      const int64_t key = k0 + ek;
      float z[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&sZ[ek][16 * et + 4 * q]);
        z[4 * q] = v.x;
        z[4 * q + 1] = v.y;
        z[4 * q + 2] = v.z;
        z[4 * q + 3] = v.w;
      }
      const float* T = sTab;
      // level 1: slots 8 et + m
      int c1[8];
      float r1[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float x = z[2 * m], y = z[2 * m + 1];
        c1[m] = code_circle<B>(x, y, sCT, sST, sTH);
        r1[m] = __builtin_amdgcn_sqrtf(fmaf(x, x, y * y));
      }
      // levels 2 - 4 inside the lane
      int c2[4], c3[2], c4[1];
      float r2[4], r3[2], r4;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float x = r1[2 * m], y = r1[2 * m + 1];
        c2[m] = code_quarter<B>(x, y, sTT[1]);
        r2[m] = __builtin_amdgcn_sqrtf(fmaf(x, x, y * y));
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float x = r2[2 * m], y = r2[2 * m + 1];
        c3[m] = code_quarter<B>(x, y, sTT[2]);
        r3[m] = __builtin_amdgcn_sqrtf(fmaf(x, x, y * y));
      }
      {
        const float x = r3[0], y = r3[1];
        c4[0] = code_quarter<B>(x, y, sTT[3]);
        r4 = __builtin_amdgcn_sqrtf(fmaf(x, x, y * y));
      }
      // levels 5 - 7 across the key's lanes: level l angle i sits in lane
      // et = i (lanes past the level's count compute unused values)
      float x5 = sh(r4, 2 * et), y5 = sh(r4, 2 * et + 1);
      const int c5 = code_quarter<B>(x5, y5, sTT[4]);
      const float r5 = __builtin_amdgcn_sqrtf(fmaf(x5, x5, y5 * y5));
      const float x6 = sh(r5, 2 * et), y6 = sh(r5, 2 * et + 1);
      const int c6 = code_quarter<B>(x6, y6, sTT[5]);
      const float r6 = __builtin_amdgcn_sqrtf(fmaf(x6, x6, y6 * y6));
      const float x7 = sh(r6, 0), y7 = sh(r6, 1);
      const int c7 = code_quarter<B>(x7, y7, sTT[6]);
      // z_hat: the lane's block is level-4 node et; its path from the top
      // takes the level-7 angle, level-6 angle et / 4 and level-5 angle
      // et / 2 (cos for an even child, sin for an odd one)
      const int c6b = shi(c6, et >> 2), c5b = shi(c5, et >> 1);
      auto fac = [&](int l, int code, int odd) { return T[(l - 1) * kPolarTab + (odd ? 32 : 16) + code]; };
      float v = 1.0f;
      v *= fac(7, c7, (et >> 2) & 1);
      v *= fac(6, c6b, (et >> 1) & 1);
      v *= fac(5, c5b, et & 1);
      float v3[2], v2[4], v1[8], zh[16];
#pragma unroll
      for (int i = 0; i < 2; ++i) v3[i] = v * fac(4, c4[0], i);
#pragma unroll
      for (int i = 0; i < 4; ++i) v2[i] = v3[i >> 1] * fac(3, c3[i >> 1], i & 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) v1[i] = v2[i >> 1] * fac(2, c2[i >> 1], i & 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) zh[i] = v1[i >> 1] * fac(1, c1[i >> 1], i & 1);
      // r = z - z_hat: rho^2 and the residual pieces
      float rr = 0.0f;
      f16x8 rh[2], rl[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float r = z[i] - zh[i];
        rr = fmaf(r, r, rr);
        const float r2 = r * 4096.0f;
        const _Float16 h = static_cast<_Float16>(r2);
        rh[i >> 3][i & 7] = h;
        rl[i >> 3][i & 7] = static_cast<_Float16>(r2 - static_cast<float>(h));
      }
      *reinterpret_cast<f16x8*>(&sR[0][ek][16 * et]) = rh[0];
      *reinterpret_cast<f16x8*>(&sR[0][ek][16 * et + 8]) = rh[1];
      *reinterpret_cast<f16x8*>(&sR[1][ek][16 * et]) = rl[0];
      *reinterpret_cast<f16x8*>(&sR[1][ek][16 * et + 8]) = rl[1];
      rr += __shfl_xor(rr, 8);
      rr += __shfl_xor(rr, 16);
      rr += __shfl_xor(rr, 32);
      // code words of plane q: word 0 = level-1 slots of lanes 0 - 3, word 1
      // of lanes 4 - 7, word 2 = level 2, word 3 = levels 3 (bits 0 - 15),
      // 4 (16 - 23), 5 (24 - 27), 6 (28, 29), 7 (30); bit 31 (slot d - 1) 0
      uint32_t wd[B][4];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const uint32_t b1 = plane_bits(c1, q);
        uint32_t w0 = et < 4 ? b1 << (8 * et) : 0u;
        uint32_t w1 = et >= 4 ? b1 << (8 * (et - 4)) : 0u;
        uint32_t w2 = plane_bits(c2, q) << (4 * et);
        uint32_t w3 = (plane_bits(c3, q) << (2 * et)) | (uint32_t((c4[0] >> q) & 1) << (16 + et));
        w3 |= et < 4 ? uint32_t((c5 >> q) & 1) << (24 + et) : 0u;
        w3 |= et < 2 ? uint32_t((c6 >> q) & 1) << (28 + et) : 0u;
        w3 |= et == 0 ? uint32_t((c7 >> q) & 1) << 30 : 0u;
#pragma unroll
        for (int o = 8; o <= 32; o <<= 1) {
          w0 |= __shfl_xor(w0, o);
          w1 |= __shfl_xor(w1, o);
          w2 |= __shfl_xor(w2, o);
          w3 |= __shfl_xor(w3, o);
        }
        wd[q][0] = w0;
        wd[q][1] = w1;
        wd[q][2] = w2;
        wd[q][3] = w3;
      }
      if (key < n) {
        // lane et stores word et % 4 of planes et / 4, et / 4 + 2
        uint32_t* crow = codes + key * (4 * B);
#pragma unroll
        for (int q = 0; q < B; ++q)
          if ((q & 1) == (et >> 2)) crow[4 * q + (et & 3)] = wd[q][et & 3];
        if (et == 0) rnorms[key] = sqrtf(rr);
      }
    }
    __syncthreads();
    // ---- 4. project: p = G r, element e of lane l is coordinate 32 w + 16 g + e of key kl ----
    {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f16x8 bh = *reinterpret_cast<const f16x8*>(&sR[0][kl][16 * s + 8 * g]);
        const f16x8 bl = *reinterpret_cast<const f16x8*>(&sR[1][kl][16 * s + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ga[s], bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ga[s], bl, acc, 0, 0, 0);
      }
      uint32_t hw = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) hw |= uint32_t(acc[e] > 0.0f) << e;
      const uint32_t other = __shfl_xor(hw, 32);
      if (g == 0 && k0 + kl < n) signs[(k0 + kl) * 4 + w] = hw | (other << 16);
    }
    cur = nxt;
  }
}

}  // namespace

bool quantize_polar128_supported(const tq_ctx* h, const void* keys, int key_dtype, int64_t ldk) {
  const int elem = key_dtype == TQ_F32 ? 4 : 2;
  return h->polar && h->d == kD && h->words == 4 && h->polar_levels == kLevels && h->g_f16 && h->d_qpi_tiles &&
         h->d_qg_tiles && h->d_polar_tab && h->code_bits >= 1 && h->code_bits <= 4 && !force_reference_kernels() &&
         (key_dtype == TQ_F32 || key_dtype == TQ_BF16) && (reinterpret_cast<uintptr_t>(keys) & 15u) == 0 &&
         (ldk * elem) % 16 == 0;
}

hipError_t launch_quantize_polar128(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                                    uint32_t* codes, uint32_t* signs, float* norms, float* rnorms,
                                    hipStream_t stream) {
  const int64_t tiles = (n + kTK - 1) / kTK;
  const int64_t slots = 2 * static_cast<int64_t>(h->cus);
  const dim3 grid{static_cast<uint32_t>(tiles < slots ? tiles : slots)};
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kPT), 0, stream, keys, n, ldk, h->d_qpi_tiles, h->d_qg_tiles,
                       h->d_polar_tab, codes, signs, norms, rnorms);
    return hipGetLastError();
  };
#define TQ_P128(B)                                                                                   \
  case B:                                                                                            \
    return key_dtype == TQ_F32 ? go(quantize_polar128_kernel<TQ_F32, B>) : go(quantize_polar128_kernel<TQ_BF16, B>);
  switch (h->code_bits) {
    TQ_P128(1)
    TQ_P128(2)
    TQ_P128(3)
    TQ_P128(4)
    default: return hipErrorInvalidValue;
  }
#undef TQ_P128
}

}  // namespace tqdev
