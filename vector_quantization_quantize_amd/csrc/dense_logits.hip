// Inner products of float32 queries with unquantized float32 or bfloat16
// keys: the uncompressed comparison for the attention-logit speedup the
// pages quote for 4-bit keys against 32-bit keys ("TurboQuant digest",
// section 3).  Layouts as for tq_logits: queries [groups][nq][d], keys
// [groups * n] rows of ldk elements, scores [groups][nq][n].
//
// dense128_kernel (d = 128, nq <= 8): HBM-bound streaming.  A key row is
// read with one 16-byte load per lane (32 lanes per float32 key, 16 per
// bfloat16 key); a wave takes U loads per lane per iteration, issued an
// iteration ahead, against NQ queries held in registers, and the U NQ
// partial sums per lane are reduced over the key's lanes by a transposing
// butterfly: at each exchange step a lane keeps half of its values and adds
// the partner's copy of that half, so U NQ values need log2(U NQ) exchanges
// of a shrinking list instead of U NQ full reductions.
// dense_any_kernel (any d, nq): one wave per key, lanes over coordinates,
// one shuffle reduction per (key, query).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

constexpr int kThreads = 256;
constexpr int kKeysPerBlock = 256;  // 4 waves x 8 iterations x 8 keys

// 16 bytes of a key row as floats: 4 float32 or 8 bfloat16 elements
__device__ __forceinline__ void widen(const uint4& u, float (&x)[4]) {
  x[0] = __uint_as_float(u.x);
  x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z);
  x[3] = __uint_as_float(u.w);
}

__device__ __forceinline__ void widen(const uint4& u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// x from a partner lane with lane bit O flipped (O <= 16; for O = 4 and 8
// the partner is the mirror within 8 or 16 lanes, which also differs in the
// lower bits: a butterfly only needs partners on the other side of bit O
// that hold the same list)
template <int O>
__device__ __forceinline__ float partner(float x) {
  const int v = __float_as_int(x);
  int r;
  if constexpr (O == 1) {
    r = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
  } else if constexpr (O == 2) {
    r = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
  } else if constexpr (O == 4) {
    r = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  } else if constexpr (O == 8) {
    r = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  } else {
    r = __builtin_amdgcn_ds_swizzle(v, 0x401F);                     // xor 16 within 32 lanes
  }
  return __int_as_float(r);
}

// transposing butterfly over the lane bits O, O/2, ..., 1 of a key's lanes:
// while the list (LEN values) is longer than one, a lane keeps the half its
// bit selects and adds the partner's copy of that half (sel records the
// kept halves, most significant first); then plain sums
template <int LEN, int O, int L>
__device__ __forceinline__ void butterfly(float (&v)[L], int kl, int& sel) {
  if constexpr (O >= 1) {
    if constexpr (LEN > 1) {
      constexpr int H = LEN / 2;
      const bool up = (kl & O) != 0;
#pragma unroll
      for (int x = 0; x < H; ++x) {
        const float keep = up ? v[H + x] : v[x];
        const float give = up ? v[x] : v[H + x];
        v[x] = keep + partner<O>(give);
      }
      sel = 2 * sel + (up ? 1 : 0);
      butterfly<H, O / 2, L>(v, kl, sel);
    } else {
      v[0] += partner<O>(v[0]);
      butterfly<1, O / 2, L>(v, kl, sel);
    }
  }
}

// EPL elements per lane per 16-byte load, KPL lanes per 128-element key,
// KPI keys per load instruction, U loads per lane per iteration (U NQ
// partial sums per lane, at most KPL of them so that the butterfly over the
// KPL lanes of a key ends with at most one value per lane)
template <typename T, int NQ>
__global__ void __launch_bounds__(kThreads)
dense128_kernel(const float* __restrict__ queries, int64_t nq, const T* __restrict__ keys, int64_t n,
                int64_t ldk, float* __restrict__ scores) {
  constexpr int EPL = 16 / sizeof(T), KPL = 128 / EPL, KPI = 64 / KPL;
  constexpr int U = KPL / NQ < 4 ? KPL / NQ : 4, L = U * NQ, KEYS = U * KPI;
  constexpr int kIters = kKeysPerBlock / 4 / KEYS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kl = lane % KPL, ks = lane / KPL;
  const int64_t grp = blockIdx.y;
  queries += grp * nq * 128;
  keys += grp * n * ldk;
  scores += grp * nq * n;
  float q[NQ][EPL];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[j][e] = j < nq ? queries[j * 128 + kl * EPL + e] : 0.0f;
  const int64_t kb0 = int64_t(blockIdx.x) * kKeysPerBlock + wave * (kKeysPerBlock / 4);
  // keys of iteration it: kb0 + it KEYS + u KPI + ks, u < U (clamped to the
  // last key; only real keys are stored)
  uint4 raw[U], nxt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int64_t t = kb0 + u * KPI + ks;
    t = t < n ? t : n - 1;
    raw[u] = *reinterpret_cast<const uint4*>(keys + t * ldk + kl * EPL);
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int64_t kb = kb0 + int64_t(it) * KEYS;
    if (it + 1 < kIters) {  // next iteration's loads go out before this one's arithmetic
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t t = kb + KEYS + u * KPI + ks;
        t = t < n ? t : n - 1;
        nxt[u] = *reinterpret_cast<const uint4*>(keys + t * ldk + kl * EPL);
      }
    }
    float v[L];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[EPL];
      widen(raw[u], x);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(q[j][e], x[e], acc);
        v[u * NQ + j] = acc;
      }
    }
    int sel = 0;
    butterfly<L, KPL / 2, L>(v, kl, sel);
    // lane holds list index sel = u NQ + j; lanes that differ only in the
    // key-lane bits below log2(KPL / L) hold copies, the lowest stores
    const int u = sel / NQ, j = sel % NQ;
    const int64_t t = kb + u * KPI + ks;
    if ((kl & (KPL / L - 1)) == 0 && j < nq && t < n) scores[j * n + t] = v[0];
#pragma unroll
    for (int w = 0; w < U; ++w) raw[w] = nxt[w];
  }
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
dense_any_kernel(const float* __restrict__ queries, int64_t nq, const T* __restrict__ keys, int64_t n, int d,
                 int64_t ldk, float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t grp = blockIdx.y;
  if (t >= n) return;
  const T* k = keys + (grp * n + t) * ldk;
  for (int64_t j = 0; j < nq; ++j) {
    const float* q = queries + (grp * nq + j) * d;
    float s = 0.0f;
    for (int c = lane; c < d; c += 64) {
      float kv;
      if constexpr (sizeof(T) == 2) {
        kv = __uint_as_float(uint32_t(k[c]) << 16);
      } else {
        kv = k[c];
      }
      s = fmaf(q[c], kv, s);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) scores[(grp * nq + j) * n + t] = s;
  }
}

template <typename T>
hipError_t launch_typed(const float* queries, int64_t groups, int64_t nq, const T* keys, int64_t n, int d,
                        int64_t ldk, float* scores, bool fast, hipStream_t s) {
  if (fast) {
    const dim3 grid(unsigned((n + kKeysPerBlock - 1) / kKeysPerBlock), unsigned(groups));
    if (nq <= 1) {
      hipLaunchKernelGGL((dense128_kernel<T, 1>), grid, dim3(kThreads), 0, s, queries, nq, keys, n, ldk, scores);
    } else if (nq <= 2) {
      hipLaunchKernelGGL((dense128_kernel<T, 2>), grid, dim3(kThreads), 0, s, queries, nq, keys, n, ldk, scores);
    } else if (nq <= 4) {
      hipLaunchKernelGGL((dense128_kernel<T, 4>), grid, dim3(kThreads), 0, s, queries, nq, keys, n, ldk, scores);
    } else {
      hipLaunchKernelGGL((dense128_kernel<T, 8>), grid, dim3(kThreads), 0, s, queries, nq, keys, n, ldk, scores);
    }
  } else {
    const dim3 grid(unsigned((n + kThreads / 64 - 1) / (kThreads / 64)), unsigned(groups));
    hipLaunchKernelGGL((dense_any_kernel<T>), grid, dim3(kThreads), 0, s, queries, nq, keys, n, d, ldk, scores);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_logits(const float* queries, int64_t groups, int64_t nq, const void* keys, int key_dtype,
                               int64_t n, int d, int64_t ldk, float* scores, hipStream_t stream) {
  const size_t esize = key_dtype == 1 ? 2 : 4;
  const bool fast = d == 128 && nq <= 8 && (reinterpret_cast<uintptr_t>(keys) & 15u) == 0 && (ldk * esize) % 16 == 0;
  if (key_dtype == 1)
    return launch_typed(queries, groups, nq, static_cast<const uint16_t*>(keys), n, d, ldk, scores, fast, stream);
  return launch_typed(queries, groups, nq, static_cast<const float*>(keys), n, d, ldk, scores, fast, stream);
}

}  // namespace tqdev
