// Matrix-core stage-1 reconstruction for d = 128 (gfx950 MFMA).
//
// "TurboQuant tutorial" (gitcode.csdn.net), polar part: the codes and the
// kept length map back to a vector, k_hat = n Pi^T c[idx].
//
// A symmetric level set is an odd multilinear function of the plane signs,
// c[idx] = sum_S alpha_S prod_{p in S} s_p (odd-size plane subsets S), so
//     k_hat = n sum_S alpha_S (s_S^T Pi),   s_S in {-1, +1}^d,
// and every s_S^T Pi is a product with a +-1 matrix: exact in float16.  Pi
// scaled by 2^12 is split into two float16 pieces (22 bits) held in
// registers; each term takes 2 MFMA passes per K step into its own float32
// accumulator, and the epilogue forms n * sum_S alpha_S acc_S / 2^12.
//
// Work split: wave w of a 4-wave block owns output coordinates [32w, 32w+32)
// and walks tiles of 32 keys (one 32 x 32 x 16 MFMA tile: M = keys,
// N = coordinates, K = 128 input coordinates in 8 steps).  Lane l supplies,
// for key l % 32, the signs of coordinates 16 s + 8 (l/32) .. +7 of step s:
// one byte of a term word, expanded to 8 float16 values +-1 through a
// 256-entry LDS table.  Lane l's results are coordinate 32w + l % 32 of keys
// 8(r/4) + 4(l/32) + r%4, r = 0..15, so each output row is written as a
// contiguous 128-byte segment.  Waves never wait on each other.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDqThreads = 256;
constexpr int kSteps = 8;
constexpr float kPiScaleInv = 1.0f / 4096.0f;

template <int B>
struct Terms;
template <>
struct Terms<1> {
  static constexpr int count = 1;
  static constexpr uint32_t mask[1] = {1};
};
template <>
struct Terms<2> {
  static constexpr int count = 2;
  static constexpr uint32_t mask[2] = {1, 2};
};
template <>
struct Terms<3> {
  static constexpr int count = 4;
  static constexpr uint32_t mask[4] = {1, 2, 4, 7};
};
template <>
struct Terms<4> {
  static constexpr int count = 8;
  static constexpr uint32_t mask[8] = {1, 2, 4, 7, 8, 11, 13, 14};
};

template <int B>
__global__ void __launch_bounds__(kDqThreads, 2)
dequant_mfma128_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms, int64_t n,
                       const uint4* __restrict__ pi_frag, PlaneExpansion pe, float* __restrict__ khat,
                       int64_t tiles) {
  using TT = Terms<B>;
  constexpr int NT = TT::count;
  // byte -> 8 float16 values (bit e set -> +1, clear -> -1)
  __shared__ uint4 spread[256];
  {
    const uint32_t x = threadIdx.x;  // 256 threads, one entry each
    uint32_t d[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = ((x >> (2 * k)) & 1u) ? 0x3C00u : 0xBC00u;
      const uint32_t hi = ((x >> (2 * k + 1)) & 1u) ? 0x3C00u : 0xBC00u;
      d[k] = lo | (hi << 16);
    }
    spread[x] = make_uint4(d[0], d[1], d[2], d[3]);
  }
  __syncthreads();

  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kl = lane & 31;
  const int g = lane >> 5;
  f16x8 bpi[kSteps][2];
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q) bpi[s][q] = __builtin_bit_cast(f16x8, pi_frag[((w * kSteps + s) * 2 + q) * 64 + lane]);
  float alpha[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) alpha[j] = pe.alpha[j] * kPiScaleInv;

  // packed codes and norm of this lane's key, one tile ahead
  auto fetch = [&](int64_t tile, uint4 (&v)[B], float& nv) {
    const int64_t key = tile * 32 + kl;
    const bool ok = tile < tiles && key < n;
#pragma unroll
    for (int p = 0; p < B; ++p)
      v[p] = ok ? *reinterpret_cast<const uint4*>(codes + (key * B + p) * 4) : make_uint4(0u, 0u, 0u, 0u);
    nv = ok ? norms[key] : 0.0f;
  };
  uint4 nxt[B];
  float nxt_n;
  fetch(blockIdx.x, nxt, nxt_n);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    uint32_t pl[B][4];
#pragma unroll
    for (int p = 0; p < B; ++p) {
      pl[p][0] = nxt[p].x;
      pl[p][1] = nxt[p].y;
      pl[p][2] = nxt[p].z;
      pl[p][3] = nxt[p].w;
    }
    const float nk = nxt_n;
    fetch(tile + gridDim.x, nxt, nxt_n);
    f32x16 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x16{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int shift = 8 * (2 * (s & 1) + g);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        uint32_t word = 0;
#pragma unroll
        for (int p = 0; p < B; ++p)
          if (TT::mask[j] & (1u << p)) word ^= pl[p][s >> 1];
        const f16x8 a = __builtin_bit_cast(f16x8, spread[(word >> shift) & 0xFFu]);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bpi[s][1], acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bpi[s][0], acc[j], 0, 0, 0);
      }
    }
    // lane holds coordinate 32w + kl of keys 8(r/4) + 4g + r%4
    float* out = khat + tile * 32 * 128 + 32 * w + kl;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * g + (r & 3);
      const float nr = __shfl(nk, kr);
      float v = 0.0f;
#pragma unroll
      for (int j = 0; j < NT; ++j) v = fmaf(alpha[j], acc[j][r], v);
      if (tile * 32 + kr < n) __builtin_nontemporal_store(nr * v, out + kr * 128);
    }
  }
}

template <int B>
hipError_t launch_b(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n, float* khat,
                    hipStream_t stream) {
  const int64_t tiles = (n + 31) / 32;
  const int64_t blocks = tiles < 1024 ? tiles : 1024;
  hipLaunchKernelGGL(dequant_mfma128_kernel<B>, dim3(static_cast<uint32_t>(blocks)), dim3(kDqThreads), 0, stream,
                     codes, norms, n, reinterpret_cast<const uint4*>(h->d_dq_frag), h->planes, khat, tiles);
  return hipGetLastError();
}

}  // namespace

bool dequant_mfma128_supported(const tq_ctx* h) {
  return h->d == 128 && h->d_dq_frag && h->code_bits >= 1 && h->code_bits <= 4;
}

hipError_t launch_dequant_mfma128(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n,
                                  float* khat, hipStream_t stream) {
  switch (h->code_bits) {
    case 1: return launch_b<1>(h, codes, norms, n, khat, stream);
    case 2: return launch_b<2>(h, codes, norms, n, khat, stream);
    case 3: return launch_b<3>(h, codes, norms, n, khat, stream);
    case 4: return launch_b<4>(h, codes, norms, n, khat, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqdev
