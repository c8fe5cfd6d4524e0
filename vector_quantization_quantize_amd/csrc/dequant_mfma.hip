// Matrix-core stage-1 reconstruction for d = 128 (gfx950 MFMA).
//
// "TurboQuant tutorial" (gitcode.csdn.net), polar part: the codes and the
// kept length map back to a vector, k_hat = n Pi^T c[idx].
//
// Values, not signs: an LDS table turns the packed indices of E consecutive
// coordinates (E B bits) straight into float16 pieces of 2^12 c[idx] (hi and
// lo, 22 significant bits), and with Pi scaled by 2^12 also split into two
// float16 pieces held in registers, k_hat = n 2^-24 (c_hi Pi_hi + c_hi Pi_lo
// + c_lo Pi_hi) takes three MFMA passes per K step into one float32
// accumulator.  The dropped c_lo Pi_lo term and the pieces' rounding are
// near 2^-21 relative, far under the 1e-5 bound.  E = 8 / B coordinates per
// lookup (B = 3 uses E = 4, a 4096-entry table), so a step of 8 coordinates
// takes 8 / E lookups.
//
// Two-pass form: when the level set has at most two magnitudes (B <= 2 and
// symmetric), the host finds a scale sigma that makes every sigma c[level] a
// float16 number to within 2^-19 relative.  The table then holds one piece
// per value, the products are exact, and k_hat = n (sigma 2^12)^-1
// (sigma c)(Pi_hi + Pi_lo) takes two passes; at the board power limit the
// matrix work is a large part of the kernel's energy.
//
// Work split: wave w of a 4-wave block owns output coordinates [32w, 32w+32)
// and walks tiles of 32 keys (one 32 x 32 x 16 MFMA tile: M = keys,
// N = coordinates, K = 128 input coordinates in 8 steps).  Lane l supplies,
// for key l % 32, the values of coordinates 16 s + 8 (l/32) .. +7 of step s:
// byte 2 (s % 2) + l/32 of word s/2 of each plane.  Lane l's results are
// coordinate 32w + l % 32 of keys 8(r/4) + 4(l/32) + r%4, r = 0..15, so each
// output row is written as a contiguous 128-byte segment.  Waves never wait
// on each other.
//
// Keys past the end of the last tile load key n - 1 instead (codes and
// norm), so their rows equal row n - 1 and are stored there: the same value
// twice, and no per-row branch.  Norms reach the lanes that need them
// through a per-wave LDS row (one write, four 16-byte reads; within one
// wave, so no barrier).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "score_mfma.h"
#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDqThreads = 256;
constexpr int kSteps = 8;
constexpr float kOutScale = 1.0f / (4096.0f * 4096.0f);  // undoes 2^12 on c and on Pi

// coordinates per table lookup and table geometry
template <int B, bool kTwo>
struct Lookup {
  static constexpr int E = B == 3 ? 4 : 8 / B;
  static constexpr int K = 8 / E;                  // lookups per step
  static constexpr int kEntries = 1 << (E * B);
  static constexpr int kDwords = kTwo ? E / 2 : E;  // E values, or E hi halves + E lo halves
};

// Entry layout: dwords [0, E/2) hold the hi halves of coordinates 0..E-1,
// dwords [E/2, E) the lo halves (three-pass form only).  Index bit p E + e is
// bit p of the level index of coordinate e.
template <int B, bool kTwo>
__device__ void build_table(uint32_t* tab, const Codebook& cb, const DequantTable& dqt) {
  using L = Lookup<B, kTwo>;
  for (int idx = threadIdx.x; idx < L::kEntries; idx += kDqThreads) {
    _Float16 hv[L::E], lv[L::E];
#pragma unroll
    for (int e = 0; e < L::E; ++e) {
      int level = 0;
#pragma unroll
      for (int p = 0; p < B; ++p) level |= ((idx >> (p * L::E + e)) & 1) << p;
      if constexpr (kTwo) {
        hv[e] = static_cast<_Float16>(dqt.v[level]);  // exact
        lv[e] = static_cast<_Float16>(0.0f);
      } else {
        const float x = cb.c[level] * 4096.0f;  // exact
        hv[e] = static_cast<_Float16>(x);
        lv[e] = static_cast<_Float16>(x - static_cast<float>(hv[e]));
      }
    }
#pragma unroll
    for (int k = 0; k < L::E / 2; ++k) {
      tab[idx * L::kDwords + k] =
          __builtin_bit_cast(uint16_t, hv[2 * k]) | (uint32_t(__builtin_bit_cast(uint16_t, hv[2 * k + 1])) << 16);
      if constexpr (!kTwo)
        tab[idx * L::kDwords + L::E / 2 + k] =
            __builtin_bit_cast(uint16_t, lv[2 * k]) | (uint32_t(__builtin_bit_cast(uint16_t, lv[2 * k + 1])) << 16);
    }
  }
}

// A operands (hi and lo pieces; hi only in the two-pass form) of step s for
// this lane, from the plane words holding the step's coordinates
template <int B, bool kTwo>
__device__ __forceinline__ void load_a(const uint32_t* tab, const uint32_t (&wp)[B], int shift, f16x8& ahi,
                                       f16x8& alo) {
  using L = Lookup<B, kTwo>;
  uint32_t hi[4], lo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < L::K; ++k) {
    uint32_t idx = 0;
#pragma unroll
    for (int p = 0; p < B; ++p) idx |= __builtin_amdgcn_ubfe(wp[p], shift + k * L::E, L::E) << (p * L::E);
    const uint32_t* ent = tab + idx * L::kDwords;
    if constexpr (kTwo) {
      if constexpr (L::E == 8) {
        const uint4 h = *reinterpret_cast<const uint4*>(ent);
        hi[0] = h.x; hi[1] = h.y; hi[2] = h.z; hi[3] = h.w;
      } else if constexpr (L::E == 4) {
        const uint2 h = *reinterpret_cast<const uint2*>(ent);
        hi[2 * k] = h.x; hi[2 * k + 1] = h.y;
      } else {
        hi[k] = ent[0];
      }
    } else if constexpr (L::E == 8) {
      const uint4 h = reinterpret_cast<const uint4*>(ent)[0];
      const uint4 l = reinterpret_cast<const uint4*>(ent)[1];
      hi[0] = h.x; hi[1] = h.y; hi[2] = h.z; hi[3] = h.w;
      lo[0] = l.x; lo[1] = l.y; lo[2] = l.z; lo[3] = l.w;
    } else if constexpr (L::E == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(ent);
      hi[2 * k] = v.x; hi[2 * k + 1] = v.y;
      lo[2 * k] = v.z; lo[2 * k + 1] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(ent);
      hi[k] = v.x;
      lo[k] = v.y;
    }
  }
  ahi = __builtin_bit_cast(f16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
  alo = __builtin_bit_cast(f16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
}

// kProd: the corrected reconstruction k_tilde = n (Pi^T c[idx] + rho kappa
// S^T (2 beta - 1)), S = G Pi: per step two more passes, the key's sign
// bits expanded to +-1 (exact in float16; a set bit stages as -1) against
// two float16 pieces of 2^10 S, into a second accumulator scaled per key by
// -n rho kappa 2^-10.
//
// kSplit (fractional widths, the first 64 of the 128 rotated coordinates one
// bit wider): a key's codes are the B planes (4 words each) and then one
// plane of 2 words for coordinates 0..63, 8-byte aligned per key.  Steps
// 0..3 (coordinates 0..63) look their values up in a second table of B + 1
// bits built from the finer level set; both tables hold the three-pass
// pieces of 2^12 c, so one accumulator and one output scale serve both.
template <int B, bool kTwo, bool kProd, bool kSplit = false>
__global__ void __launch_bounds__(kDqThreads, 2)
dequant_mfma128_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms, int64_t n,
                       const uint4* __restrict__ pi_frag, Codebook cb, DequantTable dqt, float* __restrict__ khat,
                       int64_t tiles, int64_t stride, int64_t bound1, int64_t bound2,
                       const uint32_t* __restrict__ signs, const float* __restrict__ rnorms,
                       const uint4* __restrict__ s_frag, float kappa, Codebook cbh) {
  static_assert(!kSplit || (!kTwo && B <= 3), "fractional widths use the three-pass tables, B + 1 <= 4");
  using L = Lookup<B, kTwo>;
  using LH = Lookup<kSplit ? B + 1 : B, false>;
  constexpr int kFineSteps = kSplit ? 4 : 0;         // steps of coordinates 0..63
  constexpr int64_t kCw = 4 * B + (kSplit ? 2 : 0);  // code words per key
  __shared__ uint4 tab4[L::kEntries * L::kDwords / 4];
  __shared__ uint4 tabh4[kSplit ? LH::kEntries * LH::kDwords / 4 : 1];
  __shared__ float4 nrow[4][8];  // per wave: the tile's 32 norms
  __shared__ float4 crow[4][kProd ? 8 : 1];  // per wave: the tile's correction factors
  uint32_t* tab = reinterpret_cast<uint32_t*>(tab4);
  uint32_t* tabh = reinterpret_cast<uint32_t*>(tabh4);
  build_table<B, kTwo>(tab, cb, dqt);
  if constexpr (kSplit) build_table<B + 1, false>(tabh, cbh, dqt);
  const float out_scale = kTwo ? dqt.out_scale : kOutScale;
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
  f16x8 bs[kProd ? kSteps : 1][2];
  if constexpr (kProd) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int q = 0; q < 2; ++q) bs[s][q] = __builtin_bit_cast(f16x8, s_frag[((w * kSteps + s) * 2 + q) * 64 + lane]);
  }
  uint32_t sgn_mask = 0x80008000u, sgn_one = 0x3C003C00u;
  asm volatile("" : "+v"(sgn_mask), "+v"(sgn_one));

  // packed codes and norm (and, for kProd, signs and rho) of this lane's key
  // (clamped to n - 1), one tile ahead; a fetch past the last tile also
  // reads key n - 1 and is unused
  auto fetch = [&](int64_t tile, uint4 (&v)[B], float& nv, uint4& sv, float& rv, uint2& xv) {
    int64_t key = tile * 32 + kl;
    key = key < n ? key : n - 1;
    if constexpr (kSplit) {
      // 8-byte aligned rows: two 8-byte loads per plane, then the extra plane
#pragma unroll
      for (int p = 0; p < B; ++p) {
        const uint2 a = *reinterpret_cast<const uint2*>(codes + key * kCw + 4 * p);
        const uint2 b = *reinterpret_cast<const uint2*>(codes + key * kCw + 4 * p + 2);
        v[p] = make_uint4(a.x, a.y, b.x, b.y);
      }
      xv = *reinterpret_cast<const uint2*>(codes + key * kCw + 4 * B);
    } else {
#pragma unroll
      for (int p = 0; p < B; ++p) v[p] = *reinterpret_cast<const uint4*>(codes + (key * B + p) * 4);
    }
    nv = norms[key];
    if constexpr (kProd) {
      sv = *reinterpret_cast<const uint4*>(signs + key * 4);
      rv = rnorms[key];
    }
  };
  // This block's tiles: tier t = blockIdx.x / stride walks the range
  // [bound_t, bound_t+1) (bound_0 = 0, bound_3 = tiles) from its offset
  // blockIdx.x % stride, in steps of stride.
  const int64_t bid = blockIdx.x;
  const int64_t tier = bid / stride;
  const int64_t tbeg = tier == 0 ? 0 : tier == 1 ? bound1 : bound2;
  const int64_t tend = tier == 0 ? bound1 : tier == 1 ? bound2 : tiles;
  uint4 nxt[B], nxt_s = make_uint4(0u, 0u, 0u, 0u);
  uint2 nxt_x = make_uint2(0u, 0u);
  float nxt_n, nxt_r = 0.0f;
  fetch(tbeg + bid % stride, nxt, nxt_n, nxt_s, nxt_r, nxt_x);
  for (int64_t tile = tbeg + bid % stride; tile < tend; tile += stride) {
    uint32_t pl[B][4];
#pragma unroll
    for (int p = 0; p < B; ++p) {
      pl[p][0] = nxt[p].x;
      pl[p][1] = nxt[p].y;
      pl[p][2] = nxt[p].z;
      pl[p][3] = nxt[p].w;
    }
    const uint32_t sw[4] = {nxt_s.x, nxt_s.y, nxt_s.z, nxt_s.w};
    const uint32_t xw[2] = {nxt_x.x, nxt_x.y};
    const float nk = nxt_n, rk = nxt_r;
    fetch(tile + stride, nxt, nxt_n, nxt_s, nxt_r, nxt_x);
    f32x16 acc = {}, acc2 = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      f16x8 ahi, alo;
      if (s < kFineSteps) {
        // coordinates 16 s .. 16 s + 15 < 64: B planes plus the extra one
        uint32_t wp[kSplit ? B + 1 : B];
#pragma unroll
        for (int p = 0; p < B; ++p) wp[p] = pl[p][s >> 1];
        if constexpr (kSplit) {
          wp[B] = xw[(s >> 1) & 1];
          load_a<kSplit ? B + 1 : B, false>(tabh, wp, 8 * (2 * (s & 1) + g), ahi, alo);
        }
      } else {
        uint32_t wp[B];
#pragma unroll
        for (int p = 0; p < B; ++p) wp[p] = pl[p][s >> 1];
        load_a<B, kTwo>(tab, wp, 8 * (2 * (s & 1) + g), ahi, alo);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bpi[s][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bpi[s][1], acc, 0, 0, 0);
      if constexpr (!kTwo) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bpi[s][0], acc, 0, 0, 0);
      if constexpr (kProd) {
        // signs of coordinates 16 s + 8 g .. + 7: byte 2 (s % 2) + g of word s / 2
        const uint4 sg = score::expand_signs(__builtin_amdgcn_ubfe(sw[s >> 1], 8 * (2 * (s & 1) + g), 8), sgn_mask,
                                             sgn_one);
        const f16x8 as = __builtin_bit_cast(f16x8, sg);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as, bs[s][0], acc2, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as, bs[s][1], acc2, 0, 0, 0);
      }
    }
    // lane holds coordinate 32w + kl of keys 8(r/4) + 4g + r%4
    reinterpret_cast<float*>(nrow[w])[kl] = nk * out_scale;  // both lane groups hold key kl
    if constexpr (kProd) reinterpret_cast<float*>(crow[w])[kl] = -nk * rk * kappa * (1.0f / 1024.0f);
    float o[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = nrow[w][2 * q + g];
      o[4 * q] = v.x * acc[4 * q];
      o[4 * q + 1] = v.y * acc[4 * q + 1];
      o[4 * q + 2] = v.z * acc[4 * q + 2];
      o[4 * q + 3] = v.w * acc[4 * q + 3];
      if constexpr (kProd) {
        const float4 c = crow[w][2 * q + g];
        o[4 * q] = fmaf(c.x, acc2[4 * q], o[4 * q]);
        o[4 * q + 1] = fmaf(c.y, acc2[4 * q + 1], o[4 * q + 1]);
        o[4 * q + 2] = fmaf(c.z, acc2[4 * q + 2], o[4 * q + 2]);
        o[4 * q + 3] = fmaf(c.w, acc2[4 * q + 3], o[4 * q + 3]);
      }
    }
    float* out = khat + tile * 32 * 128 + 32 * w + kl;
    if (tile * 32 + 32 <= n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) __builtin_nontemporal_store(o[r], out + (8 * (r >> 2) + 4 * g + (r & 3)) * 128);
    } else {
      const int last = static_cast<int>(n - 1 - tile * 32);  // rows past it repeat row n - 1
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * g + (r & 3);
        __builtin_nontemporal_store(o[r], out + (kr < last ? kr : last) * 128);
      }
    }
  }
}

// share of the tiles taken by each tier of the grid (dispatch order), by B
constexpr double kTierShare[4][3] = {
    {0.385, 0.33, 0.285}, {0.385, 0.33, 0.285}, {0.55, 0.45, 0.0}, {0.42, 0.33, 0.25}};

template <int B, bool kTwo, bool kProd = false, bool kSplit = false>
hipError_t launch_b(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n, float* khat,
                    hipStream_t stream, const uint32_t* signs = nullptr, const float* rnorms = nullptr) {
  const int64_t tiles = (n + 31) / 32;
  // One resident wave of blocks: R per CU (3 when registers and the table
  // allow, else 2).  The CU's wave arbiter favours older waves, so the
  // blocks dispatched first (one per CU in each tier of the grid) run ahead
  // of those dispatched after them; tier t of the grid takes a contiguous
  // tile range sized by kTierShare, so that the tiers finish together.  The
  // split only moves work between blocks; any dispatch order gives the same
  // results.
  constexpr int R = (B == 3 || kProd || kSplit) ? 2 : 3;
  const int64_t cus = h->cus;
  int64_t blocks, stride, bound1, bound2;
  if (tiles >= 4 * R * cus) {
    blocks = R * cus;
    stride = cus;
    const double* sh = kTierShare[B - 1];
    auto clamp = [](int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : x > hi ? hi : x; };
    // every tier's range holds at least cus tiles: one or more per block
    bound1 = clamp(static_cast<int64_t>(static_cast<double>(tiles) * sh[0] + 0.5), cus, tiles - (R - 1) * cus);
    bound2 = R == 2 ? tiles
                    : clamp(static_cast<int64_t>(static_cast<double>(tiles) * (sh[0] + sh[1]) + 0.5), bound1 + cus,
                            tiles - cus);
  } else {  // few tiles per block: equal shares, one tier
    blocks = tiles < R * cus ? tiles : R * cus;
    stride = blocks;
    bound1 = bound2 = tiles;
  }
  const auto kernel = dequant_mfma128_kernel<B, kTwo, kProd, kSplit>;
  const float kappa = float(1.2533141373155002512 / 128.0);  // sqrt(pi/2) / d
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kDqThreads), 0, stream, codes, norms, n,
                     reinterpret_cast<const uint4*>(h->d_dq_frag), h->cb, h->dqt, khat, tiles, stride, bound1,
                     bound2, signs, rnorms, reinterpret_cast<const uint4*>(h->d_ds_frag), kappa, h->cbh);
  return hipGetLastError();
}

// fractional widths with the first 64 coordinates one bit wider (B <= 3)
template <bool kProd>
hipError_t launch_split(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n, float* out,
                        hipStream_t stream, const uint32_t* signs, const float* rnorms) {
  switch (h->code_bits) {
    case 1: return launch_b<1, false, kProd, true>(h, codes, norms, n, out, stream, signs, rnorms);
    case 2: return launch_b<2, false, kProd, true>(h, codes, norms, n, out, stream, signs, rnorms);
    case 3: return launch_b<3, false, kProd, true>(h, codes, norms, n, out, stream, signs, rnorms);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Polar-angle keys (d = 128, 1..4 index bits per angle): k_hat = n Pi^T z_hat
// with z_hat composed from the angle levels ("TurboQuant tutorial",
// Cartesian-to-polar part): z_hat_j is the product, over the 7 levels, of
// the cos or sin (bit l - 1 of j) of the level's value on the path to j.
// The same matrix-core product as above with the A operand computed instead
// of looked up: lane l supplies, for key l % 32 and step s, coordinates
// 8 o .. 8 o + 7 of the octet o = 2 s + l / 32.  The lane forms the path
// products of the 8 level-4 nodes once per tile (levels 7..5), then per step
// the octet's 7 angles top down (level 4 factor, level 3, two level-2 and
// four level-1 angles), scaled by 2^12 and split into float16 hi and lo
// pieces (22 bits); three passes as in the three-pass form.  The waves
// differ only in output coordinates, so each composes a quarter of the K
// steps and shares them through LDS.
// ---------------------------------------------------------------------------
template <int B>
__global__ void __launch_bounds__(kDqThreads, 2)
dequant_polar128_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms, int64_t n,
                        const uint4* __restrict__ pi_frag, const float* __restrict__ ptab, float* __restrict__ khat,
                        int64_t tiles) {
  constexpr int L = 1 << B;
  __shared__ float2 lt[7][L];    // (cos, sin) of each level's values
  __shared__ float4 nrow[4][8];  // per wave: the tile's 32 norms
  __shared__ f16x8 sa[2][kSteps][2][64];  // [buffer][K step][piece][lane]: the A operand of a tile
  int buf = 0;
  if (threadIdx.x < 7 * L) {
    const int l = threadIdx.x / L, c = threadIdx.x % L;
    lt[l][c] = make_float2(ptab[l * kPolarTab + 16 + c], ptab[l * kPolarTab + 32 + c]);
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, kl = lane & 31, g = lane >> 5;
  f16x8 bpi[kSteps][2];
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q) bpi[s][q] = __builtin_bit_cast(f16x8, pi_frag[((w * kSteps + s) * 2 + q) * 64 + lane]);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    int64_t key = tile * 32 + kl;
    key = key < n ? key : n - 1;
    uint32_t pl[B][4];
#pragma unroll
    for (int p = 0; p < B; ++p) {
      const uint4 u = *reinterpret_cast<const uint4*>(codes + (key * B + p) * 4);
      pl[p][0] = u.x;
      pl[p][1] = u.y;
      pl[p][2] = u.z;
      pl[p][3] = u.w;
    }
    const float nk = norms[key];
    // index of the angle in slot 32 word + bit (word fixed, bit per lane)
    auto code = [&](int word, uint32_t bit) __attribute__((always_inline)) {
      uint32_t c = 0;
#pragma unroll
      for (int p = 0; p < B; ++p) c |= __builtin_amdgcn_ubfe(pl[p][word], bit, 1) << p;
      return c;
    };
    // Wave w composes K steps 2 w and 2 w + 1 of the A operand (its lanes'
    // keys, octets o = 2 s + g) into the tile's LDS buffer; after one
    // barrier every wave multiplies all 8 steps by its own Pi rows.  Path
    // products of the level-4 node s, times 2^12: level 7 (slot 126), level
    // 6 (124 + s / 4), level 5 (120 + s / 2).
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if ((s >> 1) != w) continue;  // (wave-uniform)
      const float2 c7 = lt[6][code(3, 30)];
      const float2 c6 = lt[5][code(3, 28 + (s >> 2))];
      const float2 c5 = lt[4][code(3, 24 + (s >> 1))];
      const float p6 = 4096.0f * (((s >> 2) & 1) ? c7.y : c7.x);
      const float p5 = p6 * (((s >> 1) & 1) ? c6.y : c6.x);
      const float p4 = p5 * ((s & 1) ? c5.y : c5.x);
      // octet o = 2 s + g: its level-4 parent is node s (slot 112 + s), the
      // octet itself level-3 node o (slot 96 + o), its quads level-2 nodes
      // 2 o, 2 o + 1 (slots 64 + 2 o ..), its pairs level-1 nodes 4 o .. 4 o + 3
      const float2 c4 = lt[3][code(3, 16 + s)];
      const float po = p4 * (g ? c4.y : c4.x);
      const float2 c3 = lt[2][code(3, uint32_t(2 * s) + g)];
      const float pq[2] = {po * c3.x, po * c3.y};
      float pp[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float2 c2 = lt[1][code(2, uint32_t(4 * s + h) + 2 * g)];
        pp[2 * h] = pq[h] * c2.x;
        pp[2 * h + 1] = pq[h] * c2.y;
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 c1 = lt[0][code(s >> 2, uint32_t(8 * (s & 3) + i) + 4 * g)];
        x[2 * i] = pp[i] * c1.x;
        x[2 * i + 1] = pp[i] * c1.y;
      }
      f16x8 ahi, alo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // x rounded to float32 once and opaque: otherwise the compiler folds
        // the product into the float16 conversion of hi (one rounding of the
        // exact product) while lo subtracts hi from the float32 product, and
        // at a rounding tie the two pieces disagree by a float16 ulp
        float xe = x[e];
        asm volatile("" : "+v"(xe));
        const _Float16 hv = static_cast<_Float16>(xe);
        ahi[e] = hv;
        alo[e] = static_cast<_Float16>(xe - static_cast<float>(hv));
      }
      sa[buf][s][0][lane] = ahi;
      sa[buf][s][1][lane] = alo;
    }
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const f16x8 ahi = sa[buf][s][0][lane], alo = sa[buf][s][1][lane];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bpi[s][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bpi[s][1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bpi[s][0], acc, 0, 0, 0);
    }
    // buffers alternate by tile: a wave writes one while a slower wave may
    // still read the other, and reaches the one it read before only after
    // the next tile's barrier
    buf ^= 1;
    // lane holds coordinate 32 w + kl of keys 8 (r / 4) + 4 g + r % 4
    reinterpret_cast<float*>(nrow[w])[kl] = nk * kOutScale;
    float o[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = nrow[w][2 * q + g];
      o[4 * q] = v.x * acc[4 * q];
      o[4 * q + 1] = v.y * acc[4 * q + 1];
      o[4 * q + 2] = v.z * acc[4 * q + 2];
      o[4 * q + 3] = v.w * acc[4 * q + 3];
    }
    // rows past row n - 1 of the last tile repeat it
    float* out = khat + tile * 32 * 128 + 32 * w + kl;
    const int64_t left = n - 1 - tile * 32;
    const int last = left < 31 ? static_cast<int>(left) : 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * g + (r & 3);
      __builtin_nontemporal_store(o[r], out + (kr < last ? kr : last) * 128);
    }
  }
}

}  // namespace

bool dequant_mfma128_supported(const tq_ctx* h) {
  if (h->d != 128 || !h->d_dq_frag || h->code_bits < 1) return false;
  return h->hi == 0 ? h->code_bits <= 4 : (h->hi == 64 && h->code_bits <= 3);
}

hipError_t launch_dequant_mfma128(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n,
                                  float* khat, hipStream_t stream) {
  if (h->hi == 64) return launch_split<false>(h, codes, norms, n, khat, stream, nullptr, nullptr);
  if (h->hi != 0) return hipErrorInvalidValue;
  const bool two = h->dqt.two_pass != 0;
  switch (h->code_bits) {
    case 1:
      return two ? launch_b<1, true>(h, codes, norms, n, khat, stream)
                 : launch_b<1, false>(h, codes, norms, n, khat, stream);
    case 2:
      return two ? launch_b<2, true>(h, codes, norms, n, khat, stream)
                 : launch_b<2, false>(h, codes, norms, n, khat, stream);
    case 3: return launch_b<3, false>(h, codes, norms, n, khat, stream);
    case 4: return launch_b<4, false>(h, codes, norms, n, khat, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequant_prod_mfma128(const tq_ctx* h, const uint32_t* codes, const uint32_t* signs,
                                       const float* norms, const float* rnorms, int64_t n, float* out,
                                       hipStream_t stream) {
  if (h->hi == 64) return launch_split<true>(h, codes, norms, n, out, stream, signs, rnorms);
  if (h->hi != 0) return hipErrorInvalidValue;
  const bool two = h->dqt.two_pass != 0;
  switch (h->code_bits) {
    case 1:
      return two ? launch_b<1, true, true>(h, codes, norms, n, out, stream, signs, rnorms)
                 : launch_b<1, false, true>(h, codes, norms, n, out, stream, signs, rnorms);
    case 2:
      return two ? launch_b<2, true, true>(h, codes, norms, n, out, stream, signs, rnorms)
                 : launch_b<2, false, true>(h, codes, norms, n, out, stream, signs, rnorms);
    case 3: return launch_b<3, false, true>(h, codes, norms, n, out, stream, signs, rnorms);
    case 4: return launch_b<4, false, true>(h, codes, norms, n, out, stream, signs, rnorms);
    default: return hipErrorInvalidValue;
  }
}

bool dequant_polar128_supported(const tq_ctx* h) {
  return h->polar && h->d == 128 && h->words == 4 && h->polar_levels == 7 && h->code_bits >= 1 &&
         h->code_bits <= 4 && h->d_dq_frag && h->d_polar_tab && !force_reference_kernels();
}

hipError_t launch_dequant_polar128(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n, float* khat,
                                   hipStream_t stream) {
  const int64_t tiles = (n + 31) / 32;
  const int64_t slots = 2 * static_cast<int64_t>(h->cus);
  const int64_t blocks = tiles < slots ? tiles : slots;
  const uint4* frag = reinterpret_cast<const uint4*>(h->d_dq_frag);
  switch (h->code_bits) {
    case 1: hipLaunchKernelGGL(dequant_polar128_kernel<1>, dim3(uint32_t(blocks)), dim3(kDqThreads), 0, stream, codes,
                               norms, n, frag, h->d_polar_tab, khat, tiles); break;
    case 2: hipLaunchKernelGGL(dequant_polar128_kernel<2>, dim3(uint32_t(blocks)), dim3(kDqThreads), 0, stream, codes,
                               norms, n, frag, h->d_polar_tab, khat, tiles); break;
    case 3: hipLaunchKernelGGL(dequant_polar128_kernel<3>, dim3(uint32_t(blocks)), dim3(kDqThreads), 0, stream, codes,
                               norms, n, frag, h->d_polar_tab, khat, tiles); break;
    case 4: hipLaunchKernelGGL(dequant_polar128_kernel<4>, dim3(uint32_t(blocks)), dim3(kDqThreads), 0, stream, codes,
                               norms, n, frag, h->d_polar_tab, khat, tiles); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tqdev
