// Byte lookup tables of the decode scorer: packed-key loads, the per-lane
// byte rotation of the bit planes, the stage-1 plane-subset terms and the
// table entry reads.  Shared by the scorer (logits_lut.hip) and the fused
// decode attention (attention.hip); the method and the table layout are
// described at the top of logits_lut.hip.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace tqdev {
namespace ltab {

constexpr int kDim = 128;                 // padded vector length handled here
constexpr int kTableBytes = 256 * 256;    // [x][tab][g] x 8 bytes = 64 KiB

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// stage-1 terms for B code planes, in the host's enumeration order
// (ascending plane mask, popcount 1 or 3)
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

struct Words {
  uint32_t w[4];
};

template <int B>
struct Packed {
  uint4 plane[B];
  uint4 sign;
  float n, rho;
};

template <int B>
__device__ __forceinline__ Packed<B> load_key(const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
                                              const float* __restrict__ norms, const float* __restrict__ rnorms,
                                              int64_t key) {
  // the packed cache is read once per call: non-temporal loads
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  auto nt4 = [](const uint32_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  Packed<B> k;
#pragma unroll
  for (int p = 0; p < B; ++p) k.plane[p] = nt4(codes + (key * B + p) * 4);
  k.sign = nt4(signs + key * 4);
  k.n = __builtin_nontemporal_load(norms + key);
  k.rho = __builtin_nontemporal_load(rnorms + key);
  return k;
}

// Fractional widths (code rows of 4B + 2 words: B full planes, then plane B
// of coordinates 0..63): rows are 8-byte aligned, so each plane is two
// 8-byte loads; the extra plane is returned as a plane whose bytes 8..15
// are zero.
template <int B>
__device__ __forceinline__ Packed<B + 1> load_key_hi(const uint32_t* __restrict__ codes,
                                                     const uint32_t* __restrict__ signs,
                                                     const float* __restrict__ norms,
                                                     const float* __restrict__ rnorms, int64_t key) {
  Packed<B + 1> k;
  const uint2* row = reinterpret_cast<const uint2*>(codes + key * (4 * B + 2));
#pragma unroll
  for (int p = 0; p < B; ++p) {
    const uint2 a = row[2 * p], b = row[2 * p + 1];
    k.plane[p] = make_uint4(a.x, a.y, b.x, b.y);
  }
  const uint2 x = row[2 * B];
  k.plane[B] = make_uint4(x.x, x.y, 0u, 0u);
  k.sign = *reinterpret_cast<const uint4*>(signs + key * 4);
  k.n = norms[key];
  k.rho = rnorms[key];
  return k;
}

// Byte order of a fractional-width lane: the 8 bytes of each half rotated
// by r (0..7), and the halves swapped when sw is set, so that out words 0-1
// are one half and words 2-3 the other.
__device__ __forceinline__ Words rotate_halves(const uint4& in, bool w1, uint32_t bs, bool sw) {
  const uint32_t a0 = w1 ? in.y : in.x, a1 = w1 ? in.x : in.y;  // half 0
  const uint32_t c0 = w1 ? in.w : in.z, c1 = w1 ? in.z : in.w;  // half 1
  const uint32_t h0 = __builtin_amdgcn_alignbyte(a1, a0, bs), h1 = __builtin_amdgcn_alignbyte(a0, a1, bs);
  const uint32_t h2 = __builtin_amdgcn_alignbyte(c1, c0, bs), h3 = __builtin_amdgcn_alignbyte(c0, c1, bs);
  Words out;
  out.w[0] = sw ? h2 : h0;
  out.w[1] = sw ? h3 : h1;
  out.w[2] = sw ? h0 : h2;
  out.w[3] = sw ? h1 : h3;
  return out;
}

// rotate the 16-byte plane right by r bytes: out.byte[k] = in.byte[(k + r) & 15]
__device__ __forceinline__ Words rotate(const uint4& in, bool w1, bool w2, uint32_t bs) {
  const uint32_t a0 = w1 ? in.y : in.x;
  const uint32_t a1 = w1 ? in.z : in.y;
  const uint32_t a2 = w1 ? in.w : in.z;
  const uint32_t a3 = w1 ? in.x : in.w;
  const uint32_t u0 = w2 ? a2 : a0;
  const uint32_t u1 = w2 ? a3 : a1;
  const uint32_t u2 = w2 ? a0 : a2;
  const uint32_t u3 = w2 ? a1 : a3;
  Words out;
  out.w[0] = __builtin_amdgcn_alignbyte(u1, u0, bs);
  out.w[1] = __builtin_amdgcn_alignbyte(u2, u1, bs);
  out.w[2] = __builtin_amdgcn_alignbyte(u3, u2, bs);
  out.w[3] = __builtin_amdgcn_alignbyte(u0, u3, bs);
  return out;
}

// v_perm selector: result byte0 = lane base byte (t & 1) of the LB word,
// byte1 = byte (t & 3) of the plane word, bytes 2-3 = zero
template <int t>
__device__ __forceinline__ constexpr uint32_t perm_sel() {
  return 0x0C0C0000u | ((4u + (t & 3)) << 8) | uint32_t(t & 1);
}

struct Entry {
  half2_t q01, q23;
};

template <int tab>
__device__ __forceinline__ Entry lut(const unsigned char* base, uint32_t addr) {
  // every entry address is a multiple of 8 bytes
  __builtin_assume((addr & 7u) == 0u);
  const uint2 e = *reinterpret_cast<const uint2*>(base + addr + tab * 128);
  Entry out;
  out.q01 = __builtin_bit_cast(half2_t, e.x);
  out.q23 = __builtin_bit_cast(half2_t, e.y);
  return out;
}

// Empty asm that reads and rewrites the accumulators: the additions before
// it must be issued here, so the compiler cannot defer them (keeping every
// looked-up entry alive) to the end of the unrolled key body.
template <int N>
__device__ __forceinline__ void pin(half2_t (&p)[N][2]) {
#pragma unroll
  for (int j = 0; j < N; ++j) asm volatile("" : "+v"(p[j][0]), "+v"(p[j][1])::"memory");
}

}  // namespace ltab
}  // namespace tqdev
