// Decode scorer for polar-angle keys at d = 128 (one or two index bits per
// angle).
//
// A polar key stores a radius of 1 and d - 1 angles of a recursive polar
// transform of z = Pi u ("TurboQuant tutorial" (gitcode.csdn.net),
// Cartesian-to-polar part; "TurboQuant deep review" (freelamp.com),
// recursive polar algorithm): level 1 turns coordinate pairs into an angle
// each, level l >= 2 pairs of level l - 1 radii, seven levels at d = 128.
// The composed vector z_hat has z_hat_j = the product, over the levels, of
// the cos or the sin of the level's angle on the path down to coordinate j
// (bit l - 1 of j picks sin).  The score against a query with v = Pi q and
// w = S q is n (<v, z_hat> + rho sqrt(pi/2)/d <w, 2 beta - 1>).
//
// <v, z_hat> factors along the tree: a node's value is cos(phi) times its
// first child's value plus sin(phi) times its second's, the leaves are v.
// Per (group, 4 queries), a block tabulates the value of each 4-coordinate
// subtree (two level-1 angles and their level-2 parent: 3 B index bits, 64
// entries for B = 2) for the 4 queries in float32, and the sign term per
// byte of the sign word (256 entries per byte position, the 4 queries in
// float32).  Per key, one lane: 32 subtree lookups, the 31 upper nodes of
// the tree in float32 (cos and sin of each node's level value from a small
// table), and 16 sign lookups.  Byte-table scoring of the scalar codes
// follows the same plan (logits_lut.hip); here the upper tree levels are
// products, not sums, so only the bottom two levels go into the tables.
//
// Slots: the angles of level l are slots 128 - 2^(8-l) .. of the key's bit
// planes (level 1: 0..63, level 2: 64..95, ..., level 7: 126); plane p holds
// bit p of each slot's index.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

constexpr int kPThreads = 1024;  // 16 waves: one block per CU
constexpr int kPWaves = kPThreads / 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// offset of level l's first slot at d = 128
__host__ __device__ constexpr int slot0(int l) { return 128 - (128 >> (l - 1)); }

// index bits of slot s (compile-time s) from the B planes
template <int B>
__device__ __forceinline__ uint32_t code_of(const uint32_t (&pl)[B][4], int s) {
  uint32_t c = 0;
#pragma unroll
  for (int p = 0; p < B; ++p) c |= ((pl[p][s >> 5] >> (s & 31)) & 1u) << p;
  return c;
}

// table index of 4-coordinate subtree k: plane p contributes its bits of
// slots 2k, 2k + 1 (the two level-1 angles) at 2p, 2p + 1 and its bit of
// slot 64 + k (the level-2 angle) at 2B + p
template <int B>
__device__ __forceinline__ uint32_t quad_index(const uint32_t (&pl)[B][4], int k) {
  uint32_t x = 0;
#pragma unroll
  for (int p = 0; p < B; ++p) {
    x |= __builtin_amdgcn_ubfe(pl[p][(2 * k) >> 5], (2 * k) & 31, 2) << (2 * p);
    x |= ((pl[p][(64 + k) >> 5] >> ((64 + k) & 31)) & 1u) << (2 * B + p);
  }
  return x;
}

// Blocks: (group, query quad, chunk of the group's keys); a block builds its
// tables, then each wave takes 64-key batches of the chunk, one key per lane.
template <int B>
__global__ void __launch_bounds__(kPThreads, 1)
logits_polar128_kernel(const float* __restrict__ vw, int64_t nq, int64_t n, int64_t stride, int64_t half,
                       int quads, int chunks, int64_t keys_per_block, const uint32_t* __restrict__ codes,
                       const uint32_t* __restrict__ signs, const float* __restrict__ norms,
                       const float* __restrict__ rnorms, const float* __restrict__ ptab,
                       float* __restrict__ scores) {
  constexpr int L = 1 << B;           // levels per angle
  constexpr int kIdx = 1 << (3 * B);  // entries per subtree table
  __shared__ f32x4 qt[32 * kIdx];     // [subtree][index] -> 4 queries
  __shared__ f32x4 st[16 * 256];      // [byte position][byte] -> 4 queries
  __shared__ float2 lt[5][L];         // levels 3..7: (cos, sin) of each level value
  __shared__ float vs[2][4][128];     // v and w of the 4 queries

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t pair = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int64_t grp = pair / quads, q0 = (pair % quads) * 4;
  const int qc = int(nq - q0 < 4 ? nq - q0 : 4);
  const int64_t kbeg = c * keys_per_block;
  const int64_t kend = kbeg + keys_per_block < n ? kbeg + keys_per_block : n;

  // ---- prologue: the queries' v and w (zero past qc), the level tables
  for (int i = tid; i < 2 * 4 * 128; i += kPThreads) {
    const int part = i >> 9, q = (i >> 7) & 3, j = i & 127;
    const int64_t row = grp * nq + q0 + (q < qc ? q : 0);
    vs[part][q][j] = q < qc ? vw[row * stride + part * half + j] : 0.0f;
  }
  if (tid < 5 * L) {
    const int l = 3 + tid / L, code = tid % L;
    const float* t = ptab + (l - 1) * kPolarTab;
    lt[l - 3][code] = make_float2(t[16 + code], t[32 + code]);
  }
  __syncthreads();
  // subtree tables: entry x of subtree k = cos psi (v_4k cos a + v_4k+1 sin a)
  // + sin psi (v_4k+2 cos b + v_4k+3 sin b), a, b the level-1 and psi the
  // level-2 values of the index bits (quad_index's order)
  for (int i = tid; i < 32 * kIdx; i += kPThreads) {
    const int k = i / kIdx, x = i % kIdx;
    int ca = 0, cb = 0, cp = 0;
#pragma unroll
    for (int p = 0; p < B; ++p) {
      ca |= ((x >> (2 * p)) & 1) << p;
      cb |= ((x >> (2 * p + 1)) & 1) << p;
      cp |= ((x >> (2 * B + p)) & 1) << p;
    }
    const float* t1 = ptab;               // level 1
    const float* t2 = ptab + kPolarTab;   // level 2
    const float ca_c = t1[16 + ca], ca_s = t1[32 + ca], cb_c = t1[16 + cb], cb_s = t1[32 + cb];
    const float pc = t2[16 + cp], ps = t2[32 + cp];
    f32x4 e;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* v = vs[0][q] + 4 * k;
      const float lo = fmaf(v[1], ca_s, v[0] * ca_c);
      const float hi = fmaf(v[3], cb_s, v[2] * cb_c);
      e[q] = fmaf(ps, hi, pc * lo);
    }
    qt[i] = e;
  }
  // sign tables: entry x of byte position g = sum over its 8 coordinates of
  // w_j (+1 for a set bit, -1 otherwise), in coordinate order
  for (int i = tid; i < 16 * 256; i += kPThreads) {
    const int g = i >> 8, x = i & 255;
    f32x4 e;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* wv = vs[1][q] + 8 * g;
      float s = 0.0f;
#pragma unroll
      for (int b = 0; b < 8; ++b) s += ((x >> b) & 1) ? wv[b] : -wv[b];
      e[q] = s;
    }
    st[i] = e;
  }
  __syncthreads();

  const float kappa = 1.2533141373155002512f / 128.0f;  // sqrt(pi/2) / d
  const int64_t nbatch = (kend - kbeg + 63) / 64;
  for (int64_t b = wave; b < nbatch; b += kPWaves) {
    const int64_t t = kbeg + b * 64 + lane;
    const int64_t key = grp * n + (t < kend ? t : kend - 1);
    uint32_t pl[B][4];
#pragma unroll
    for (int p = 0; p < B; ++p) {
      const uint4 u = *reinterpret_cast<const uint4*>(codes + (key * B + p) * 4);
      pl[p][0] = u.x;
      pl[p][1] = u.y;
      pl[p][2] = u.z;
      pl[p][3] = u.w;
    }
    const uint4 sg = *reinterpret_cast<const uint4*>(signs + key * 4);
    const float nk = norms[key], rho = rnorms[key];

    // <v, z_hat>: subtrees of 4 coordinates from the table, then levels 3..7
    f32x4 y5[4];
#pragma unroll
    for (int m5 = 0; m5 < 4; ++m5) {
      f32x4 y4[2];
#pragma unroll
      for (int i4 = 0; i4 < 2; ++i4) {
        const int m4 = 2 * m5 + i4;
        f32x4 y3[2];
#pragma unroll
        for (int i3 = 0; i3 < 2; ++i3) {
          const int m3 = 2 * m4 + i3;
          const f32x4 a = qt[(2 * m3) * kIdx + quad_index<B>(pl, 2 * m3)];
          const f32x4 bq = qt[(2 * m3 + 1) * kIdx + quad_index<B>(pl, 2 * m3 + 1)];
          const float2 cs = lt[0][code_of<B>(pl, slot0(3) + m3)];
          y3[i3] = cs.x * a + cs.y * bq;
        }
        const float2 cs = lt[1][code_of<B>(pl, slot0(4) + m4)];
        y4[i4] = cs.x * y3[0] + cs.y * y3[1];
      }
      const float2 cs = lt[2][code_of<B>(pl, slot0(5) + m5)];
      y5[m5] = cs.x * y4[0] + cs.y * y4[1];
    }
    const float2 c60 = lt[3][code_of<B>(pl, slot0(6))], c61 = lt[3][code_of<B>(pl, slot0(6) + 1)];
    const f32x4 y60 = c60.x * y5[0] + c60.y * y5[1];
    const f32x4 y61 = c61.x * y5[2] + c61.y * y5[3];
    const float2 c7 = lt[4][code_of<B>(pl, slot0(7))];
    const f32x4 s1 = c7.x * y60 + c7.y * y61;

    // <w, 2 beta - 1>, byte by byte
    const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
    f32x4 s2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < 16; ++g) s2 += st[g * 256 + __builtin_amdgcn_ubfe(sw[g >> 2], 8 * (g & 3), 8)];

    if (t < kend) {
      const float corr = rho * kappa;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < qc) __builtin_nontemporal_store(nk * fmaf(corr, s2[q], s1[q]), &scores[(grp * nq + q0 + q) * n + t]);
    }
  }
}

}  // namespace

bool logits_polar128_supported(const tq_ctx* h) {
  return h->polar && h->d == 128 && h->words == 4 && h->polar_levels == 7 && (h->code_bits == 1 || h->code_bits == 2) &&
         h->d_polar_tab && !force_reference_kernels();
}

hipError_t launch_logits_polar128(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                                  const uint32_t* signs, const float* norms, const float* rnorms, int64_t n,
                                  float* scores, hipStream_t stream) {
  const int64_t quads = (nq + 3) / 4;
  const int64_t pairs = groups * quads;
  // about one block per CU in all, each on a whole number of 64-key batches
  int64_t chunks = (h->cus + pairs - 1) / pairs;
  const int64_t batches = (n + 63) / 64;
  chunks = chunks < batches ? chunks : batches;
  chunks = chunks < 1 ? 1 : chunks;
  const int64_t per = (batches + chunks - 1) / chunks * 64;
  chunks = (n + per - 1) / per;  // no empty chunk
  const dim3 grid(static_cast<uint32_t>(pairs * chunks));
  auto kernel = h->code_bits == 1 ? logits_polar128_kernel<1> : logits_polar128_kernel<2>;
  hipLaunchKernelGGL(kernel, grid, dim3(kPThreads), 0, stream, vw, nq, n, vw_stride(h->d), vw_half(h->d), int(quads),
                     int(chunks), per, codes, signs, norms, rnorms, h->d_polar_tab, scores);
  return hipGetLastError();
}

}  // namespace tqdev
