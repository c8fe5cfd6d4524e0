// Decode-style scoring kernel for d in (96, 128] (four 32-bit words per bit
// plane): streams packed keys once, one key per lane, and scores the 4
// queries of a (group, quad) per pass with byte-indexed lookup tables in LDS.
//
// Method ("TurboQuant digest" (juejin.cn) section 2; "TurboQuant deep review"
// (freelamp.com), error-compensation section): the score of query q against a
// packed key is
//     n * ( <v, c[idx]> + rho * sqrt(pi/2) / d * <w, 2 beta - 1> ),
// v = Pi q, w = G v.  A symmetric level set is an odd multilinear function of
// the plane signs s_p = 2 b_p - 1, c[idx] = sum_S alpha_S prod_{p in S} s_p
// over odd-size plane subsets S, and prod_{p in S} s_p = 2 (XOR_{p in S} b_p) - 1.
// So every term is a signed sum <x, 2 b - 1> of a vector x (v or w) over one bit
// word b, which a table indexed by one byte of b evaluates 8 coordinates at a
// time:  T_x[g][byte] = sum_{i<8} (bit i of byte ? +1 : -1) x[8 g + i].
//
// One workgroup per CU takes a range of one (group, quad)'s keys.  It first
// computes v = Pi q and w = S q (S = G Pi, formed on the host) of its 4
// queries, reading the matrices straight from L2 (the first keys are already
// loading), scales each vector by a power of two so that
// its norm lies in [1, 2), and stores the tables as float16 (4 queries per
// 8-byte entry):
//   entry (byte x, table tab (0 = v, 1 = w), position g) at x*256 + tab*128 + g*8.
// Lane l walks the 16 byte positions starting at g = l mod 16 (its bit planes
// are rotated by l mod 16 bytes), so the 16 lanes served by one LDS pass read
// 16 distinct positions whose entries fill the 32 banks exactly, whatever the
// key bytes are.  One v_perm builds the byte address (key byte -> bits 8..15,
// 8 g -> bits 0..7).  Lookups of one word (32 coordinates) are summed in
// float16 pairs and then added into float32 accumulators with v_dot2_f32_f16.
// Waves take the keys in batches of 64 from a counter in LDS, so that the
// waves sharing a CU finish together whichever of them the arbiter favours.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lut_tables.h"
#include "tq_internal.h"

namespace tqdev {
namespace {

using namespace ltab;

// Block size: 16 waves (one block per CU) while the key loop fits 128
// registers, else 8.
template <int B>
struct Shape {
  static constexpr int kThreads = B == 4 ? 512 : 1024;
  static constexpr int kParts = kThreads / kDim;        // row slices of the query transform
  static constexpr int kRows = kDim / kParts;           // rows per slice
  static constexpr int kWalk = 256 * 2 * 16 * 4 / kThreads;  // table entries per thread
};

// HI: fractional widths with hi = 64: coordinates 0..63 (bytes 0..7 of
// each plane) carry B + 1 index bits and the finer level set, whose plane
// expansion is peh; 64..127 carry B bits and pe.  A lane scores one half in
// byte steps 0..7 and the other in steps 8..15 (lanes 8..15 of every 16 the
// other way round), so the 16 lanes of an LDS pass still read 16 distinct
// byte positions; each step looks up the finer set's term count, and a
// lane in its coarse half leaves the surplus terms' sums out.
template <int B, bool HI>
__global__ void __launch_bounds__(Shape<HI ? B + 1 : B>::kThreads, 1)
logits_lut128_kernel(const float* __restrict__ queries, int quads, int64_t nq, int64_t n, int d,
                     const float* __restrict__ piT, const float* __restrict__ sT,  // 128 x 128, zero-padded
                     const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
                     const float* __restrict__ norms, const float* __restrict__ rnorms,
                     float* __restrict__ scores, PlaneExpansion pe, PlaneExpansion peh, float kappa, int chunks,
                     int64_t keys_per_block) {
  constexpr int NPL = HI ? B + 1 : B;  // planes loaded per key
  using TT = Terms<NPL>;               // terms of the (finer) level set
  using TB = Terms<B>;                 // terms of the coarse set
  using SH = Shape<NPL>;
  constexpr int NT = TT::count;
  constexpr int kThreads = SH::kThreads, kWaves = kThreads / 64;
  __shared__ __align__(16) unsigned char tabs[kTableBytes];
  __shared__ float4 qs[kDim];  // the 4 queries, coordinate-major
  __shared__ float vec[2][4][kDim];  // scaled v and w
  __shared__ float scale[2][4];
  __shared__ uint32_t next_batch;
  const int tid = threadIdx.x;
  const int64_t pair = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int64_t grp = pair / quads;
  const int64_t q0 = (pair % quads) * 4;
  const int qc = int(nq - q0 < 4 ? nq - q0 : 4);
  const int64_t kbeg = c * keys_per_block;
  const int64_t kend = kbeg + keys_per_block < n ? kbeg + keys_per_block : n;
  if (kbeg >= kend) return;  // whole block: no keys in its range
  // keys go out in batches of 64 (one per lane); wave w starts on batch w
  // and then takes the next unclaimed batch from a counter in LDS, so the
  // waves of the CU finish together however its arbiter favours them
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t nbatch = (kend - kbeg + 63) / 64;
  // this lane's key of a batch, within the group; past the end: the last key
  auto key_of = [&](int64_t batch) {
    const int64_t k = kbeg + batch * 64 + lane;
    return k < kend ? k : kend - 1;
  };

  // ---- v = Pi q and w = S q (float32) ----
  // Thread (part, j) sums rows i in [kRows part, kRows part + kRows) of
  // output j for the 4 queries and both matrices, loading them in batches of
  // 16 rows per matrix; the first batch is in flight while the queries are
  // staged.  The tables' space holds the partial sums [part][tab][q][j]
  // until the parts are added.
  const int mj = tid & (kDim - 1), part = tid / kDim;
  // the matrices are zero-padded to 128 x 128: no bounds checks
  const float* pcol = piT + SH::kRows * part * kDim + mj;
  const float* scol = sT + SH::kRows * part * kDim + mj;
  auto load_batch = [&](int i0, float (&pv)[16], float (&pw)[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      pv[k] = pcol[(i0 + k) * kDim];
      pw[k] = scol[(i0 + k) * kDim];
    }
  };
  // Loads complete in issue order, so the order below lets each wait cover
  // only what it needs: queries, the first matrix batch, then the wave's
  // first keys (they arrive while the tables are built).  Threads below 512
  // load coordinate tid % 128 of query tid / 128 (addresses clamped in
  // range, values past d or nq zeroed).
  const int qi = tid & (kDim - 1), qq = (tid >> 7) & 3;
  const bool qok = q0 + qq < nq && qi < d;
  const float qraw = queries[(grp * nq + (q0 + qq < nq ? q0 + qq : nq - 1)) * d + (qi < d ? qi : d - 1)];
  float pv0[16], pw0[16];
  load_batch(0, pv0, pw0);
  if (tid < 4 * kDim) reinterpret_cast<float*>(qs)[qi * 4 + qq] = qok ? qraw : 0.0f;
  if (tid == 0) next_batch = kWaves;
  __syncthreads();
  auto load = [&](int64_t key) {
    if constexpr (HI)
      return load_key_hi<B>(codes, signs, norms, rnorms, key);
    else
      return load_key<B>(codes, signs, norms, rnorms, key);
  };
  Packed<NPL> cur = load(grp * n + key_of(wave));
  {
    float av[4] = {0.0f, 0.0f, 0.0f, 0.0f}, aw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    auto accumulate = [&](int i0, const float (&pv)[16], const float (&pw)[16]) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float4 x = qs[SH::kRows * part + i0 + k];
        av[0] = fmaf(pv[k], x.x, av[0]);
        av[1] = fmaf(pv[k], x.y, av[1]);
        av[2] = fmaf(pv[k], x.z, av[2]);
        av[3] = fmaf(pv[k], x.w, av[3]);
        aw[0] = fmaf(pw[k], x.x, aw[0]);
        aw[1] = fmaf(pw[k], x.y, aw[1]);
        aw[2] = fmaf(pw[k], x.z, aw[2]);
        aw[3] = fmaf(pw[k], x.w, aw[3]);
      }
    };
    accumulate(0, pv0, pw0);
    if constexpr (SH::kRows > 16) {
      float pv1[16], pw1[16];
      load_batch(16, pv1, pw1);
      accumulate(16, pv1, pw1);
    }
    float* red = reinterpret_cast<float*>(tabs);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      red[((part * 2 + 0) * 4 + q) * kDim + mj] = av[q];
      red[((part * 2 + 1) * 4 + q) * kDim + mj] = aw[q];
    }
  }
  __syncthreads();
  for (int e = tid; e < 2 * 4 * kDim; e += kThreads) {  // e = (tab * 4 + q) * kDim + j
    const float* red = reinterpret_cast<const float*>(tabs);
    float sum = 0.0f;
#pragma unroll
    for (int pp = 0; pp < SH::kParts; ++pp) sum += red[pp * 1024 + e];
    vec[e >> 9][(e >> 7) & 3][e & (kDim - 1)] = sum;
  }
  __syncthreads();
  // power-of-two scale per (table, query): scaled norm in [1, 2); wave w < 8
  // reduces vector (w >> 2, w & 3)
  if (tid < 8 * 64) {
    const int tab = wave >> 2, q = wave & 3;
    const float x0 = vec[tab][q][lane], x1 = vec[tab][q][lane + 64];
    float ss = fmaf(x0, x0, x1 * x1);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) {
      int e = 0;
      (void)frexpf(sqrtf(ss), &e);
      scale[tab][q] = ss > 0.0f ? ldexpf(1.0f, 1 - e) : 1.0f;
    }
  }
  __syncthreads();
  // Byte tables (tab 0 = v, 1 = w) by Gray-code walks: thread (tab, seg,
  // position g, query q) = tid bits (top, middle, 5..2, 1..0) visits the kWalk
  // bytes x = rank ^ (rank >> 1), rank in [kWalk seg, kWalk seg + kWalk).
  // Successive bytes differ in one bit b, so each entry is the previous one
  // plus or minus twice coordinate 8 g + b; a wave writes 128 contiguous
  // bytes per step.  The running float32 sum drifts by well under the
  // float16 rounding of the stored entry.
  {
    constexpr int kW = SH::kWalk, kSegs = 256 / kW, kHi = kW / 2;
    const int q = tid & 3, gg = (tid >> 2) & 15, seg = (tid >> 6) & (kSegs - 1), tab = tid / (64 * kSegs);
    const float sc = scale[tab][q];
    float xs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[i] = sc * vec[tab][q][8 * gg + i];
    unsigned char* col = tabs + tab * 128 + gg * 8 + q * 2;
    // x(rank0 + m) = gb ^ gray(m) with gb = gray(kW seg) a multiple of kW / 2:
    // only bit kW / 2 of gray(m) interacts with gb, so two bases and a
    // compile-time offset address every entry
    const int rank0 = kW * seg, gb = rank0 ^ (rank0 >> 1);
    unsigned char* base0 = col + 256 * gb;
    unsigned char* base1 = col + 256 * (gb ^ kHi);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += ((gb >> i) & 1) ? xs[i] : -xs[i];
    *reinterpret_cast<_Float16*>(base0) = static_cast<_Float16>(acc);
#pragma unroll
    for (int m = 1; m < kW; ++m) {
      const int gm = m ^ (m >> 1), b = __builtin_ctz(m);
      const bool up = (1 << b) == kHi ? (((gb ^ gm) >> b) & 1) != 0 : ((gm >> b) & 1) != 0;
      acc += up ? 2.0f * xs[b] : -2.0f * xs[b];
      *reinterpret_cast<_Float16*>(((gm & kHi) ? base1 : base0) + 256 * (gm & (kHi - 1))) =
          static_cast<_Float16>(acc);
    }
  }
  __syncthreads();

  // per-lane rotation and address bases
  const uint32_t r = uint32_t(tid) & 15u;
  const bool w1 = (r >> 2) & 1u, w2 = (r >> 3) & 1u;
  const uint32_t bs = r & 3u;
  uint32_t lb[8];
  // byte position of step t: (t + r) mod 16, or for fractional widths
  // ((t + r) mod 8) in the half that step t covers
  auto pos = [&](uint32_t t) -> uint32_t {
    if constexpr (HI)
      return ((((t >> 3) & 1u) ^ (w2 ? 1u : 0u)) << 3) | ((t + r) & 7u);
    else
      return (t + r) & 15u;
  };
#pragma unroll
  for (int k = 0; k < 8; ++k) lb[k] = (pos(2u * k) * 8u) | ((pos(2u * k + 1u) * 8u) << 8);
  float inv_v[4], inv_w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    inv_v[q] = 1.0f / scale[0][q];
    inv_w[q] = kappa / scale[1][q];
  }
  // HI: coefficients of the term sums of the lane's first and second half
  // (finer set peh, coarse set pe with no terms past its count)
  float al_a[NT], al_b[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const float af = HI ? peh.alpha[j] : pe.alpha[j];
    const float ac = j < TB::count ? pe.alpha[j] : 0.0f;
    al_a[j] = w2 ? ac : af;
    al_b[j] = w2 ? af : ac;
  }
  const half2_t pick_lo = {(_Float16)1.0f, (_Float16)0.0f};
  const half2_t pick_hi = {(_Float16)0.0f, (_Float16)1.0f};
  // claims: one LDS add per batch, made a batch ahead of the load it feeds
  auto claim = [&]() -> int64_t {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(&next_batch, 1u);
    return __builtin_amdgcn_readfirstlane(v);
  };

  int64_t b = wave;         // batch being scored
  int64_t bn = claim();     // the one after it
  while (b < nbatch) {
    const int64_t bnn = claim();
    const Packed<NPL> nxt = load(grp * n + key_of(bn));  // unused past the end
    Words pl[NPL];
#pragma unroll
    for (int p = 0; p < NPL; ++p) pl[p] = HI ? rotate_halves(cur.plane[p], w1, bs, w2) : rotate(cur.plane[p], w1, w2, bs);
    const Words sg = HI ? rotate_halves(cur.sign, w1, bs, w2) : rotate(cur.sign, w1, w2, bs);
    Words term[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t x = 0;
#pragma unroll
        for (int p = 0; p < NPL; ++p)
          if (TT::mask[j] & (1u << p)) x ^= pl[p].w[i];
        if constexpr (HI) {
          // words 0-1 are this lane's first half: the finer one unless the
          // halves are swapped (w2)
          uint32_t y = 0;
          if (j < TB::count) {
#pragma unroll
            for (int p = 0; p < B; ++p)
              if (TB::mask[j] & (1u << p)) y ^= pl[p].w[i];
          }
          x = ((i < 2) != w2) ? x : y;
        }
        term[j].w[i] = x;
      }
    }
    float acc[NT + 1][4];
#pragma unroll
    for (int j = 0; j <= NT; ++j) acc[j][0] = acc[j][1] = acc[j][2] = acc[j][3] = 0.0f;
    float s1h[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // HI: level-set sums of the first half
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // one 32-bit word (4 byte steps) at a time
      half2_t part[NT + 1][2];
#pragma unroll
      for (int j = 0; j <= NT; ++j) part[j][0] = part[j][1] = half2_t{(_Float16)0.0f, (_Float16)0.0f};
#define TQ_STEP(T)                                                                                   \
  {                                                                                                  \
    _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                                 \
      const Entry e = lut<0>(tabs, __builtin_amdgcn_perm(term[j].w[i], lb[(T) >> 1], perm_sel<(T)>())); \
      part[j][0] += e.q01;                                                                           \
      part[j][1] += e.q23;                                                                           \
    }                                                                                                \
    const Entry e = lut<1>(tabs, __builtin_amdgcn_perm(sg.w[i], lb[(T) >> 1], perm_sel<(T)>()));     \
    part[NT][0] += e.q01;                                                                            \
    part[NT][1] += e.q23;                                                                            \
    if ((T) & 1) pin<NT + 1>(part);                                                                  \
  }
      // steps 4i .. 4i+3; lb and the selector depend only on (T & 3) and (T >> 1)
      if (i == 0) { TQ_STEP(0) TQ_STEP(1) TQ_STEP(2) TQ_STEP(3) }
      if (i == 1) { TQ_STEP(4) TQ_STEP(5) TQ_STEP(6) TQ_STEP(7) }
      if (i == 2) { TQ_STEP(8) TQ_STEP(9) TQ_STEP(10) TQ_STEP(11) }
      if (i == 3) { TQ_STEP(12) TQ_STEP(13) TQ_STEP(14) TQ_STEP(15) }
#undef TQ_STEP
#pragma unroll
      for (int j = 0; j <= NT; ++j) {
        acc[j][0] = __builtin_amdgcn_fdot2(part[j][0], pick_lo, acc[j][0], false);
        acc[j][1] = __builtin_amdgcn_fdot2(part[j][0], pick_hi, acc[j][1], false);
        acc[j][2] = __builtin_amdgcn_fdot2(part[j][1], pick_lo, acc[j][2], false);
        acc[j][3] = __builtin_amdgcn_fdot2(part[j][1], pick_hi, acc[j][3], false);
      }
      if constexpr (HI) {
        if (i == 1) {
          // end of the first half: its level set's coefficients, then the
          // term sums start again for the second half
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int j = 0; j < NT; ++j) s1h[q] = fmaf(al_a[j], acc[j][q], s1h[q]);
          }
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[j][0] = acc[j][1] = acc[j][2] = acc[j][3] = 0.0f;
        }
      }
    }
    // lanes past the end scored key kend - 1 again and store the same value
    // there: no branch around the stores
    const int64_t key = key_of(b);
    const float corr = cur.rho;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float s1 = s1h[q];
#pragma unroll
      for (int j = 0; j < NT; ++j) s1 = fmaf(HI ? al_b[j] : pe.alpha[j], acc[j][q], s1);
      const float sw = acc[NT][q] * inv_w[q];
      if (q < qc) __builtin_nontemporal_store(cur.n * fmaf(corr, sw, s1 * inv_v[q]), &scores[(grp * nq + q0 + q) * n + key]);
    }
    cur = nxt;
    b = bn;
    bn = bnn;
  }
}

template <int B, bool HI>
hipError_t launch_b(const tq_ctx* h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
                    const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores,
                    hipStream_t stream) {
  const int64_t quads = (nq + 3) / 4;
  const int64_t pairs = groups * quads;
  // about one block per CU, each on one (group, query quad) pair's range of
  // keys (a multiple of 64)
  const int64_t cus = h->cus;
  int64_t chunks = (cus + pairs - 1) / pairs;
  int64_t kpb = (n + chunks - 1) / chunks;
  kpb = (kpb + 63) / 64 * 64;
  chunks = (n + kpb - 1) / kpb;
  const int64_t blocks = chunks * pairs;
  if (blocks > 0x7FFFFFFF || chunks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const float kappa = 1.2533141373155002512f / float(h->d);
  hipLaunchKernelGGL((logits_lut128_kernel<B, HI>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(Shape<HI ? B + 1 : B>::kThreads), 0, stream, queries, int(quads), nq, n, h->d, h->d_piT128,
                     h->d_sT128, codes, signs, norms, rnorms, scores, h->planes, h->planes_hi, kappa,
                     static_cast<int>(chunks), kpb);
  return hipGetLastError();
}

}  // namespace

bool logits_lut128_supported(const tq_ctx* h) {
  // fractional widths: the finer set on bytes 0..7 (hi = 64), at most 4
  // index bits there
  const bool widths = h->hi == 0 || (h->hi == 64 && h->code_bits <= 3);
  return widths && h->words == 4 && h->d <= kDim && h->d_piT128 && h->d_sT128 && h->code_bits >= 1 &&
         h->code_bits <= 4;
}

hipError_t launch_logits_lut128(const tq_ctx* h, const float* queries, int64_t groups, int64_t nq,
                                const uint32_t* codes, const uint32_t* signs, const float* norms,
                                const float* rnorms, int64_t n, float* scores, hipStream_t stream) {
  if (h->hi > 0) {
    switch (h->code_bits) {
      case 1: return launch_b<1, true>(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
      case 2: return launch_b<2, true>(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
      case 3: return launch_b<3, true>(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (h->code_bits) {
    case 1: return launch_b<1, false>(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    case 2: return launch_b<2, false>(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    case 3: return launch_b<3, false>(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    case 4: return launch_b<4, false>(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqdev
