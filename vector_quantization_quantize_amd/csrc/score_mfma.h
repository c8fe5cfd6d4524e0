// Matrix-core scorer for many queries against packed keys, d <= 256.
//
// Method ("TurboQuant digest" section 2; "TurboQuant deep review",
// error-compensation section): the score of query q against a packed key is
//     n * ( <v, c[idx]> + rho * sqrt(pi/2) / d * <w, 2 beta - 1> ),
// v = Pi q, w = G v.  With many queries per key set (search), both inner
// products are dense contractions over the coordinates: scores = n (V C^T +
// kappa rho W Sgn^T) for the query rows V, W and the keys' level values C
// and signs Sgn.  They run on the matrix cores, 32 x 32 x 16 f16 tiles.
// Level values, by form:
//   * sign: one index bit and a symmetric level set, c[idx] = c[1] (2 idx -
//     1): C is c[1] times a +-1 matrix, one exact piece;
//   * one piece: at most two level magnitudes; sigma c[level] is a float16
//     number for the scale sigma found at init (to 2^-19 relative);
//   * two pieces: hi and lo float16 pieces of 2^10 c[level] (22 bits).
// Signs are exact.  Each query row takes one power-of-two scale s_R that
// puts max(||v||, lambda ||w||) in [2^9, 2^10), lambda being the form's
// ratio that lets both products share one output scale:
//     u = n (acc_v + rho acc_w),   score = (gamma / s_R) u.
// Rounding the rows to float16 (11 significant bits, all elements normal,
// round to nearest: relative error at most 2^-11 per element) moves <v, c>
// by at most 2^-11 ||v|| ||c|| (Cauchy-Schwarz, ||c[idx]|| below 1) and the
// sign term by at most 2^-11 ||w||_1 sqrt(pi/2) rho / d, which is about
// 2^-11 rho ||q|| for a Gaussian G (||w||_1 near sqrt(2/pi) d ||q||):
// together at most about 0.7 of the 1e-3 ||q|| n bound when every rounding
// error lines up with the key; for data not built against the rounding the
// errors add incoherently and stay near 2^-11 / sqrt(d) of the score scale.
//
// The number of K steps (d / 16, rounded up) is a template parameter, so the
// step loop is straight-line code the compiler can pipeline; one translation
// unit per form instantiates all sixteen.
//
// Work split: a block of 4 waves takes 128 queries (wave w: rows 32w ..
// 32w + 31, A operands loaded once into registers) and walks 32-key tiles.
// Thread (key, word) of a tile expands 32 coordinates of one key from its
// bit planes into LDS rows of float16 values: signs with integer ops (bit ->
// sign bit of +-1), level values through small LDS tables indexed by packed
// index bits.  One- and two-plane forms double-buffer the rows: tile t + 1 is
// expanded while tile t is multiplied, one barrier per tile.  Rows past nq
// and keys past the end repeat the last one and store the same value there,
// so stores carry no branch.
//
// Search form ("TurboQuant digest" section 3: the k best keys per query by
// this score): instead of storing the tile, each wave keeps, in LDS, the k
// best (u, key) pairs seen so far for each of its 32 rows, best first, with
// each row's k-th u (-inf while the list is short) in registers.  u orders a
// row's keys as the score does (gamma / s_R > 0).  A key enters when its u
// beats the row's k-th: candidates are found with one compare and ballot
// per accumulator register and inserted one at a time by the whole wave
// (insert position = entries at least as high, which all hold smaller keys
// since keys arrive in ascending order).  At the end each block writes its
// lists as scores; a merge pass combines the lists of all blocks that walked
// a row's keys.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace score {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kTileKeys = 32;     // MFMA N
constexpr float kCScale = 1024.0f;
constexpr int kBlocksPerCu = 2;   // resident blocks per CU (registers, LDS)

template <int B, int F>
struct Form {
  static constexpr int E = B == 1 ? 8 : B == 2 ? 4 : 2;  // coordinates per table lookup
  static constexpr int kPieces = F == kTwoPiece ? 2 : 1;
  static constexpr int kEntries = F == kSignForm ? 1 : 1 << (E * B);
  static constexpr int kHalves = kPieces * E;  // halves per table entry
  static constexpr int kPlanes = kPieces + 1;  // staged planes: level piece(s), QJL signs
  static constexpr int kBufs = kPlanes == 2 ? 2 : 1;
};

// staged row of KS steps in halves: 16 KS of coordinates, then (odd KS) room
// for the two bytes the half-used last word expands to (never read), then a
// 16-byte pad: an odd number of 16-byte chunks, so the 32 rows' b128 reads
// at one offset are conflict-free
template <int KS>
constexpr int row_halves() {
  return 16 * KS + (KS % 2 ? 24 : 8);
}

__device__ __forceinline__ f16x8 to_f16x8(const float4& a, const float4& b, float s) {
  f16x8 h;
  h[0] = static_cast<_Float16>(a.x * s);
  h[1] = static_cast<_Float16>(a.y * s);
  h[2] = static_cast<_Float16>(a.z * s);
  h[3] = static_cast<_Float16>(a.w * s);
  h[4] = static_cast<_Float16>(b.x * s);
  h[5] = static_cast<_Float16>(b.y * s);
  h[6] = static_cast<_Float16>(b.z * s);
  h[7] = static_cast<_Float16>(b.w * s);
  return h;
}

// scores as unsigned integers in the same order (for atomicMax)
__device__ __forceinline__ unsigned int enc_score(float x) {
  const unsigned int b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float dec_score(unsigned int e) {
  return __uint_as_float((e & 0x80000000u) ? (e & 0x7FFFFFFFu) : ~e);
}

__device__ __forceinline__ float read_lane(float x, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
}

// 8 sign bits (x < 256) -> 8 float16 values, element e from bit e: set -> -1,
// clear -> +1 (the query rows carry the compensating minus).  With bit i of
// X at i and i + 15, X << (15 - 2m) puts bit 2m at 15 and bit 2m + 1 at 31:
// the sign bits of the two halves of dword m.
// The two constants come in registers (mask, one): three-operand integer ops
// take no literal on this target, and with registers (a & mask) | one is a
// single instruction.
__device__ __forceinline__ uint4 expand_signs(uint32_t x, uint32_t mask, uint32_t one) {
  const uint32_t X = x | (x << 15);
  uint4 r;
  r.x = ((X << 15) & mask) | one;
  r.y = ((X << 13) & mask) | one;
  r.z = ((X << 11) & mask) | one;
  r.w = ((X << 9) & mask) | one;
  return r;
}

template <int B, int F, int KS, bool kTopk>
__global__ void __launch_bounds__(kThreads, kBlocksPerCu)
score_mfma_kernel(const float* __restrict__ vw, int64_t vw_stride, int64_t vw_half, int64_t nq,
                  const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
                  const float* __restrict__ norms, const float* __restrict__ rnorms, int64_t nkeys,
                  int64_t key_stride, float* __restrict__ scores, int64_t sstride, ScoreForm fp,
                  int64_t tiles_per_block, float* __restrict__ top_s, int64_t* __restrict__ top_i, int top_k,
                  unsigned int* __restrict__ bound) {
  static_assert(F != kSignForm || B == 1, "sign form is for one index bit");
  using Fm = Form<B, F>;
  constexpr int E = Fm::E;
  constexpr int P = Fm::kPlanes;
  constexpr int rs = row_halves<KS>();
  constexpr int plane = kTileKeys * rs;
  constexpr int kWords = (KS + 1) / 2;  // packed words per key and plane (d in (16 KS - 16, 16 KS])
  __shared__ uint4 stage4[Fm::kBufs * P * plane / 8];
  __shared__ _Float16 vtab[F == kSignForm ? 8 : Fm::kEntries * Fm::kHalves];
  __shared__ __align__(16) float row_f[128];  // gamma / s_R of the block's rows
  __shared__ float row_t[128];                // search form: shared bound of each row, in u units
  extern __shared__ float lst_all[];          // search form: [128][k] u, then [128][k] keys
  _Float16* stage = reinterpret_cast<_Float16*>(stage4);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kl = lane & 31, g = lane >> 5;
  const int64_t grp = blockIdx.z;
  vw += grp * nq * vw_stride;
  codes += grp * key_stride * B * kWords;
  signs += grp * key_stride * kWords;
  norms += grp * key_stride;
  rnorms += grp * key_stride;
  if constexpr (!kTopk) scores += grp * nq * sstride;

  // level-value table: entry idx holds the pieces of E coordinates whose
  // index bits (plane p, coordinate e) are bit p * E + e of idx
  if constexpr (F != kSignForm) {
    for (int idx = tid; idx < Fm::kEntries; idx += kThreads) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        int level = 0;
#pragma unroll
        for (int p = 0; p < B; ++p) level |= ((idx >> (p * E + e)) & 1) << p;
        const float x = fp.val[level];
        const _Float16 hi = static_cast<_Float16>(x);
        vtab[idx * Fm::kHalves + e] = hi;
        if constexpr (F == kTwoPiece) vtab[idx * Fm::kHalves + E + e] = static_cast<_Float16>(x - float(hi));
      }
    }
  }

  // A operands of this wave's 32 query rows (rows past nq repeat the last)
  const int64_t qrow = blockIdx.x * 128 + 32 * w + kl;
  const float* vrow = vw + (qrow < nq ? qrow : nq - 1) * vw_stride + 8 * g;
  // pass 1: norms of the row's v and w (the row's two halves sit in lanes
  // l and l ^ 32); pass 2 reloads them (from cache) scaled into float16
  // (loads are kept few in flight: this runs once per block, and every
  // register it holds counts against the tile loop's budget)
  float ssv = 0.0f, ssw = 0.0f;
#pragma unroll 1
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 a = *reinterpret_cast<const float4*>(vrow + 16 * s + 4 * h);
      const float4 b = *reinterpret_cast<const float4*>(vrow + vw_half + 16 * s + 4 * h);
      ssv += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
      ssw += b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
    }
  }
  ssv += __shfl_xor(ssv, 32);
  ssw += __shfl_xor(ssw, 32);
  float sr = 1.0f;
  {
    const float m = fmaxf(sqrtf(ssv), fp.lambda * sqrtf(ssw));
    if (m > 0.0f && m < INFINITY) {
      int e = 0;
      (void)frexpf(m, &e);
      sr = ldexpf(1.0f, 10 - e);  // m * sr in [2^9, 2^10)
    }
  }
  // staged signs are negated: the rows that meet them carry a minus
  const float sv = F == kSignForm ? -sr : sr, sw = -sr * fp.lambda;
  f16x8 av[KS], aw[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    av[s] = to_f16x8(*reinterpret_cast<const float4*>(vrow + 16 * s),
                     *reinterpret_cast<const float4*>(vrow + 16 * s + 4), sv);
    aw[s] = to_f16x8(*reinterpret_cast<const float4*>(vrow + vw_half + 16 * s),
                     *reinterpret_cast<const float4*>(vrow + vw_half + 16 * s + 4), sw);
    if (s & 1) __builtin_amdgcn_sched_barrier(0);
  }
  if (g == 0) row_f[32 * w + kl] = fp.gamma / sr;

  // search form: this wave's 32 row lists (filled once the row factors are
  // known, below)
  float* lst_s = lst_all + 32 * w * top_k;
  int* lst_i = reinterpret_cast<int*>(lst_all + 128 * top_k) + 32 * w * top_k;

  // staging role: thread (key kk, word wi) of the tile, 32 coordinates
  const int kk = tid / kWords, wi = tid % kWords;
  const bool stager = tid < kTileKeys * kWords;
  const int64_t ntiles = (nkeys + kTileKeys - 1) / kTileKeys;
  const int64_t t0 = blockIdx.y * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < ntiles ? t0 + tiles_per_block : ntiles;
  auto fetch = [&](int64_t tile, uint32_t(&pw)[B + 1]) {
    int64_t key = tile * kTileKeys + kk;
    key = key < nkeys ? key : nkeys - 1;
#pragma unroll
    for (int p = 0; p < B; ++p) pw[p] = stager ? codes[(key * B + p) * kWords + wi] : 0u;
    pw[B] = stager ? signs[key * kWords + wi] : 0u;
  };
  // expand one tile's words into buffer buf; byte order rotated by word to
  // spread the rows' stores over the banks
  // sign-bit mask and +1 +1 in float16, opaque to the compiler (see expand_signs)
  uint32_t sgn_mask = 0x80008000u, sgn_one = 0x3C003C00u;
  asm volatile("" : "+v"(sgn_mask), "+v"(sgn_one));
  auto expand = [&](const uint32_t(&pw)[B + 1], _Float16* buf) {
    if (!stager) return;
    _Float16* row = buf + kk * rs;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int bq = (q + wi) & 3;
      {
        const int off = 8 * (4 * wi + bq);
        if constexpr (F == kSignForm) {
          *reinterpret_cast<uint4*>(row + off) = expand_signs(__builtin_amdgcn_ubfe(pw[0], 8 * bq, 8), sgn_mask, sgn_one);
        } else {
          _Float16 hv[8], lv[8];
#pragma unroll
          for (int k = 0; k < 8 / E; ++k) {
            uint32_t idx = 0;
#pragma unroll
            for (int p = 0; p < B; ++p) idx |= __builtin_amdgcn_ubfe(pw[p], 8 * bq + k * E, E) << (p * E);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              hv[k * E + e] = vtab[idx * Fm::kHalves + e];
              if constexpr (F == kTwoPiece) lv[k * E + e] = vtab[idx * Fm::kHalves + E + e];
            }
          }
          *reinterpret_cast<f16x8*>(row + off) = f16x8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
          if constexpr (F == kTwoPiece)
            *reinterpret_cast<f16x8*>(row + plane + off) = f16x8{lv[0], lv[1], lv[2], lv[3], lv[4], lv[5], lv[6], lv[7]};
        }
        *reinterpret_cast<uint4*>(row + (P - 1) * plane + off) =
            expand_signs(__builtin_amdgcn_ubfe(pw[B], 8 * bq, 8), sgn_mask, sgn_one);
      }
      __builtin_amdgcn_sched_barrier(0);  // one byte's values in registers at a time
    }
  };
  // norm and rho of this lane's key column (keys past the end repeat the last)
  auto key_of = [&](int64_t tile) {
    const int64_t key = tile * kTileKeys + kl;
    return key < nkeys ? key : nkeys - 1;
  };

  uint32_t nw[B + 1];
  float nk_next = 0.0f, rk_next = 0.0f;
  if (t0 < t1) {
    __syncthreads();  // value table
    fetch(t0, nw);
    expand(nw, stage);
    if (t0 + 1 < t1) fetch(t0 + 1, nw);
    nk_next = norms[key_of(t0)];
    rk_next = rnorms[key_of(t0)];
  }
  __syncthreads();  // first tile staged; row factors written
  // search form: a row's list starts as k placeholders (key -1, u -inf).
  // Keys enter above the row's threshold pr (per lane, for accumulator
  // element r: query row 8(r/4) + 4g + r%4 of the wave; rows past nq take
  // nothing), which is the larger of the list's k-th u and the row's shared
  // bound.  The bound (ordered-integer encoding, see enc_score) is the best
  // k-th score any block walking this row's keys has published: a lower
  // bound of the row's k-th best score over all keys.  Blocks publish and
  // read it every so many tiles; read back in u units it is taken a little
  // low, so that no key whose score reaches it is left out by rounding.
  float pr[16];
  auto sync_bounds = [&]() {
    if (lane < 32) {
      const int lrow = 32 * w + lane;
      const int64_t q = blockIdx.x * 128 + lrow;
      float t = -INFINITY;
      if (q < nq) {
        const float mine = lst_s[lane * top_k + top_k - 1] * row_f[lrow];
        const unsigned int e = enc_score(mine);
        const unsigned int old = atomicMax(bound + grp * nq + q, e);
        const float best = dec_score(old > e ? old : e);
        if (best > -INFINITY && best < INFINITY) {
          const float tu = best / row_f[lrow];
          t = tu - fabsf(tu) * 0x1p-20f;
        }
      }
      row_t[lrow] = t;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = fmaxf(pr[r], row_t[32 * w + 8 * (r >> 2) + 4 * g + (r & 3)]);
  };
  if constexpr (kTopk) {
    for (int i = lane; i < 32 * top_k; i += 64) {
      lst_s[i] = -INFINITY;
      lst_i[i] = -1;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pr[r] = blockIdx.x * 128 + 32 * w + 8 * (r >> 2) + 4 * g + (r & 3) < nq ? -INFINITY : INFINITY;
  }

  for (int64_t tile = t0; tile < t1; ++tile) {
    const int cur = Fm::kBufs == 2 ? static_cast<int>((tile - t0) & 1) : 0;
    const _Float16* buf = stage + cur * P * plane;
    const int64_t key_raw = tile * kTileKeys + kl;
    const float nk = nk_next, rk = rk_next;
    if (tile + 1 < t1) {
      nk_next = norms[key_of(tile + 1)];
      rk_next = rnorms[key_of(tile + 1)];
    }
    // B fragments of step s: lane reads key kl, coordinates 16s + 8g ..;
    // two steps in flight (step s + 2 is requested once step s is issued),
    // and no further: a scheduling fence after each step keeps the compiler
    // from hoisting every read (registers would run out)
    const _Float16* bb = buf + kl * rs + 8 * g;
    f16x8 pb[2][P];
    auto load_step = [&](int s, f16x8(&dst)[P]) {
#pragma unroll
      for (int p = 0; p < P; ++p) dst[p] = *reinterpret_cast<const f16x8*>(bb + p * plane + 16 * s);
    };
    load_step(0, pb[0]);
    if constexpr (KS > 1) load_step(1, pb[1]);
    f32x16 acc1 = {}, acc2 = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      f16x8(&cur)[P] = pb[s & 1];
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s], cur[0], acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(aw[s], cur[P - 1], acc2, 0, 0, 0);
      if constexpr (F == kTwoPiece) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s], cur[1], acc1, 0, 0, 0);
      if (s + 2 < KS) load_step(s + 2, cur);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (Fm::kBufs == 2) {
      // next tile into the other buffer while the matrix cores work
      if (tile + 1 < t1) {
        expand(nw, stage + (cur ^ 1) * P * plane);
        if (tile + 2 < t1) fetch(tile + 2, nw);
      }
    }
    if constexpr (!kTopk) {
      const int64_t key = key_raw < nkeys ? key_raw : nkeys - 1;
      // row offsets recomputed per tile, not held across the loop in registers
      int64_t ss = sstride;
      asm volatile("" : "+s"(ss));
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        // the four rows' score factors
        const float4 f = *reinterpret_cast<const float4*>(row_f + 32 * w + 8 * rq + 4 * g);
        const float fr[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int64_t q = blockIdx.x * 128 + 32 * w + 8 * rq + 4 * g + i;
          q = q < nq ? q : nq - 1;
          scores[q * ss + key] = nk * fmaf(rk, acc2[4 * rq + i], acc1[4 * rq + i]) * fr[i];
        }
      }
    } else {
      const float nkm = key_raw < nkeys ? nk : __builtin_nanf("");  // keys past the end never enter
      const int key_base = static_cast<int>(tile * kTileKeys);
      // candidates are rare: one branch for the whole tile
      float uu[16];
      uint64_t any = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        uu[r] = nkm * fmaf(rk, acc2[r], acc1[r]);
        any |= __ballot(uu[r] > pr[r]);
      }
      if (any) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float u = uu[r];
        uint64_t m = __ballot(u > pr[r]);
        while (m) {
          const int j = __ffsll(static_cast<unsigned long long>(m)) - 1;
          m &= m - 1;
          const int gj = j >> 5;
          const float s = read_lane(u, j);
          if (!(s > read_lane(pr[r], j))) continue;  // the threshold rose meanwhile
          const int wr = 8 * (r >> 2) + 4 * gj + (r & 3);  // row within the wave
          float* ls_row = lst_s + wr * top_k;
          int* li_row = lst_i + wr * top_k;
          const bool in = lane < top_k;
          const float ls = in ? ls_row[lane] : -INFINITY;
          const int li = in ? li_row[lane] : -1;
          // entries ahead of the candidate: u at least as high (placeholders
          // hold -inf, below any candidate)
          const int pos = __popcll(__ballot(in && ls >= s));
          // each entry from the lane before (a whole-wave shift by one lane)
          const float ps = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, ls), 0x138, 0xF, 0xF, false));
          const int pi = __builtin_amdgcn_update_dpp(0, li, 0x138, 0xF, 0xF, false);
          const float ns = lane == pos ? s : lane > pos ? ps : ls;
          const int ni = lane == pos ? key_base + (j & 31) : lane > pos ? pi : li;
          if (in && lane >= pos) {
            ls_row[lane] = ns;
            li_row[lane] = ni;
          }
          const float nt = read_lane(ns, top_k - 1);
          if (g == gj) pr[r] = fmaxf(pr[r], nt);
        }
      }
      }
    }
    if constexpr (kTopk) {
      const int64_t done = tile - t0 + 1;
      if (bound && (done & (done < 16 ? done - 1 : 15)) == 0) sync_bounds();
    }
    if constexpr (Fm::kBufs == 1) {
      __syncthreads();  // the tile's rows are no longer read
      if (tile + 1 < t1) {
        expand(nw, stage);
        if (tile + 2 < t1) fetch(tile + 2, nw);
      }
    }
    __syncthreads();
  }
  if constexpr (kTopk) {
    // this block's lists as scores: row q, split blockIdx.y
    const int64_t splits = gridDim.y;
    for (int i = lane; i < 32 * top_k; i += 64) {
      const int wr = i / top_k, e = i - wr * top_k;
      const int64_t q = blockIdx.x * 128 + 32 * w + wr;
      if (q < nq) {
        const int64_t o = ((grp * nq + q) * splits + blockIdx.y) * top_k + e;
        const int key_in = lst_i[i];
        top_s[o] = key_in < 0 ? -INFINITY : lst_s[i] * row_f[32 * w + wr];  // empty: no score
        top_i[o] = key_in < 0 ? INT64_MAX : key_in;
      }
    }
  }
}

template <int B, int F, int KS, bool kTopk>
hipError_t launch_ks(const ScoreArgs& a) {
  const auto kernel = score_mfma_kernel<B, F, KS, kTopk>;
  const size_t dyn = kTopk ? score_list_bytes(a.k) : 0;
  if (dyn > 0) {
    hipFuncAttributes attr{};
    hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel));
    if (e != hipSuccess) return e;
    if (attr.sharedSizeBytes + dyn > size_t(a.h->lds_per_block)) return hipErrorInvalidValue;
    if (attr.sharedSizeBytes + dyn > 65536) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(dyn));
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(a.qtiles), static_cast<uint32_t>(a.splits),
                                  static_cast<uint32_t>(a.groups)),
                     dim3(kThreads), dyn, a.stream, a.vw, vw_stride(a.h->d), vw_half(a.h->d), a.nq, a.codes, a.signs,
                     a.norms, a.rnorms, a.n, a.key_stride, a.scores, a.n, a.form, a.tiles_per_block, a.part_s,
                     a.part_i, a.k, a.bound);
  return hipGetLastError();
}

// LDS bytes of the search form's kernel (static part), or SIZE_MAX
template <int B, int F, int KS>
size_t static_lds_ks() {
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(score_mfma_kernel<B, F, KS, true>)) != hipSuccess)
    return SIZE_MAX;
  return attr.sharedSizeBytes;
}

// the K-step count of the handle's d picks the instantiation
template <int B, int F>
hipError_t launch_form(const ScoreArgs& a) {
  const int ks = (a.h->d + 15) / 16;
#define TQ_SCORE_CASE(K) \
  case K: return a.topk ? launch_ks<B, F, K, true>(a) : launch_ks<B, F, K, false>(a);
  switch (ks) {
    TQ_SCORE_CASE(1) TQ_SCORE_CASE(2) TQ_SCORE_CASE(3) TQ_SCORE_CASE(4)
    TQ_SCORE_CASE(5) TQ_SCORE_CASE(6) TQ_SCORE_CASE(7) TQ_SCORE_CASE(8)
    TQ_SCORE_CASE(9) TQ_SCORE_CASE(10) TQ_SCORE_CASE(11) TQ_SCORE_CASE(12)
    TQ_SCORE_CASE(13) TQ_SCORE_CASE(14) TQ_SCORE_CASE(15) TQ_SCORE_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef TQ_SCORE_CASE
}

template <int B, int F>
size_t static_lds_form(int d) {
  switch ((d + 15) / 16) {
    case 1: return static_lds_ks<B, F, 1>();
    case 2: return static_lds_ks<B, F, 2>();
    case 3: return static_lds_ks<B, F, 3>();
    case 4: return static_lds_ks<B, F, 4>();
    case 5: return static_lds_ks<B, F, 5>();
    case 6: return static_lds_ks<B, F, 6>();
    case 7: return static_lds_ks<B, F, 7>();
    case 8: return static_lds_ks<B, F, 8>();
    case 9: return static_lds_ks<B, F, 9>();
    case 10: return static_lds_ks<B, F, 10>();
    case 11: return static_lds_ks<B, F, 11>();
    case 12: return static_lds_ks<B, F, 12>();
    case 13: return static_lds_ks<B, F, 13>();
    case 14: return static_lds_ks<B, F, 14>();
    case 15: return static_lds_ks<B, F, 15>();
    case 16: return static_lds_ks<B, F, 16>();
    default: return SIZE_MAX;
  }
}

}  // namespace score
}  // namespace tqdev
