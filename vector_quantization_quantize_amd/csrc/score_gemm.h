// Matrix-core scorer for many queries against packed keys, d > 256.
//
// Same estimator and level-value forms as score_mfma.h ("TurboQuant
// digest" section 2; "TurboQuant deep review", error-compensation section):
//     score = n * ( <v, c[idx]> + rho * sqrt(pi/2) / d * <w, 2 beta - 1> ),
// computed as u = n (acc_v + rho acc_w), score = (gamma / s_R) u, with each
// query row's v and lambda w scaled by one power of two s_R.  With d > 256
// the query rows no longer fit in registers, so this is a plain tiled
// product: a block takes 128 queries x 128 keys and both operands go through
// LDS 16 coordinates (one K step) at a time, double-buffered.  The block's 8
// waves split the work: 4 multiply (wave (wm, wn): 64 x 64, 2 x 2
// matrix-core tiles of 32 x 32 x 16 f16, holding only accumulators and
// fragments, so a step's fragment reads all issue before its matrix-core
// passes), 4 load and stage the next step (with both roles in one wave,
// register pressure had the compiler reload fragments one pass at a time,
// each pass waiting out an LDS round trip):
//   * queries: float16 rows pre-scaled once per call (query_f16_kernel) and
//     stored K-major by 128-row tile, so that one step of a tile (128 rows x
//     v, w x 16 coordinates, 8 KB) is contiguous: two 16-byte loads per
//     thread per step, fully coalesced;
//   * keys: every 8 steps the block moves the next 4 words of each of its
//     128 keys' bit planes (one 16-byte load per key and plane, issued 8
//     steps ahead) into a raw LDS buffer; per step thread (key, byte)
//     expands 8 coordinates from it:
//     signs with integer ops (bit -> sign bit of +-1), level values through
//     an LDS table indexed by packed index bits.  (Per-step 4-byte loads of
//     one word per key and plane had every lane on its own cache line: the
//     loads, not the matrix cores, set the pace.)
// Per step a wave reads 4 + 2P 16-byte fragments per lane (P = 2 or 3
// staged planes) for 4P matrix-core passes.
//
// The epilogue runs once per 128 x 128 x d tile.  Scores form: store.
// Search form ("TurboQuant digest" section 3: the k best keys per query):
// the block keeps per query row the k best (u, key) in LDS; the waves of a
// row group insert their candidates in turn (a barrier between), and the
// block shares its rows' k-th scores with the other blocks walking the same
// queries through an atomic max (a lower bound of each query's k-th best).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "score_mfma.h"

namespace tqdev {
namespace gemm {

using score::f16x8;
using score::f32x16;

constexpr int kMmaWaves = 4;                 // waves that multiply (the other 4 load and stage)
constexpr int kThreads = 2 * kMmaWaves * 64;
constexpr int kBM = 128;   // queries per block
constexpr int kBN = 128;   // keys per tile
constexpr int kRow = 24;   // staged row: 16 coordinates + 8 pad halves (3 chunks: conflict-free b128 reads)
constexpr int kBlocksPerCu = 1;
constexpr int kAhead = 6;  // steps of query chunks the producers load ahead

struct Chunks {  // a producer thread's two 16-byte query chunks of one step
  uint4 x, y;
};


// per query row: v and lambda w scaled by s_R (negated where they meet
// staged signs), float16, zero-padded to kp; rows past nq (up to whole
// 128-row tiles) repeat the last query, so that the scores form's clamped
// stores for them write the same values; the row's score factor.  Layout:
// [group][tile][step][row 128][v, w][16].
template <int F>
__global__ void __launch_bounds__(256)
query_f16_kernel(const float* __restrict__ vw, int64_t vw_stride, int64_t vw_half, int d, int kp, int64_t nq,
                 int64_t qtiles, int64_t rows, ScoreForm fp, _Float16* __restrict__ qa, float* __restrict__ row_f) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // over groups x qtiles x 128
  if (row >= rows) return;
  const int64_t grp = row / (qtiles * kBM), rt = row % (qtiles * kBM), tile = rt / kBM, r = rt % kBM;
  const int64_t q = tile * kBM + r, qs = q < nq ? q : nq - 1;
  const int ks = kp / 16;
  _Float16* out = qa + ((grp * qtiles + tile) * ks * kBM + r) * 32;  // step t at + t * kBM * 32
  const float* v = vw + (grp * nq + qs) * vw_stride;
  const float* w = v + vw_half;
  float ssv = 0.0f, ssw = 0.0f;
  for (int i = lane; i < d; i += 64) {
    ssv = fmaf(v[i], v[i], ssv);
    ssw = fmaf(w[i], w[i], ssw);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ssv += __shfl_xor(ssv, o);
    ssw += __shfl_xor(ssw, o);
  }
  float sr = 1.0f;
  const float m = fmaxf(sqrtf(ssv), fp.lambda * sqrtf(ssw));
  if (m > 0.0f && m < INFINITY) {
    int e = 0;
    (void)frexpf(m, &e);
    sr = ldexpf(1.0f, 10 - e);  // m * sr in [2^9, 2^10)
  }
  const float sv = F == kSignForm ? -sr : sr, sw = -sr * fp.lambda;
  for (int i = lane; i < kp; i += 64) {
    out[(i / 16) * kBM * 32 + (i % 16)] = static_cast<_Float16>(i < d ? v[i] * sv : 0.0f);
    out[(i / 16) * kBM * 32 + 16 + (i % 16)] = static_cast<_Float16>(i < d ? w[i] * sw : 0.0f);
  }
  if (lane == 0 && q < nq) row_f[grp * nq + q] = fp.gamma / sr;
}

template <int B, int F, bool kTopk>
__global__ void __launch_bounds__(kThreads, kBlocksPerCu)
score_gemm_kernel(const _Float16* __restrict__ qa, const float* __restrict__ row_fg, int64_t nq, int kp,
                  const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
                  const float* __restrict__ norms, const float* __restrict__ rnorms, int words, int64_t nkeys,
                  int64_t key_stride, float* __restrict__ scores, int64_t sstride, ScoreForm fp,
                  int64_t tiles_per_block, float* __restrict__ top_s, int64_t* __restrict__ top_i, int top_k,
                  unsigned int* __restrict__ bound) {
  using Fm = score::Form<B, F>;
  constexpr int E = Fm::E;
  constexpr int P = Fm::kPlanes;
  constexpr int kRawWords = (B + 1) * 4 * kBN;
  __shared__ uint4 sA4[2][2][kBM * kRow / 8];  // [buf][v, w][row][kRow]
  __shared__ uint4 sB4[2][P][kBN * kRow / 8];  // [buf][plane][key][kRow]
  __shared__ uint32_t raw[2][kRawWords];       // [group parity][index planes, sign plane][4 words][key]
  __shared__ _Float16 vtab[F == kSignForm ? 8 : Fm::kEntries * Fm::kHalves];
  __shared__ __align__(16) float row_f[kBM];
  __shared__ __align__(16) float row_t[kBM];  // search form: the row's threshold (u units)
  extern __shared__ float lst_all[];          // search form: [128][k] u, then [128][k] keys

  // waves 0-3 multiply (wave (wm, wn): rows 64 wm .., keys 64 wn ..); waves
  // 4-7 load and stage (producer thread pt)
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kl = lane & 31, g = lane >> 5;
  const bool producer = w >= kMmaWaves;
  const int wm = w & 1, wn = (w >> 1) & 1, pt = tid - kMmaWaves * 64;
  const int64_t grp = blockIdx.z;
  const int64_t q0 = int64_t(blockIdx.x) * kBM;
  const int ks = kp / 16;
  const int64_t qtiles = gridDim.x;
  qa += (grp * qtiles + blockIdx.x) * int64_t(ks) * kBM * 32;  // this tile's steps, 8 KB each
  row_fg += grp * nq;
  codes += grp * key_stride * B * words;
  signs += grp * key_stride * words;
  norms += grp * key_stride;
  rnorms += grp * key_stride;
  if constexpr (!kTopk) scores += grp * nq * sstride;

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
  if (tid < kBM) {
    const int64_t q = q0 + tid;
    row_f[tid] = row_fg[q < nq ? q : nq - 1];
    if constexpr (kTopk) row_t[tid] = q < nq ? -INFINITY : INFINITY;
  }
  float* lst_s = lst_all;
  int* lst_i = reinterpret_cast<int*>(lst_all + kBM * top_k);
  if constexpr (kTopk) {
    for (int i = tid; i < kBM * top_k; i += kThreads) {
      lst_s[i] = -INFINITY;
      lst_i[i] = -1;
    }
  }

  const int64_t ntiles = (nkeys + kBN - 1) / kBN;
  const int64_t t0 = blockIdx.y * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < ntiles ? t0 + tiles_per_block : ntiles;
  const int64_t steps = (t1 > t0 ? t1 - t0 : 0) * ks;

  // ---- producers.  Per step: query chunks c = pt and pt + 256 of the step's
  // 8 KB (row c / 4, part (c / 2) % 2, half c % 2), and key byte (key pt %
  // 128, byte pt / 128).  Steps come in groups of 8 (4 packed words); a
  // group's words sit in raw[group parity].  At a group's first step the
  // producers move the next group's words (loaded a group ago: 16 bytes per
  // key and plane, items i = pt, pt + 256, ...: plane i / 128, key i % 128)
  // into the other parity, last read a group ago, and start loading the
  // group after.  Positions advance by counters.
  constexpr int kItems = kBN * (B + 1);
  constexpr int kRawPer = (kItems + 255) / 256;
  const int skey = pt & (kBN - 1), sbyte = pt >> 7;
  int aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = pt + 256 * i, row = c >> 2, part = (c >> 1) & 1, half = c & 1;
    aoff[i] = part * kBM * kRow + row * kRow + 8 * half;
  }
  // query chunks of the next 6 steps: a ring of six named slots, passed by
  // value (slots whose address is taken, or an array of them, end up in
  // scratch memory)
  Chunks pa0, pa1, pa2, pa3, pa4, pa5;
  uint4 rb[kRawPer];
  int64_t r_tile = t0;  // next group to load: tile r_tile, first step r_t
  int r_t = 0;
  auto load_raw = [&]() __attribute__((always_inline)) {
    const int w0 = r_t >> 1;
    if (r_tile < t1) {
#pragma unroll
      for (int j = 0; j < kRawPer; ++j) {
        const int item = pt + 256 * j;
        if (item < kItems) {
          const int kk = item % kBN, p = item / kBN;
          int64_t key = r_tile * kBN + kk;
          key = key < nkeys ? key : nkeys - 1;
          const uint32_t* src = p < B ? codes + (key * B + p) * words : signs + key * words;
          if (w0 + 4 <= words) {
            rb[j] = *reinterpret_cast<const uint4*>(src + w0);
          } else {  // the row's last, partial group of words
            rb[j].x = w0 < words ? src[w0] : 0u;
            rb[j].y = w0 + 1 < words ? src[w0 + 1] : 0u;
            rb[j].z = w0 + 2 < words ? src[w0 + 2] : 0u;
            rb[j].w = 0u;
          }
        }
      }
    }
    r_t += 8;
    if (r_t >= ks) {
      r_t = 0;
      ++r_tile;
    }
  };
  auto put_raw = [&](int parity) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kRawPer; ++j) {
      const int item = pt + 256 * j;
      if (item < kItems) {
        uint32_t* dst = raw[parity] + (item / kBN) * 4 * kBN + (item % kBN);
        dst[0] = rb[j].x;
        dst[kBN] = rb[j].y;
        dst[2 * kBN] = rb[j].z;
        dst[3 * kBN] = rb[j].w;
      }
    }
  };
  int f_t = 0;  // step within its tile of the next step to fetch
  // ring of kAhead steps: step s's chunks in slot s % kAhead; slots are
  // fixed by the unrolled loop below (a shifted ring would make every move
  // wait for its load), and every helper is inlined so that the ring stays
  // in registers
  auto fetch = [&]() __attribute__((always_inline)) {
    const _Float16* ap = qa + int64_t(f_t) * kBM * 32;
    Chunks c;
    c.x = *reinterpret_cast<const uint4*>(ap + 8 * pt);
    c.y = *reinterpret_cast<const uint4*>(ap + 8 * (pt + 256));
    if (++f_t == ks) f_t = 0;
    return c;
  };
  uint32_t sgn_mask = 0x80008000u, sgn_one = 0x3C003C00u;
  asm volatile("" : "+v"(sgn_mask), "+v"(sgn_one));
  int s_t = 0;  // step within its tile of the next step to stage
  int sg = 0;   // parity of its group
  auto stage = [&](int buf, Chunks src) __attribute__((always_inline)) {
    if ((s_t & 7) == 0) {
      put_raw(sg ^ 1);
      load_raw();
    }
    _Float16* a = reinterpret_cast<_Float16*>(sA4[buf]);
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(a + aoff[i]) = i == 0 ? src.x : src.y;
    const int rbyte = 4 * ((s_t & 7) >> 1) + 2 * (s_t & 1) + sbyte;  // byte of the key's 16-byte group
    const uint32_t* rw = raw[sg] + (rbyte >> 2) * kBN + skey;
    uint32_t pw[B + 1];
#pragma unroll
    for (int p = 0; p <= B; ++p) pw[p] = __builtin_amdgcn_ubfe(rw[p * 4 * kBN], 8 * (rbyte & 3), 8);
    _Float16* b = reinterpret_cast<_Float16*>(sB4[buf]) + skey * kRow + 8 * sbyte;
    if constexpr (F == kSignForm) {
      *reinterpret_cast<uint4*>(b) = score::expand_signs(pw[0], sgn_mask, sgn_one);
    } else {
      _Float16 hv[8], lv[8];
#pragma unroll
      for (int k = 0; k < 8 / E; ++k) {
        uint32_t idx = 0;
#pragma unroll
        for (int p = 0; p < B; ++p) idx |= __builtin_amdgcn_ubfe(pw[p], k * E, E) << (p * E);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          hv[k * E + e] = vtab[idx * Fm::kHalves + e];
          if constexpr (F == kTwoPiece) lv[k * E + e] = vtab[idx * Fm::kHalves + E + e];
        }
      }
      *reinterpret_cast<f16x8*>(b) = f16x8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
      if constexpr (F == kTwoPiece)
        *reinterpret_cast<f16x8*>(b + kBN * kRow) = f16x8{lv[0], lv[1], lv[2], lv[3], lv[4], lv[5], lv[6], lv[7]};
    }
    *reinterpret_cast<uint4*>(b + (P - 1) * kBN * kRow) = score::expand_signs(pw[B], sgn_mask, sgn_one);
    if (++s_t == ks) s_t = 0;
    if ((s_t & 7) == 0) sg ^= 1;  // the next step starts a group
  };

  __syncthreads();  // table, row factors, lists
  // The two roles run separate loops (so that their registers need not
  // coexist) with the same barriers: one per step, and in the search form
  // two more at the end of each key tile.
  int c_t = 0;          // step within the current tile
  int64_t c_tile = t0;  // current tile
  if (producer) {
    if (steps > 0) {
      load_raw();  // group 0
      put_raw(0);
      load_raw();  // group 1
      pa0 = fetch();
      pa1 = fetch();
      pa2 = fetch();
      pa3 = fetch();
      pa4 = fetch();
      pa5 = fetch();
    }
    __syncthreads();  // group 0's words
    if (steps > 0) {
      stage(0, pa0);
      pa0 = fetch();
    }
    __syncthreads();
    // iteration it: step it + 1 into buffer (it + 1) % 2 from slot
    // (it + 1) % kAhead, which then takes step it + 1 + kAhead (past the
    // last step this stages into the buffer no one reads and fetches a
    // valid address); kAhead even, so it's parity is the unrolled index's
    static_assert(kAhead == 6, "six named slots");
#define TQ_PRODUCER_STEP(D, PAR, SLOT)  \
  if (it0 + (D) < steps) {              \
    stage(PAR, SLOT);                   \
    SLOT = fetch();                     \
    if (++c_t == ks) {                  \
      c_t = 0;                          \
      if constexpr (kTopk) {            \
        __syncthreads();                \
        __syncthreads();                \
      }                                 \
    }                                   \
    __syncthreads();                    \
  }
    for (int64_t it0 = 0; it0 < steps; it0 += kAhead) {
      TQ_PRODUCER_STEP(0, 1, pa1)
      TQ_PRODUCER_STEP(1, 0, pa2)
      TQ_PRODUCER_STEP(2, 1, pa3)
      TQ_PRODUCER_STEP(3, 0, pa4)
      TQ_PRODUCER_STEP(4, 1, pa5)
      TQ_PRODUCER_STEP(5, 0, pa0)
    }
#undef TQ_PRODUCER_STEP
  } else {
    __syncthreads();
    __syncthreads();
    f32x16 acc1[2][2], acc2[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc1[i][j] = acc2[i][j] = f32x16{};
    for (int64_t it = 0; it < steps; ++it) {
      const int buf = static_cast<int>(it & 1);
      const _Float16* a = reinterpret_cast<const _Float16*>(sA4[buf]);
      const _Float16* b = reinterpret_cast<const _Float16*>(sB4[buf]);
      f16x8 fv[2], fw[2], fb[P][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int off = (64 * wm + 32 * i + kl) * kRow + 8 * g;
        fv[i] = *reinterpret_cast<const f16x8*>(a + off);
        fw[i] = *reinterpret_cast<const f16x8*>(a + kBM * kRow + off);
      }
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[p][j] = *reinterpret_cast<const f16x8*>(b + p * kBN * kRow + (64 * wn + 32 * j + kl) * kRow + 8 * g);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc1[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fv[i], fb[0][j], acc1[i][j], 0, 0, 0);
          acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fw[i], fb[P - 1][j], acc2[i][j], 0, 0, 0);
        }
      if constexpr (F == kTwoPiece) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc1[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fv[i], fb[1][j], acc1[i][j], 0, 0, 0);
      }
      if (++c_t == ks) {
        c_t = 0;
        // the tile's scores: element r of tile (i, j) is query row
        // 64 wm + 32 i + 8 (r / 4) + 4 g + r % 4, key 64 wn + 32 j + kl
        const int64_t tile = c_tile++;
        float nk[2], rk[2];
        bool kin[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          int64_t key = tile * kBN + 64 * wn + 32 * j + kl;
          kin[j] = key < nkeys;
          key = kin[j] ? key : nkeys - 1;
          nk[j] = norms[key];
          rk[j] = rnorms[key];
        }
        if constexpr (!kTopk) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int lr = 64 * wm + 32 * i + 8 * rq + 4 * g;
              const float4 f = *reinterpret_cast<const float4*>(row_f + lr);
              const float fr[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                int64_t key = tile * kBN + 64 * wn + 32 * j + kl;
                key = key < nkeys ? key : nkeys - 1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  int64_t q = q0 + lr + e;
                  q = q < nq ? q : nq - 1;
                  const int r = 4 * rq + e;
                  scores[q * sstride + key] = nk[j] * fmaf(rk[j], acc2[i][j][r], acc1[i][j][r]) * fr[e];
                }
              }
            }
        } else {
          // waves wn = 0, then wn = 1, insert into the block's row lists
#pragma unroll 1
          for (int ph = 0; ph < 2; ++ph) {
            if (wn == ph) {
#pragma unroll
              for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                  for (int rq = 0; rq < 4; ++rq) {
                    const int lr = 64 * wm + 32 * i + 8 * rq + 4 * g;
                    const float4 tv = *reinterpret_cast<const float4*>(row_t + lr);
                    const float th[4] = {tv.x, tv.y, tv.z, tv.w};
                    const float nkm = kin[j] ? nk[j] : __builtin_nanf("");
                    float uu[4];
                    uint64_t any = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                      uu[e] = nkm * fmaf(rk[j], acc2[i][j][4 * rq + e], acc1[i][j][4 * rq + e]);
                      any |= __ballot(uu[e] > th[e]);
                    }
                    if (!any) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                      uint64_t m = __ballot(uu[e] > th[e]);
                      while (m) {
                        const int jl = __ffsll(static_cast<unsigned long long>(m)) - 1;
                        m &= m - 1;
                        const float sc = score::read_lane(uu[e], jl);
                        const int R = 64 * wm + 32 * i + 8 * rq + 4 * (jl >> 5) + e;
                        if (!(sc > row_t[R])) continue;  // the threshold rose meanwhile
                        float* ls_row = lst_s + R * top_k;
                        int* li_row = lst_i + R * top_k;
                        const bool in = lane < top_k;
                        const float ls = in ? ls_row[lane] : -INFINITY;
                        const int li = in ? li_row[lane] : -1;
                        const int pos = __popcll(__ballot(in && ls >= sc));
                        const float ps = __builtin_bit_cast(
                            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, ls), 0x138, 0xF, 0xF, false));
                        const int pi = __builtin_amdgcn_update_dpp(0, li, 0x138, 0xF, 0xF, false);
                        const float ns = lane == pos ? sc : lane > pos ? ps : ls;
                        const int ni = lane == pos ? static_cast<int>(tile * kBN + 64 * wn + 32 * j + (jl & 31))
                                                   : lane > pos ? pi : li;
                        if (in && lane >= pos) {
                          ls_row[lane] = ns;
                          li_row[lane] = ni;
                        }
                        const float nt = score::read_lane(ns, top_k - 1);
                        if (lane == 0) row_t[R] = fmaxf(row_t[R], nt);
                      }
                    }
                  }
            }
            __syncthreads();
          }
          // share the rows' k-th scores with the other blocks walking these
          // queries; read back the best as a bound (a little low in u units)
          if (bound && wn == 0) {
            const int lr = 64 * wm + lane;
            const int64_t q = q0 + lr;
            if (q < nq) {
              const float mine = lst_s[lr * top_k + top_k - 1] * row_f[lr];
              const unsigned int e = score::enc_score(mine);
              const unsigned int old = atomicMax(bound + grp * nq + q, e);
              const float best = score::dec_score(old > e ? old : e);
              if (best > -INFINITY && best < INFINITY) {
                const float tu = best / row_f[lr];
                row_t[lr] = fmaxf(row_t[lr], tu - fabsf(tu) * 0x1p-20f);
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc1[i][j] = acc2[i][j] = f32x16{};
      }
      __syncthreads();
    }
  }
  if constexpr (kTopk) {
    const int64_t splits = gridDim.y;
    for (int i = tid; i < kBM * top_k; i += kThreads) {
      const int lr = i / top_k, e = i - lr * top_k;
      const int64_t q = q0 + lr;
      if (q < nq) {
        const int64_t o = ((grp * nq + q) * splits + blockIdx.y) * top_k + e;
        const int key_in = lst_i[i];
        top_s[o] = key_in < 0 ? -INFINITY : lst_s[i] * row_f[lr];
        top_i[o] = key_in < 0 ? INT64_MAX : key_in;
      }
    }
  }
}

template <int B, int F, bool kTopk>
hipError_t launch(const ScoreArgs& a) {
  const auto kernel = score_gemm_kernel<B, F, kTopk>;
  const size_t dyn = kTopk ? size_t(kBM) * size_t(a.k) * (sizeof(float) + sizeof(int)) : 0;
  hipFuncAttributes attr{};
  hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel));
  if (e != hipSuccess) return e;
  if (attr.sharedSizeBytes + dyn > size_t(a.h->lds_per_block)) return hipErrorInvalidValue;
  if (attr.sharedSizeBytes + dyn > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(dyn));
    if (e != hipSuccess) return e;
  }
  const int kp = (a.h->d + 15) / 16 * 16;
  const int64_t rows = a.groups * a.qtiles * kBM;
  if ((rows + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(query_f16_kernel<F>, dim3(static_cast<uint32_t>((rows + 3) / 4)), dim3(256), 0, a.stream, a.vw,
                     vw_stride(a.h->d), vw_half(a.h->d), a.h->d, kp, a.nq, a.qtiles, rows, a.form,
                     static_cast<_Float16*>(a.qa), a.row_f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(a.qtiles), static_cast<uint32_t>(a.splits),
                                  static_cast<uint32_t>(a.groups)),
                     dim3(kThreads), dyn, a.stream, static_cast<const _Float16*>(a.qa), a.row_f, a.nq, kp, a.codes, a.signs, a.norms, a.rnorms,
                     a.h->words, a.n, a.key_stride, a.scores, a.n, a.form, a.tiles_per_block, a.part_s, a.part_i, a.k,
                     a.bound);
  return hipGetLastError();
}

template <int B, int F>
hipError_t launch_form(const ScoreArgs& a) {
  return a.topk ? launch<B, F, true>(a) : launch<B, F, false>(a);
}

template <int B, int F>
size_t static_lds() {
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(score_gemm_kernel<B, F, true>)) != hipSuccess)
    return SIZE_MAX;
  return attr.sharedSizeBytes;
}

}  // namespace gemm
}  // namespace tqdev
