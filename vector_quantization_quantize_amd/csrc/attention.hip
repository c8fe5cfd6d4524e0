// Decode attention over a compressed cache, and the value layout it reads.
//
// The cache holds key-value pairs ("Why KV-cache compression works",
// section 2); keys are scored by the asymmetric estimate (tq_logits), values
// are stored with stage 1 only and read back through the stage-1
// reconstruction v_hat = n_v Pi^T c[idx_v] ("TurboQuant tutorial", end of
// the polar part).  Per query
//     o = sum_t softmax_t(scale s_t) v_hat_t = Pi^T ( sum_t p_t n_t c[idx_t] ),
// so the weighted sum runs in the rotated domain, over the stored levels,
// and the rotation back is one d x d product per query at the end.
//
// Value layout (token blocks): vcodes[group][ceil(n/32)][B][32 W] uint32.
// For plane p of block b, the token word T_c of coordinate c has bit i =
// bit p of the index of coordinate c of token 32 b + i: the contraction
// over tokens is the matrix-core K dimension, and one byte of T_c is the
// operand of 8 tokens for one coordinate, expanded without a bit transpose.
// The bits are stored in the order the value pass's lanes read them: the
// planes of one coordinate and token octet are interleaved so that each
// run of B E bits is a level-table index for E tokens, and within each
// group of 128 coordinates lane L finds its octet's integers for
// coordinates L mod 16 + 16 j (j < 8) contiguous, so a tile costs one
// 8 B-byte read per lane, no byte read twice, and one bit-field extract
// per table lookup.
//
// Kernels:
//  * pack_values_kernel: key-layout codes -> token blocks (a 32 x 32 bit
//    transpose per word by wave ballots, then the planes interleaved).
//  * attn_pv_kernel: one wave per (key split, group of 4 words = 128
//    coordinates, group, up to 16 query rows), with no block-wide barrier
//    after the level table.  A first pass over the split's norms finds the
//    largest (weights are scaled by a power of two so that they fit
//    float16); then the wave walks 32-token tiles with the next two tiles'
//    scores, norms and value words already loading, keeping running row
//    maxima (online softmax: sums so far are rescaled when a maximum
//    grows).  Weights p = exp(scale s - max) n / 2^e go through the wave's
//    own LDS slice as two float16 pieces (22 bits), and per word the wave
//    expands its levels (the scorer's level forms) and runs
//    v_mfma_f32_16x16x32_f16: 16 query rows x 32 tokens x 16 coordinates
//    per pass.  Writes the split's (max, sum of exp) per row and its
//    partial sums per coordinate.
//  * attn_merge_kernel: per (group, query): combines the splits (rescaled to
//    the overall max), divides by the sum, and applies Pi^T.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "lut_tables.h"
#include "score_mfma.h"
#include "tq_internal.h"

namespace tqdev {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
using score::f16x8;

constexpr int kRows = 16;   // query rows per block (matrix-core M)
constexpr int kTile = 32;   // tokens per tile (matrix-core K; one word of a value plane)
constexpr int kWaves = 4;   // waves per block, each on its own key split
constexpr int kWordsPerWave = 4;  // 32-coordinate words per wave (128 coordinates)
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSplits = 1024;
constexpr float kSlack = 8.0f;  // weights relative to a row's reference maximum stay <= 2^kSlack

// ---------------------------------------------------------------------------
// value packing
// ---------------------------------------------------------------------------

// Tokens per index run in the value layout (the level forms' table width)
__host__ __device__ constexpr int value_e(int B) { return B == 1 ? 8 : B == 2 ? 4 : 2; }

// Byte offset, within a block, of the B-byte integer X of coordinate c and
// token octet o: coordinates come in groups of 128 (4 key-layout words; the
// last group has G = W mod 4 words when that is not 0), group g starts at
// byte 512 B g, and (r = c mod 128) X sits at ((r mod 16) + 16 o) 2 G B +
// (r div 16) B.  Lane L of the value pass (L mod 16 = r mod 16, L div 16 =
// o) then finds its 2 G integers contiguous at 2 G B L.  X holds, for token
// 8 o + t and plane p, bit p of the index at bit (t div E) B E + p E +
// (t mod E): each run of B E bits indexes the level table for E tokens.
__device__ __forceinline__ int value_slot(int c, int o, int W, int B) {
  const int g = c >> 7, r = c & 127;
  const int gw = W - 4 * g < 4 ? W - 4 * g : 4;
  return 512 * B * g + ((r & 15) + 16 * o) * 2 * gw * B + (r >> 4) * B;
}

// block (token block, group).  Phase 1: the token words T of every plane
// and coordinate (bit i = bit p of the index of coordinate c of token
// 32 b + i) into LDS, by wave ballots over key-layout words: lanes 0-31
// hold word `pw` of tokens 0-31, lanes 32-63 word `pw + 1`, ballot j
// collects bit j of each half.  Phase 2: thread per (coordinate, token
// octet) interleaves the planes' bytes into X and writes its B bytes.
// Dynamic LDS: B * 32 W words.
// B is a template argument so that the interleave below unrolls with
// constant shifts; each token block's 128 B W output bytes are assembled in
// LDS and leave with 16-byte stores (a block is 16-byte aligned: the
// caller's buffer is, and 128 B W is a multiple of 16).  A workgroup takes
// TB consecutive token blocks and issues their loads together, so that the
// load latency is paid once per TB blocks.
template <int B, int TB>
__global__ void __launch_bounds__(kThreads)
pack_values_kernel(const uint32_t* __restrict__ codes, int64_t n, int W, int64_t nb, uint32_t* __restrict__ vcodes) {
  extern __shared__ uint32_t tw[];  // [TB][B][32 W] transposed planes, then [TB][B][32 W] output staging
  const int bw = B * 32 * W;        // words per token block
  uint8_t* stage = reinterpret_cast<uint8_t*>(tw + TB * bw);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t blk0 = int64_t(blockIdx.x) * TB, grp = blockIdx.y;
  const int pws = B * W;  // words per token in the key layout
  codes += grp * n * pws;
  for (int pw = 2 * wave; pw < pws; pw += 2 * kWaves) {
    const int mine = pw + (lane >> 5);
    uint32_t x[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int64_t tok = (blk0 + tb) * 32 + (lane & 31);  // past n (and past the last block): zero
      x[tb] = (mine < pws && tok < n) ? codes[tok * pws + mine] : 0u;
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      uint32_t t = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint64_t m = __ballot((x[tb] >> j) & 1u);
        const uint32_t part = lane < 32 ? uint32_t(m) : uint32_t(m >> 32);
        t = (lane & 31) == j ? part : t;
      }
      if (mine < pws) {
        const int p = mine / W, w = mine % W;
        tw[tb * bw + p * 32 * W + 32 * w + (lane & 31)] = t;
      }
    }
  }
  __syncthreads();
  constexpr int E = value_e(B);
  for (int i = threadIdx.x; i < TB * 4 * 32 * W; i += kThreads) {
    const int tb = i / (128 * W), ii = i - tb * 128 * W;
    const int c = ii >> 2, o = ii & 3;
    const uint32_t* src = tw + tb * bw;
    uint32_t x = 0;
#pragma unroll
    for (int p = 0; p < B; ++p) {
      const uint32_t byte = (src[p * 32 * W + c] >> (8 * o)) & 0xFFu;
#pragma unroll
      for (int t = 0; t < 8; ++t) x |= ((byte >> t) & 1u) << ((t / E) * B * E + p * E + (t % E));
    }
    uint8_t* dst = stage + size_t(tb) * 4 * bw + value_slot(c, o, W, B);
#pragma unroll
    for (int k = 0; k < B; ++k) dst[k] = uint8_t(x >> (8 * k));
  }
  __syncthreads();
  // the blocks that exist, as one contiguous run of 16-byte words
  const int64_t blocks = nb - blk0 < TB ? nb - blk0 : TB;
  uint4* out = reinterpret_cast<uint4*>(vcodes + (grp * nb + blk0) * int64_t(bw));
  const uint4* st4 = reinterpret_cast<const uint4*>(stage);
  for (int64_t i = threadIdx.x; i < blocks * 8 * B * W; i += kThreads) out[i] = st4[i];
}

// ---------------------------------------------------------------------------
// weighted sum of the stored levels
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// one 32-token tile of a wave's inputs: its share of the scores (pairs
// lane + 64 k: row (lane + 64 k) / 32, token lane % 32), the token's norm,
// and per plane the lane's 2 G value bytes (byte j: tokens 8 (lane / 16) ..
// + 7 of coordinate 16 j + lane % 16 of its group); passed by value so that
// the prefetch stays in registers
template <int B, int RQ, int G>
struct TileIn {
  float s[RQ * kTile / 64];
  float nv;
  uint32_t w[(2 * G * B + 3) / 4];  // the lane's 2 G integers X (B bytes each)
};

// bits [pos, pos + width) of a little-endian multi-word value
template <int N>
__device__ __forceinline__ uint32_t bit_field(const uint32_t (&w)[N], int pos, int width) {
  const int i = pos >> 5, sh = pos & 31;
  if (sh + width <= 32) return __builtin_amdgcn_ubfe(w[i], sh, width);
  return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[i + 1], w[i], sh), 0, width);
}

// RQ: query rows per wave (4, 8 or 16; the matrix-core M is 16 either way,
// rows past RQ stay 0).  G: words in the wave's coordinate group (4, or
// W mod 4 for the last group); the group starts at word word_base + 4
// blockIdx.y.  Blocks with blockIdx.y = 0 of the launch that has write_ml
// set write the (max, sum) of each row.
template <int B, int F, int RQ, int G>
__global__ void __launch_bounds__(kThreads)
attn_pv_kernel(const float* __restrict__ scores, int64_t nq, int64_t n, const uint32_t* __restrict__ vcodes,
               const float* __restrict__ vnorms, int W, int word_base, bool write_ml, float scale, int64_t tps,
               int qchunks, ScoreForm fp, float* __restrict__ part_y, float2* __restrict__ part_ml,
               int64_t splits) {
  using Fm = score::Form<B, F>;
  constexpr int E = Fm::E;
  constexpr int kPairs = RQ * kTile / 64;  // (row, token) weights per lane per tile
  __shared__ _Float16 vtab[F == kSignForm ? 8 : Fm::kEntries * Fm::kHalves];
  __shared__ __align__(16) _Float16 pa[kWaves][2][kRows][kTile];  // per wave: [hi, lo][row][token]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t split = int64_t(blockIdx.x) * kWaves + wave;
  const int word0 = word_base + kWordsPerWave * blockIdx.y;
  const int64_t grp = blockIdx.z / qchunks;
  const int64_t q0 = int64_t(blockIdx.z % qchunks) * RQ;
  const int rows = nq - q0 < RQ ? int(nq - q0) : RQ;
  const int64_t nb = (n + kTile - 1) / kTile;
  const int dp = 32 * W;
  scores += (grp * nq + q0) * n;
  vnorms += grp * n;
  vcodes += grp * nb * B * dp;

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
  // rows past nq keep weight 0 for the whole kernel
  for (int i = lane; i < 2 * kRows * kTile; i += 64) (&pa[wave][0][0][0])[i] = static_cast<_Float16>(0.0f);
  __syncthreads();  // the table; the only block-wide barrier
  if (split >= splits) return;
  // the split's token range is the same in every lane: scalar registers
  const int64_t t0 = (int64_t(__builtin_amdgcn_readfirstlane(int(split))) * tps);
  const int64_t t1r = t0 + tps < n ? t0 + tps : n;
  const int64_t t1 = int64_t(__builtin_amdgcn_readfirstlane(int(t1r >> 32))) << 32 |
                     uint32_t(__builtin_amdgcn_readfirstlane(int(t1r & 0xFFFFFFFF)));

  // ---- 32-token tiles, inputs loaded two tiles ahead
  const int n16 = lane & 15, g16 = lane >> 4, tl = lane & 31;
  // every load is unconditional from a clamped, valid address (a tile past
  // the split reloads the first, rows and tokens past the end repeat the
  // last); the arithmetic gives such entries weight 0, so no load waits
  // behind a branch
  auto load = [&](int64_t tb) __attribute__((always_inline)) {
    TileIn<B, RQ, G> x;
    const int64_t tbc = tb < t1 ? tb : t0;
    const int64_t tok = tbc + tl < t1 ? tbc + tl : t1 - 1;
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int r = 2 * k + (lane >> 5);
      x.s[k] = scores[(r < rows ? r : rows - 1) * n + tok];
    }
    x.nv = vnorms[tok];
    // the lane's 2 G B bytes at 2 G B lane of its group (group word0 / 4
    // starts at byte 512 B (word0 / 4) = 128 B word0), loaded in the widest
    // chunks their alignment allows
    constexpr int kBytes = 2 * G * B;
    constexpr int kChunk = kBytes % 16 == 0 ? 16 : kBytes % 8 == 0 ? 8 : kBytes % 4 == 0 ? 4 : 2;
    const uint8_t* q = reinterpret_cast<const uint8_t*>(vcodes + (tbc / kTile) * B * dp) + 128 * B * word0 +
                       kBytes * lane;
#pragma unroll
    for (int c = 0; c < kBytes / kChunk; ++c) {
      if constexpr (kChunk == 16) {
        const uint4 u = *reinterpret_cast<const uint4*>(q + 16 * c);
        x.w[4 * c] = u.x, x.w[4 * c + 1] = u.y, x.w[4 * c + 2] = u.z, x.w[4 * c + 3] = u.w;
      } else if constexpr (kChunk == 8) {
        const uint2 u = *reinterpret_cast<const uint2*>(q + 8 * c);
        x.w[2 * c] = u.x, x.w[2 * c + 1] = u.y;
      } else if constexpr (kChunk == 4) {
        x.w[c] = *reinterpret_cast<const uint32_t*>(q + 4 * c);
      } else {
        const uint32_t h = *reinterpret_cast<const uint16_t*>(q + 2 * c);
        if (c % 2 == 0) x.w[c / 2] = h;
        else x.w[c / 2] |= h << 16;
      }
    }
    return x;
  };
  float lsum[kPairs];
#pragma unroll
  for (int k = 0; k < kPairs; ++k) lsum[k] = 0.0f;
  uint32_t sgn_mask = 0x80008000u, sgn_one = 0x3C003C00u;
  asm volatile("" : "+v"(sgn_mask), "+v"(sgn_one));
  f32x4 acc[2 * G];  // coordinate 32 word0 + 16 j + n16
#pragma unroll
  for (int j = 0; j < 2 * G; ++j) acc[j] = f32x4{};
  // three tiles in flight in a ring of named slots: a slot is refilled with
  // the tile three ahead right after its own tile is used (rotating the
  // slots would move registers whose loads are still landing, which waits
  // for every load in flight)
  TileIn<B, RQ, G> s0 = load(t0), s1 = load(t0 + kTile), s2 = load(t0 + 2 * kTile);
  // (the first tiles' loads are in flight while the norm pass runs)
  // ---- the split's largest norm (weights carry n / 2^e <= 1 times at most
  // 2^kSlack, so their float16 pieces cannot overflow); eight loads in
  // flight per lane
  const float a = scale * 1.4426950408889634f;  // weights are 2^(a s - max)
  float nmax = 0.0f;
  for (int64_t tb = t0; tb < t1; tb += 8 * 64) {
    float nv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t t = tb + 64 * u + lane;
      nv[u] = vnorms[t < t1 ? t : t1 - 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) nmax = fmaxf(nmax, nv[u]);
  }
  nmax = wave_max(nmax);
  int ne = 0;
  if (nmax > 0.0f && nmax < INFINITY) (void)frexpf(nmax, &ne);
  const float nscale = ldexpf(1.0f, -ne);
  // reference row maxima of a s (the same in every lane).  A vector value,
  // not an array: a per-lane choice between two of its elements must stay
  // a select of two registers (an array indexed that way was moved to
  // per-work-item LDS, whose address every wave then computed from the
  // dispatch packet, and that cost more than the tiles of a decode call)
  typedef float rowvec __attribute__((ext_vector_type(RQ)));
  rowvec lm;
#pragma unroll
  for (int r = 0; r < RQ; ++r) lm[r] = -INFINITY;

  auto step = [&](int64_t tb, const TileIn<B, RQ, G> in) __attribute__((always_inline)) {
    // weights of (row 2k + lane / 32, token lane % 32) into this wave's slice;
    // LDS is in order within a wave, so the reads below see these writes
    const float nv = in.nv * nscale;
    const bool tin = tb + tl < t1;
    // online softmax with a reference maximum per row: weights are
    // 2^(a s - ref) <= 2^kSlack, so the reference moves (and what was summed
    // so far is rescaled) only when a score passes it by more than kSlack;
    // one ballot per tile tests that
    float x[kPairs];
    bool over = false;
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int r = 2 * k + (lane >> 5);
      x[k] = tin && r < rows ? a * in.s[k] : -INFINITY;
      over |= x[k] > ((lane >> 5) ? lm[2 * k + 1] : lm[2 * k]) + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      float f[RQ];
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {
        float m = x[k];
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
        const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int rr = 2 * k + e;
          const float nm = fmaxf(lm[rr], e ? hi : lo);
          f[rr] = nm > lm[rr] ? exp2f(lm[rr] - nm) : 1.0f;
          lm[rr] = nm;
        }
      }
#pragma unroll
      for (int k = 0; k < kPairs; ++k) lsum[k] *= (lane >> 5) ? f[2 * k + 1] : f[2 * k];
#pragma unroll
      for (int j = 0; j < 2 * G; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float fr = f[i];
          if constexpr (RQ > 4) fr = g16 == 1 ? f[4 + i] : fr;
          if constexpr (RQ > 8) {
            fr = g16 == 2 ? f[8 + i] : fr;
            fr = g16 == 3 ? f[12 + i] : fr;
          }
          acc[j][i] *= fr;
        }
    }
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int r = 2 * k + (lane >> 5);
      const float w = __builtin_amdgcn_exp2f(x[k] - ((lane >> 5) ? lm[2 * k + 1] : lm[2 * k]));
      const bool use = tin && r < rows;
      lsum[k] += use ? w : 0.0f;
      float p = use ? w * nv : 0.0f;
      // p rounded to float32 once: folded into the float16 conversion, hi
      // would round the exact product and disagree with lo at a tie
      asm volatile("" : "+v"(p));
      const _Float16 hi = static_cast<_Float16>(p);
      pa[wave][0][r][tl] = hi;
      pa[wave][1][r][tl] = static_cast<_Float16>(p - float(hi));
    }
    // A: row n16, tokens 8 g16 .. 8 g16 + 7 (both pieces); B: coordinate
    // 32 word0 + 16 j + n16, the same tokens, from the lane's integer j
    const f16x8 ah = *reinterpret_cast<const f16x8*>(&pa[wave][0][n16][8 * g16]);
    const f16x8 al = *reinterpret_cast<const f16x8*>(&pa[wave][1][n16][8 * g16]);
#pragma unroll
    for (int j = 0; j < 2 * G; ++j) {
      f16x8 bv, bl;
      if constexpr (F == kSignForm) {
        const uint4 sg = score::expand_signs(bit_field(in.w, 8 * B * j, 8), sgn_mask, sgn_one);
        bv = *reinterpret_cast<const f16x8*>(&sg);
      } else {
#pragma unroll
        for (int k = 0; k < 8 / E; ++k) {
          // tokens k E .. k E + E - 1: one run of B E bits is the table index
          const uint32_t idx = bit_field(in.w, 8 * B * j + k * B * E, B * E);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            bv[k * E + e] = vtab[idx * Fm::kHalves + e];
            if constexpr (F == kTwoPiece) bl[k * E + e] = vtab[idx * Fm::kHalves + E + e];
          }
        }
      }
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv, acc[j], 0, 0, 0);
      if constexpr (F == kTwoPiece) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc[j], 0, 0, 0);
    }
  };
  // whole rounds of three tiles: tiles past the split's end carry weight 0
  // (a branch per step would leave the loop head unable to count the loads
  // in flight, and it would wait for all of them)
  for (int64_t tb = t0; tb < t1; tb += 3 * kTile) {
    step(tb, s0);
    s0 = load(tb + 3 * kTile);
    step(tb + kTile, s1);
    s1 = load(tb + 4 * kTile);
    step(tb + 2 * kTile, s2);
    s2 = load(tb + 5 * kTile);
  }

  // ---- partial results of the split (rows 2k + lane / 32 summed over the
  // 32 lanes of each half)
  const int64_t rowbase = grp * nq + q0;
  const float ln2 = 0.6931471805599453f;
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) lsum[k] += __shfl_xor(lsum[k], o);
    const int r = 2 * k + (lane >> 5);
    if (write_ml && blockIdx.y == 0 && tl == 0 && r < rows)
      part_ml[(rowbase + r) * splits + split] = make_float2(((lane >> 5) ? lm[2 * k + 1] : lm[2 * k]) * ln2, lsum[k]);
  }
  // element i of acc[j]: row 4 g16 + i, coordinate 32 word0 + 16 j + n16
  const float f = fp.gamma * ldexpf(1.0f, ne);
#pragma unroll
  for (int j = 0; j < 2 * G; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g16 + i;
      if (r < rows) part_y[((rowbase + r) * splits + split) * dp + 32 * word0 + 16 * j + n16] = acc[j][i] * f;
    }
}

// ---------------------------------------------------------------------------
// fused form: key scores by the byte tables and the value pass in one kernel
// ---------------------------------------------------------------------------
// For d = 128 and a key handle the byte-table scorer takes: a workgroup of 8
// waves takes every token of a chunk of one (group, query quad), builds the
// scorer's tables for its 4 queries (the scorer's prologue), and then each
// wave walks batches of 64 tokens claimed from a counter in LDS: the keys'
// scores (one token per lane, the scorer's lookups), the online softmax
// with a reference maximum per row (as in the value pass), the weights
// p = 2^(a s - ref) n_v / 2^e through the wave's LDS slice as two float16
// pieces, and the value levels of the batch's two 32-token blocks against
// them on v_mfma_f32_16x16x32_f16 (rows 4..15 of the A operand are zero).
// The score matrix never leaves the chip.  The waves' (max, sum, partial
// sums) are combined in LDS into one split per workgroup, in the layout the
// merge kernel reads.
constexpr int kFPro = 512;  // threads that build the tables (the rest join the key loop)

// a wave's inputs for one batch: the lane's key, and per 32-token block the
// lane's 8 VB value bytes (octet lane / 16, coordinates lane % 16 + 16 j)
// and its token's value norm
template <int KB, int VB>
struct FusedIn {
  ltab::Packed<KB> key;
  uint32_t vw[2][2 * VB];
  float vn;
};

// NTH: 512 or 768 threads (2 or 3 waves per SIMD, as the key loop's
// registers allow)
template <int KB, int VB, int VF, int NTH>
__global__ void __launch_bounds__(NTH, 1)
attn_fused_kernel(const float* __restrict__ queries, int quads, int64_t nq, int64_t n, int d,
                  const float* __restrict__ piT, const float* __restrict__ sT, const uint32_t* __restrict__ codes,
                  const uint32_t* __restrict__ signs, const float* __restrict__ norms,
                  const float* __restrict__ rnorms, PlaneExpansion pe, float kappa,
                  const uint32_t* __restrict__ vcodes, const float* __restrict__ vnorms, ScoreForm fp, float scale,
                  int chunks, int64_t keys_per_block, float* __restrict__ part_y, float2* __restrict__ part_ml) {
  using namespace ltab;
  using TT = Terms<KB>;
  constexpr int NT = TT::count;
  using Fm = score::Form<VB, VF>;
  constexpr int E = Fm::E;
  constexpr int kFWaves = NTH / 64;
  constexpr int kParts = kFPro / kDim;   // row slices of the query transform
  constexpr int kPRows = kDim / kParts;  // 32 rows per slice
  constexpr int kWalk = 256 * 2 * 16 * 4 / kFPro;
  constexpr int dp = 128;                   // value coordinates per token block row
  __shared__ __align__(16) unsigned char tabs[kTableBytes];
  // the prologue's queries and vectors, then the waves' weight slices
  __shared__ __align__(16) union {
    struct {
      float4 qs[kDim];
      float vec[2][4][kDim];
    } pro;
    _Float16 pa[kFWaves][2][4][64];  // [wave][hi, lo][row][token of the batch]
  } sh;
  __shared__ _Float16 vtab[VF == kSignForm ? 8 : Fm::kEntries * Fm::kHalves];
  __shared__ float scale_t[2][4];
  __shared__ float wmax[kFWaves][4], wsum[kFWaves][4], nred[kFWaves];
  __shared__ uint32_t next_batch;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t pair = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int64_t grp = pair / quads, q0 = (pair % quads) * 4;
  const int qc = int(nq - q0 < 4 ? nq - q0 : 4);
  const int64_t kbeg = c * keys_per_block;  // a multiple of 64: whole value blocks
  const int64_t kend = kbeg + keys_per_block < n ? kbeg + keys_per_block : n;  // the launch leaves no block empty
  const int64_t nbatch = (kend - kbeg + 63) / 64;
  const int64_t nbv = (n + kTile - 1) / kTile;  // value blocks of the group
  vcodes += grp * nbv * VB * dp;
  vnorms += grp * n;
  auto key_of = [&](int64_t batch) {
    const int64_t k = kbeg + batch * 64 + lane;
    return k < kend ? k : kend - 1;
  };
  auto load_in = [&](int64_t batch) __attribute__((always_inline)) {
    FusedIn<KB, VB> x;
    const int64_t k = key_of(batch);
    x.key = load_key<KB>(codes, signs, norms, rnorms, grp * n + k);
    x.vn = vnorms[k];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      int64_t tb = (kbeg + batch * 64) / kTile + kk;
      tb = tb < nbv ? tb : nbv - 1;
      const uint2* q = reinterpret_cast<const uint2*>(vcodes + tb * VB * dp) + VB * lane;
#pragma unroll
      for (int u = 0; u < VB; ++u) {
        const uint2 v = q[u];
        x.vw[kk][2 * u] = v.x;
        x.vw[kk][2 * u + 1] = v.y;
      }
    }
    return x;
  };

  // ---- prologue: v = Pi q, w = S q, power-of-two scales, byte tables (the
  // scorer's), the value level table, and the chunk's largest value norm
  const bool pro = tid < kFPro;  // a table-building thread
  const int mj = tid & (kDim - 1), part = (tid / kDim) & (kParts - 1);
  const float* pcol = piT + kPRows * part * kDim + mj;
  const float* scol = sT + kPRows * part * kDim + mj;
  const int qi = tid & (kDim - 1), qq = (tid >> 7) & 3;
  const bool qok = q0 + qq < nq && qi < d;
  const float qraw = queries[(grp * nq + (q0 + qq < nq ? q0 + qq : nq - 1)) * d + (qi < d ? qi : d - 1)];
  float pv[kPRows], pw[kPRows];
#pragma unroll
  for (int k = 0; k < kPRows; ++k) {
    pv[k] = pro ? pcol[k * kDim] : 0.0f;
    pw[k] = pro ? scol[k * kDim] : 0.0f;
  }
  FusedIn<KB, VB> cur = load_in(wave);
  if (pro) reinterpret_cast<float*>(sh.pro.qs)[qi * 4 + qq] = qok ? qraw : 0.0f;  // every (q, i) once
  if (tid == 0) next_batch = kFWaves;
  float nmax = 0.0f;
  for (int64_t t = kbeg + tid; t < kend; t += NTH) nmax = fmaxf(nmax, vnorms[t]);
  nmax = wave_max(nmax);
  if (lane == 0) nred[wave] = nmax;
  __syncthreads();
  if (pro) {
    float av[4] = {0.0f, 0.0f, 0.0f, 0.0f}, aw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kPRows; ++k) {
      const float4 x = sh.pro.qs[kPRows * part + k];
      av[0] = fmaf(pv[k], x.x, av[0]);
      av[1] = fmaf(pv[k], x.y, av[1]);
      av[2] = fmaf(pv[k], x.z, av[2]);
      av[3] = fmaf(pv[k], x.w, av[3]);
      aw[0] = fmaf(pw[k], x.x, aw[0]);
      aw[1] = fmaf(pw[k], x.y, aw[1]);
      aw[2] = fmaf(pw[k], x.z, aw[2]);
      aw[3] = fmaf(pw[k], x.w, aw[3]);
    }
    float* red = reinterpret_cast<float*>(tabs);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      red[((part * 2 + 0) * 4 + q) * kDim + mj] = av[q];
      red[((part * 2 + 1) * 4 + q) * kDim + mj] = aw[q];
    }
  }
  __syncthreads();
  for (int e = tid; e < 2 * 4 * kDim; e += NTH) {  // e = (tab * 4 + q) * kDim + j
    const float* red = reinterpret_cast<const float*>(tabs);
    float sum = 0.0f;
#pragma unroll
    for (int pp = 0; pp < kParts; ++pp) sum += red[pp * 1024 + e];
    sh.pro.vec[e >> 9][(e >> 7) & 3][e & (kDim - 1)] = sum;
  }
  if constexpr (VF != kSignForm) {
    for (int idx = tid; idx < Fm::kEntries; idx += NTH) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        int level = 0;
#pragma unroll
        for (int p = 0; p < VB; ++p) level |= ((idx >> (p * E + e)) & 1) << p;
        const float x = fp.val[level];
        const _Float16 hi = static_cast<_Float16>(x);
        vtab[idx * Fm::kHalves + e] = hi;
        if constexpr (VF == kTwoPiece) vtab[idx * Fm::kHalves + E + e] = static_cast<_Float16>(x - float(hi));
      }
    }
  }
  __syncthreads();
  if (wave < 8) {
    const int tab = wave >> 2, q = wave & 3;  // waves 0..7: one (table, query) vector each
    const float x0 = sh.pro.vec[tab][q][lane], x1 = sh.pro.vec[tab][q][lane + 64];
    float ss = fmaf(x0, x0, x1 * x1);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) {
      int e = 0;
      (void)frexpf(sqrtf(ss), &e);
      scale_t[tab][q] = ss > 0.0f ? ldexpf(1.0f, 1 - e) : 1.0f;
    }
  }
  __syncthreads();
  if (pro) {
    constexpr int kSegs = 256 / kWalk, kHi = kWalk / 2;
    const int q = tid & 3, gg = (tid >> 2) & 15, seg = (tid >> 6) & (kSegs - 1), tab = tid / (64 * kSegs);
    const float sc = scale_t[tab][q];
    float xs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[i] = sc * sh.pro.vec[tab][q][8 * gg + i];
    unsigned char* col = tabs + tab * 128 + gg * 8 + q * 2;
    const int rank0 = kWalk * seg, gb = rank0 ^ (rank0 >> 1);
    unsigned char* base0 = col + 256 * gb;
    unsigned char* base1 = col + 256 * (gb ^ kHi);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += ((gb >> i) & 1) ? xs[i] : -xs[i];
    *reinterpret_cast<_Float16*>(base0) = static_cast<_Float16>(acc);
#pragma unroll
    for (int m = 1; m < kWalk; ++m) {
      const int gm = m ^ (m >> 1), b = __builtin_ctz(m);
      const bool up = (1 << b) == kHi ? (((gb ^ gm) >> b) & 1) != 0 : ((gm >> b) & 1) != 0;
      acc += up ? 2.0f * xs[b] : -2.0f * xs[b];
      *reinterpret_cast<_Float16*>(((gm & kHi) ? base1 : base0) + 256 * (gm & (kHi - 1))) =
          static_cast<_Float16>(acc);
    }
  }
  float nm_all = 0.0f;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) nm_all = fmaxf(nm_all, nred[w]);
  int ne = 0;
  if (nm_all > 0.0f && nm_all < INFINITY) (void)frexpf(nm_all, &ne);
  const float nscale = ldexpf(1.0f, -ne);
  __syncthreads();  // tables; the prologue's LDS becomes the weight slices

  // ---- per-lane scorer setup (the scorer's rotation and address bases)
  const uint32_t r = uint32_t(tid) & 15u;
  const bool w1 = (r >> 2) & 1u, w2 = (r >> 3) & 1u;
  const uint32_t bs = r & 3u;
  uint32_t lb[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) lb[k] = (((2u * k + r) & 15u) * 8u) | ((((2u * k + 1u + r) & 15u) * 8u) << 8);
  float inv_v[4], inv_w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    inv_v[q] = 1.0f / scale_t[0][q];
    inv_w[q] = kappa / scale_t[1][q];
  }
  const half2_t pick_lo = {(_Float16)1.0f, (_Float16)0.0f};
  const half2_t pick_hi = {(_Float16)0.0f, (_Float16)1.0f};
  auto claim = [&]() -> int64_t {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(&next_batch, 1u);
    return __builtin_amdgcn_readfirstlane(v);
  };
  const int n16 = lane & 15, g16 = lane >> 4;
  uint32_t sgn_mask = 0x80008000u, sgn_one = 0x3C003C00u;
  asm volatile("" : "+v"(sgn_mask), "+v"(sgn_one));
  const float a = scale * 1.4426950408889634f;  // weights are 2^(a s - ref)
  float lm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // reference maxima (log2), the same in every lane
  float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 acc2[8];  // row 4 g16 + i, coordinate 16 j + n16
#pragma unroll
  for (int j = 0; j < 8; ++j) acc2[j] = f32x4{};

  int64_t b = wave;
  int64_t bn = claim();
  while (b < nbatch) {
    const int64_t bnn = claim();
    const FusedIn<KB, VB> nxt = load_in(bn);  // unused past the end
    // scores of the batch's tokens (the scorer's inner loop)
    float sc[4];
    {
      Words pl[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) pl[p] = rotate(cur.key.plane[p], w1, w2, bs);
      const Words sg = rotate(cur.key.sign, w1, w2, bs);
      Words term[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t x = 0;
#pragma unroll
          for (int p = 0; p < KB; ++p)
            if (TT::mask[j] & (1u << p)) x ^= pl[p].w[i];
          term[j].w[i] = x;
        }
      }
      float acc[NT + 1][4];
#pragma unroll
      for (int j = 0; j <= NT; ++j) acc[j][0] = acc[j][1] = acc[j][2] = acc[j][3] = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half2_t part[NT + 1][2];
#pragma unroll
        for (int j = 0; j <= NT; ++j) part[j][0] = part[j][1] = half2_t{(_Float16)0.0f, (_Float16)0.0f};
#define TQ_FSTEP(T)                                                                                    \
  {                                                                                                    \
    _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                                   \
      const Entry e = lut<0>(tabs, __builtin_amdgcn_perm(term[j].w[i], lb[(T) >> 1], perm_sel<(T)>())); \
      part[j][0] += e.q01;                                                                             \
      part[j][1] += e.q23;                                                                             \
    }                                                                                                  \
    const Entry e = lut<1>(tabs, __builtin_amdgcn_perm(sg.w[i], lb[(T) >> 1], perm_sel<(T)>()));       \
    part[NT][0] += e.q01;                                                                              \
    part[NT][1] += e.q23;                                                                              \
    if ((T) & 1) pin<NT + 1>(part);                                                                    \
  }
        if (i == 0) { TQ_FSTEP(0) TQ_FSTEP(1) TQ_FSTEP(2) TQ_FSTEP(3) }
        if (i == 1) { TQ_FSTEP(4) TQ_FSTEP(5) TQ_FSTEP(6) TQ_FSTEP(7) }
        if (i == 2) { TQ_FSTEP(8) TQ_FSTEP(9) TQ_FSTEP(10) TQ_FSTEP(11) }
        if (i == 3) { TQ_FSTEP(12) TQ_FSTEP(13) TQ_FSTEP(14) TQ_FSTEP(15) }
#undef TQ_FSTEP
#pragma unroll
        for (int j = 0; j <= NT; ++j) {
          acc[j][0] = __builtin_amdgcn_fdot2(part[j][0], pick_lo, acc[j][0], false);
          acc[j][1] = __builtin_amdgcn_fdot2(part[j][0], pick_hi, acc[j][1], false);
          acc[j][2] = __builtin_amdgcn_fdot2(part[j][1], pick_lo, acc[j][2], false);
          acc[j][3] = __builtin_amdgcn_fdot2(part[j][1], pick_hi, acc[j][3], false);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s1 = 0.0f;
#pragma unroll
        for (int j = 0; j < NT; ++j) s1 = fmaf(pe.alpha[j], acc[j][q], s1);
        const float sw = acc[NT][q] * inv_w[q];
        sc[q] = cur.key.n * fmaf(cur.key.rho, sw, s1 * inv_v[q]);
      }
    }
    // online softmax: the reference maximum of a row moves (and what was
    // summed so far is rescaled) only when a score passes it by kSlack
    const bool tin = kbeg + b * 64 + lane < kend;
    float x[4];
    bool over = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] = tin && q < qc ? a * sc[q] : -INFINITY;
      over |= x[q] > lm[q] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      float f[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float nm = fmaxf(lm[q], wave_max(x[q]));
        f[q] = nm > lm[q] ? exp2f(lm[q] - nm) : 1.0f;
        lm[q] = nm;
        lsum[q] *= f[q];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc2[j][i] *= f[i];  // rows 4..15 (g16 > 0) hold zeros
    }
    const float nv = cur.vn * nscale;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool use = tin && q < qc;
      // the hardware exp2 (a weight below 2^-126 of the reference flushes to 0)
      const float w = use ? __builtin_amdgcn_exp2f(x[q] - lm[q]) : 0.0f;
      lsum[q] += w;
      float p = w * nv;
      asm volatile("" : "+v"(p));  // one float32 rounding for both pieces (as above)
      const _Float16 hi = static_cast<_Float16>(p);
      sh.pa[wave][0][q][lane] = hi;
      sh.pa[wave][1][q][lane] = static_cast<_Float16>(p - float(hi));
    }
    // the value levels of the batch's two token blocks against the weights
    // (LDS is in order within a wave: the reads see the writes above)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f16x8 ah = {}, al = {};
      if (n16 < 4) {
        ah = *reinterpret_cast<const f16x8*>(&sh.pa[wave][0][n16][32 * kk + 8 * g16]);
        al = *reinterpret_cast<const f16x8*>(&sh.pa[wave][1][n16][32 * kk + 8 * g16]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f16x8 bv, bl;
        if constexpr (VF == kSignForm) {
          const uint4 sg = score::expand_signs(bit_field(cur.vw[kk], 8 * VB * j, 8), sgn_mask, sgn_one);
          bv = *reinterpret_cast<const f16x8*>(&sg);
        } else {
#pragma unroll
          for (int k = 0; k < 8 / E; ++k) {
            const uint32_t idx = bit_field(cur.vw[kk], 8 * VB * j + k * VB * E, VB * E);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              bv[k * E + e] = vtab[idx * Fm::kHalves + e];
              if constexpr (VF == kTwoPiece) bl[k * E + e] = vtab[idx * Fm::kHalves + E + e];
            }
          }
        }
        acc2[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv, acc2[j], 0, 0, 0);
        acc2[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv, acc2[j], 0, 0, 0);
        if constexpr (VF == kTwoPiece) acc2[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc2[j], 0, 0, 0);
      }
    }
    cur = nxt;
    b = bn;
    bn = bnn;
  }

  // ---- the waves' partials combined into the workgroup's split
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lsum[q] += __shfl_xor(lsum[q], o);
  }
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wmax[wave][q] = lm[q];
      wsum[wave][q] = lsum[q];
    }
  }
  __syncthreads();  // every wave is past its last lookup: the tables' space is free
  float mq[4], fw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) m = fmaxf(m, wmax[w][q]);
    mq[q] = m;
    fw[q] = lm[q] > -INFINITY ? exp2f(lm[q] - m) : 0.0f;
  }
  float* red = reinterpret_cast<float*>(tabs);  // [wave][row][coordinate]
  if (g16 == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * dp + 16 * j + n16] = acc2[j][i] * fw[i];
  }
  __syncthreads();
  {
    const int row = (tid >> 7) & 3, coord = tid & 127;  // threads below 512: 4 rows x 128 coordinates
    float y = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) {
      y += red[(w * 4 + row) * dp + coord];
      if (coord == 0) l += wmax[w][row] > -INFINITY ? wsum[w][row] * exp2f(wmax[w][row] - mq[row]) : 0.0f;
    }
    if (tid < 4 * dp && row < qc) {
      const int64_t rr = (grp * nq + q0 + row) * chunks + c;
      part_y[rr * dp + coord] = y * (fp.gamma * ldexpf(1.0f, ne));
      if (coord == 0) part_ml[rr] = make_float2(mq[row] * 0.6931471805599453f, l);
    }
  }
}

// ---------------------------------------------------------------------------
// merge of the splits and the rotation back
// ---------------------------------------------------------------------------

__device__ __forceinline__ float block_reduce(float x, float* sh, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  __syncthreads();
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  float r = sh[0];
  for (int w = 1; w < kWaves; ++w) r = is_max ? fmaxf(r, sh[w]) : r + sh[w];
  return r;
}

// block per (group, query) row; dynamic LDS: the normalised sum (d floats)
// and the partials (kThreads float4).  With d a multiple of 4 (dp, the
// padded width, always is), thread t takes coordinates 4 (t mod Q) .. + 3
// (Q = min(dp, 4 kThreads) / 4 quads per pass) and partition t div Q of the
// P = kThreads / Q partitions: each partition sums every P-th split (then
// every P-th row of Pi^T) with float4 loads, 8 in flight, and the
// partitions meet in LDS.  A decode-sized call has few rows, so the
// latency of these load rounds, not their bytes, sets its time.
__global__ void __launch_bounds__(kThreads)
attn_merge_kernel(const float* __restrict__ part_y, const float2* __restrict__ part_ml, int64_t splits, int dp,
                  int d, const float* __restrict__ pi, float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float dyn[];
  float* yh = dyn;                                   // [dp]
  float4* parts = reinterpret_cast<float4*>(dyn + dp);  // [kThreads]
  __shared__ float wts[kMaxSplits];
  __shared__ float sh[kWaves];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  part_ml += row * splits;
  part_y += row * splits * dp;
  float m = -INFINITY;
  for (int64_t s = tid; s < splits; s += kThreads) m = fmaxf(m, part_ml[s].x);
  const float M = block_reduce(m, sh, true);
  float l = 0.0f;
  for (int64_t s = tid; s < splits; s += kThreads) {
    const float2 ml = part_ml[s];
    const float w = ml.y > 0.0f ? expf(ml.x - M) : 0.0f;  // a split with no tokens adds nothing
    wts[s] = w;
    l += ml.y * w;
  }
  const float L = block_reduce(l, sh, false);  // (its barriers also publish wts)
  const float inv = 1.0f / L;
  const int quads = dp / 4;
  const int Q = quads < kThreads ? quads : kThreads;
  const int P = kThreads / Q;
  const int part = tid / Q, ql = tid % Q;
  // combine the splits: coordinates 4 c4 .. 4 c4 + 3, splits part, part + P, ...
  for (int q0 = 0; q0 < quads; q0 += Q) {
    const int c4 = q0 + ql;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (part < P && c4 < quads) {
      const float4* py = reinterpret_cast<const float4*>(part_y) + c4;
      int64_t s = part;
      for (; s + 7 * P < splits; s += 8 * P) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = py[(s + u * P) * quads];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wv = wts[s + u * P];
          a.x = fmaf(v[u].x, wv, a.x), a.y = fmaf(v[u].y, wv, a.y);
          a.z = fmaf(v[u].z, wv, a.z), a.w = fmaf(v[u].w, wv, a.w);
        }
      }
      for (; s < splits; s += P) {
        const float4 v = py[s * quads];
        const float wv = wts[s];
        a.x = fmaf(v.x, wv, a.x), a.y = fmaf(v.y, wv, a.y), a.z = fmaf(v.z, wv, a.z), a.w = fmaf(v.w, wv, a.w);
      }
    }
    parts[tid] = a;
    __syncthreads();
    if (part == 0 && c4 < quads) {
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int q = 0; q < P; ++q) {
        const float4 v = parts[q * Q + ql];
        t.x += v.x, t.y += v.y, t.z += v.z, t.w += v.w;
      }
      yh[4 * c4] = t.x * inv, yh[4 * c4 + 1] = t.y * inv, yh[4 * c4 + 2] = t.z * inv, yh[4 * c4 + 3] = t.w * inv;
    }
    __syncthreads();
  }
  // out_i = sum_c Pi[c][i] yh[c] (c < d): outputs 4 i4 .. + 3, rows part, part + P, ...
  // (Pi rows are d floats; d % 4 == 0 takes float4 loads)
  const int oq = (d + 3) / 4;
  const int Qo = oq < kThreads ? oq : kThreads;
  const int Po = kThreads / Qo;
  const int parto = tid / Qo, qo = tid % Qo;
  const bool vec = (d & 3) == 0;
  for (int i0 = 0; i0 < oq; i0 += Qo) {
    const int i4 = i0 + qo;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (parto < Po && i4 < oq) {
      if (vec) {
        const float4* pr = reinterpret_cast<const float4*>(pi) + i4;
        int c = parto;
        for (; c + 7 * Po < d; c += 8 * Po) {
          float4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = pr[int64_t(c + u * Po) * oq];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float y = yh[c + u * Po];
            o.x = fmaf(v[u].x, y, o.x), o.y = fmaf(v[u].y, y, o.y);
            o.z = fmaf(v[u].z, y, o.z), o.w = fmaf(v[u].w, y, o.w);
          }
        }
        for (; c < d; c += Po) {
          const float4 v = pr[int64_t(c) * oq];
          const float y = yh[c];
          o.x = fmaf(v.x, y, o.x), o.y = fmaf(v.y, y, o.y), o.z = fmaf(v.z, y, o.z), o.w = fmaf(v.w, y, o.w);
        }
      } else {
        for (int c = parto; c < d; c += Po) {
          const float y = yh[c];
          const float* pr = pi + int64_t(c) * d + 4 * i4;
          o.x = fmaf(pr[0], y, o.x);
          if (4 * i4 + 1 < d) o.y = fmaf(pr[1], y, o.y);
          if (4 * i4 + 2 < d) o.z = fmaf(pr[2], y, o.z);
          if (4 * i4 + 3 < d) o.w = fmaf(pr[3], y, o.w);
        }
      }
    }
    parts[tid] = o;
    __syncthreads();
    if (parto == 0 && i4 < oq) {
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int q = 0; q < Po; ++q) {
        const float4 v = parts[q * Qo + qo];
        t.x += v.x, t.y += v.y, t.z += v.z, t.w += v.w;
      }
      float* dst = out + row * d + 4 * i4;
      dst[0] = t.x;
      if (4 * i4 + 1 < d) dst[1] = t.y;
      if (4 * i4 + 2 < d) dst[2] = t.z;
      if (4 * i4 + 3 < d) dst[3] = t.w;
    }
    __syncthreads();
  }
  if (tid == 0 && lse) lse[row] = M + logf(L);
}

// level form of the value handle: the scorer's forms, with the staged signs'
// minus folded into gamma for the sign form
int value_form(const tq_ctx* h) {
  if (h->code_bits == 1 && h->symmetric) return kSignForm;
  if (h->code_bits == 2 && h->dqt.two_pass) return kOnePiece;
  return kTwoPiece;
}

ScoreForm value_params(const tq_ctx* h) {
  ScoreForm fp{};
  switch (value_form(h)) {
    case kSignForm:
      fp.gamma = -h->cb.c[1];  // bit 1 stages as -1 and stands for +c[1]
      break;
    case kOnePiece:
      for (int i = 0; i < kMaxLevels; ++i) fp.val[i] = h->dqt.v[i];
      fp.gamma = float(double(h->dqt.out_scale) * 4096.0);  // 1 / sigma
      break;
    default:
      for (int i = 0; i < kMaxLevels; ++i) fp.val[i] = h->cb.c[i] * 1024.0f;
      fp.gamma = 1.0f / 1024.0f;
  }
  return fp;
}

struct PvArgs {
  const float* scores;
  int64_t nq, n;
  const uint32_t* vcodes;
  const float* vnorms;
  int W;
  int word_base;
  bool write_ml;
  float scale;
  int64_t tps;
  int qchunks;
  ScoreForm fp;
  float* part_y;
  float2* part_ml;
  int64_t splits;
};

template <int B, int F, int RQ, int G>
void launch_pv_g(const PvArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_pv_kernel<B, F, RQ, G>), grid, dim3(kThreads), 0, s, a.scores, a.nq, a.n, a.vcodes,
                     a.vnorms, a.W, a.word_base, a.write_ml, a.scale, a.tps, a.qchunks, a.fp, a.part_y, a.part_ml,
                     a.splits);
}

template <int B, int F, int RQ>
void launch_pv_rq(const PvArgs& a, dim3 grid, int g, hipStream_t s) {
  switch (g) {
    case 1: launch_pv_g<B, F, RQ, 1>(a, grid, s); break;
    case 2: launch_pv_g<B, F, RQ, 2>(a, grid, s); break;
    case 3: launch_pv_g<B, F, RQ, 3>(a, grid, s); break;
    default: launch_pv_g<B, F, RQ, 4>(a, grid, s);
  }
}

// full coordinate groups (4 words) in one launch, the last partial group
// (W mod 4 words) in another
template <int B, int F>
hipError_t launch_pv(PvArgs a, dim3 grid, hipStream_t s) {
  const int full = a.W / kWordsPerWave, rest = a.W % kWordsPerWave;
  auto go = [&](int g) {
    if (a.nq <= 4) launch_pv_rq<B, F, 4>(a, grid, g, s);
    else if (a.nq <= 8) launch_pv_rq<B, F, 8>(a, grid, g, s);
    else launch_pv_rq<B, F, kRows>(a, grid, g, s);
  };
  if (full > 0) {
    grid.y = unsigned(full);
    a.word_base = 0;
    a.write_ml = true;
    go(4);
  }
  if (rest > 0) {
    grid.y = 1;
    a.word_base = kWordsPerWave * full;
    a.write_ml = full == 0;
    go(rest);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_values(const tq_ctx* h, const uint32_t* codes, int64_t groups, int64_t n, uint32_t* vcodes,
                              hipStream_t stream) {
  const int64_t nb = (n + kTile - 1) / kTile;
  if (nb == 0 || groups == 0) return hipSuccess;
  // transposed planes and the output staging, B x 32 W words each per token
  // block; 4 token blocks per workgroup while that fits 64 KiB, else 1
  const size_t per = size_t(2) * h->code_bits * 32 * h->words * sizeof(uint32_t);
  const bool four = 4 * per <= 65536;
  const size_t lds = four ? 4 * per : per;
  const int64_t wgs = four ? (nb + 3) / 4 : nb;
  auto launch = [&](auto kernel) {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, dim3(unsigned(wgs), unsigned(groups)), dim3(kThreads), lds, stream, codes, n,
                       h->words, nb, vcodes);
    return hipGetLastError();
  };
  switch (h->code_bits * 2 + (four ? 1 : 0)) {
    case 2: return launch(pack_values_kernel<1, 1>);
    case 3: return launch(pack_values_kernel<1, 4>);
    case 4: return launch(pack_values_kernel<2, 1>);
    case 5: return launch(pack_values_kernel<2, 4>);
    case 6: return launch(pack_values_kernel<3, 1>);
    case 7: return launch(pack_values_kernel<3, 4>);
    case 8: return launch(pack_values_kernel<4, 1>);
    case 9: return launch(pack_values_kernel<4, 4>);
    default: return hipErrorInvalidValue;
  }
}

// tokens per split: enough blocks to fill the GPU a few times over, at
// most kMaxSplits splits; TQ_ATTN_SPLIT=<tokens> overrides (tests use it to
// cover many splits)
int64_t attn_split_tokens(const tq_ctx* hv, int64_t groups, int64_t nq, int64_t n) {
  int64_t tps;
  if (const char* v = std::getenv("TQ_ATTN_SPLIT")) {
    tps = std::atoll(v);
  } else {
    const int64_t per = int64_t((hv->words + kWordsPerWave - 1) / kWordsPerWave) * groups * ((nq + kRows - 1) / kRows);
    const int64_t target = 8 * int64_t(hv->cus > 0 ? hv->cus : 256);  // waves: 2 per SIMD, one round
    int64_t splits = (target + per - 1) / per;
    const int64_t tiles = (n + kTile - 1) / kTile;
    splits = splits < tiles ? splits : tiles;
    splits = splits < 1 ? 1 : splits;
    tps = (n + splits - 1) / splits;
  }
  tps = (tps + kTile - 1) / kTile * kTile;
  if (tps < kTile) tps = kTile;
  const int64_t minimum = (n + kMaxSplits - 1) / kMaxSplits;
  if (tps < minimum) tps = (minimum + kTile - 1) / kTile * kTile;
  return tps;
}

size_t attn_partial_bytes(const tq_ctx* hv, int64_t groups, int64_t nq, int64_t n) {
  const int64_t tps = attn_split_tokens(hv, groups, nq, n);
  const int64_t splits = n > 0 ? (n + tps - 1) / tps : 0;
  const size_t y = size_t(groups) * nq * splits * 32 * hv->words * sizeof(float);
  const size_t ml = size_t(groups) * nq * splits * sizeof(float2);
  return ws_align(y) + ws_align(ml);
}

bool attention_fused_supported(const tq_ctx* hk, const tq_ctx* hv) {
  if (const char* v = std::getenv("TQ_ATTN_FUSED"))
    if (std::strcmp(v, "0") == 0) return false;
  return logits_lut128_supported(hk) && hk->hi == 0 && hk->code_bits <= 3 && hv->words == 4 && hv->hi == 0 &&
         hv->code_bits <= 3 && hk->d == hv->d;
}

namespace {
// one workgroup per CU, each on a chunk of one pair's tokens (a multiple of
// 64, so that every chunk holds whole value blocks); no chunk is empty
void fused_chunks(const tq_ctx* hk, int64_t pairs, int64_t n, int64_t* chunks, int64_t* kpb) {
  int64_t c = (hk->cus + pairs - 1) / pairs;
  int64_t k = (n + c - 1) / c;
  k = (k + 63) / 64 * 64;
  *kpb = k;
  *chunks = (n + k - 1) / k;
}
}  // namespace

size_t attn_fused_partial_bytes(const tq_ctx* hk, int64_t groups, int64_t nq, int64_t n) {
  if (n <= 0) return 0;
  int64_t chunks, kpb;
  fused_chunks(hk, groups * ((nq + 3) / 4), n, &chunks, &kpb);
  return ws_align(size_t(groups) * nq * chunks * 128 * sizeof(float)) + ws_align(size_t(groups) * nq * chunks * sizeof(float2));
}

hipError_t launch_attention_fused(const tq_ctx* hk, const tq_ctx* hv, const float* queries, int64_t groups,
                                  int64_t nq, const uint32_t* kcodes, const uint32_t* ksigns, const float* knorms,
                                  const float* krnorms, int64_t n, const uint32_t* vcodes, const float* vnorms,
                                  float scale, void* partials, float* out, float* lse, hipStream_t stream) {
  const int64_t quads = (nq + 3) / 4;
  const int64_t pairs = groups * quads;
  int64_t chunks, kpb;
  fused_chunks(hk, pairs, n, &chunks, &kpb);
  const int64_t blocks = chunks * pairs;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const size_t ybytes = size_t(groups) * nq * chunks * 128 * sizeof(float);
  float* part_y = static_cast<float*>(partials);
  float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(partials) + ws_align(ybytes));
  const float kappa = 1.2533141373155002512f / float(hk->d);
  const ScoreForm fp = value_params(hv);
  auto go = [&](auto kernel, int nth) {
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(nth), 0, stream, queries, int(quads), nq,
                       n, hk->d, hk->d_piT128, hk->d_sT128, kcodes, ksigns, knorms, krnorms, hk->planes, kappa, vcodes,
                       vnorms, fp, scale, static_cast<int>(chunks), kpb, part_y, part_ml);
    return hipGetLastError();
  };
  auto by_value = [&](auto kbc) {
    constexpr int KB = decltype(kbc)::value;
    switch (hv->code_bits * 4 + value_form(hv)) {
      // three waves per SIMD while the key loop fits 168 registers
      case 1 * 4 + kSignForm: return go(attn_fused_kernel<KB, 1, kSignForm, KB <= 2 ? 768 : 512>, KB <= 2 ? 768 : 512);
      case 1 * 4 + kTwoPiece: return go(attn_fused_kernel<KB, 1, kTwoPiece, 512>, 512);
      case 2 * 4 + kOnePiece: return go(attn_fused_kernel<KB, 2, kOnePiece, KB <= 2 ? 768 : 512>, KB <= 2 ? 768 : 512);
      case 2 * 4 + kTwoPiece: return go(attn_fused_kernel<KB, 2, kTwoPiece, 512>, 512);
      case 3 * 4 + kTwoPiece: return go(attn_fused_kernel<KB, 3, kTwoPiece, 512>, 512);
      default: return hipErrorInvalidValue;
    }
  };
  hipError_t e;
  switch (hk->code_bits) {
    case 1: e = by_value(std::integral_constant<int, 1>{}); break;
    case 2: e = by_value(std::integral_constant<int, 2>{}); break;
    case 3: e = by_value(std::integral_constant<int, 3>{}); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(unsigned(groups * nq)), dim3(kThreads),
                     size_t(32 * hv->words) * sizeof(float) + size_t(kThreads) * sizeof(float4), stream, part_y, part_ml,
                     chunks, 32 * hv->words, hv->d, hv->d_pi, out, lse);
  return hipGetLastError();
}

hipError_t launch_attention_values(const tq_ctx* hv, const float* scores, int64_t groups, int64_t nq, int64_t n,
                                   const uint32_t* vcodes, const float* vnorms, float scale, void* partials,
                                   float* out, float* lse, hipStream_t stream) {
  PvArgs a{};
  a.scores = scores;
  a.nq = nq;
  a.n = n;
  a.vcodes = vcodes;
  a.vnorms = vnorms;
  a.W = hv->words;
  a.scale = scale;
  a.tps = attn_split_tokens(hv, groups, nq, n);
  a.splits = (n + a.tps - 1) / a.tps;
  a.qchunks = int((nq + kRows - 1) / kRows);
  a.fp = value_params(hv);
  const size_t ybytes = size_t(groups) * nq * a.splits * 32 * hv->words * sizeof(float);
  a.part_y = static_cast<float*>(partials);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(partials) + ws_align(ybytes));
  const dim3 grid(unsigned((a.splits + kWaves - 1) / kWaves), unsigned((hv->words + kWordsPerWave - 1) / kWordsPerWave),
                  unsigned(groups * a.qchunks));
  hipError_t e;
  switch (hv->code_bits) {
    case 1:
      e = value_form(hv) == kSignForm ? launch_pv<1, kSignForm>(a, grid, stream) : launch_pv<1, kTwoPiece>(a, grid, stream);
      break;
    case 2:
      e = value_form(hv) == kOnePiece ? launch_pv<2, kOnePiece>(a, grid, stream) : launch_pv<2, kTwoPiece>(a, grid, stream);
      break;
    case 3: e = launch_pv<3, kTwoPiece>(a, grid, stream); break;
    case 4: e = launch_pv<4, kTwoPiece>(a, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(unsigned(groups * nq)), dim3(kThreads),
                     size_t(32 * hv->words) * sizeof(float) + size_t(kThreads) * sizeof(float4),
                     stream, a.part_y, a.part_ml, a.splits, 32 * hv->words, hv->d, hv->d_pi, out, lse);
  return hipGetLastError();
}

}  // namespace tqdev
