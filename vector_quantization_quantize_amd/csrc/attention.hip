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
// Value layout (token blocks): vcodes[group][ceil(n/32)][B][32 W] uint32,
// bit i of word (block b, plane p, coordinate j) = bit p of the index of
// coordinate j of token 32 b + i.  One word then holds one coordinate of 32
// tokens: the contraction over tokens is the matrix-core K dimension, and a
// lane expands its operand from one byte without a bit transpose.
//
// Kernels:
//  * pack_values_kernel: key-layout codes -> token blocks (a 32 x 32 bit
//    transpose per word by wave ballots).
//  * attn_pv_kernel: per (key split, 4-word coordinate group, group, 16
//    query rows): pass 1 finds each row's max of scale s over the split and
//    the split's largest norm; pass 2 walks 32-token tiles: weights
//    p = exp(scale s - max) n / 2^e go to LDS as two float16 pieces (22
//    bits), each wave expands its word's levels (the scorer's level forms)
//    and runs v_mfma_f32_16x16x32_f16: 16 query rows x 32 tokens x 16
//    coordinates per pass.  Writes the split's (max, sum of exp) per row and
//    its partial sums per coordinate.
//  * attn_merge_kernel: per (group, query): combines the splits (rescaled to
//    the overall max), divides by the sum, and applies Pi^T.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "score_mfma.h"
#include "tq_internal.h"

namespace tqdev {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
using score::f16x8;

constexpr int kRows = 16;   // query rows per block (matrix-core M)
constexpr int kTile = 32;   // tokens per tile (matrix-core K; one word of a value plane)
constexpr int kWaves = 4;   // waves per block: one 32-coordinate word each
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSplits = 1024;

// ---------------------------------------------------------------------------
// value packing
// ---------------------------------------------------------------------------

// block (token block, group); wave pairs of key-layout words: lanes 0-31
// hold word `pw` of tokens 0-31, lanes 32-63 word `pw + 1`; ballot j
// collects bit j (coordinate 32 w + j) of the 32 tokens of each half.
__global__ void __launch_bounds__(kThreads)
pack_values_kernel(const uint32_t* __restrict__ codes, int64_t n, int B, int W, int64_t nb,
                   uint32_t* __restrict__ vcodes) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t blk = blockIdx.x, grp = blockIdx.y;
  const int pws = B * W;  // words per token in the key layout
  codes += grp * n * pws;
  vcodes += (grp * nb + blk) * int64_t(pws) * 32;
  const int64_t tok = blk * 32 + (lane & 31);
  for (int pw = 2 * wave; pw < pws; pw += 2 * kWaves) {
    const int mine = pw + (lane >> 5);
    const uint32_t x = (mine < pws && tok < n) ? codes[tok * pws + mine] : 0u;
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint64_t m = __ballot((x >> j) & 1u);
      const uint32_t part = lane < 32 ? uint32_t(m) : uint32_t(m >> 32);
      out = (lane & 31) == j ? part : out;
    }
    if (mine < pws) {
      const int p = mine / W, w = mine % W;
      vcodes[int64_t(p) * 32 * W + 32 * w + (lane & 31)] = out;
    }
  }
}

// ---------------------------------------------------------------------------
// weighted sum of the stored levels
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

template <int B, int F>
__global__ void __launch_bounds__(kThreads)
attn_pv_kernel(const float* __restrict__ scores, int64_t nq, int64_t n, const uint32_t* __restrict__ vcodes,
               const float* __restrict__ vnorms, int W, float scale, int64_t tps, int qchunks, ScoreForm fp,
               float* __restrict__ part_y, float2* __restrict__ part_ml, int64_t splits) {
  using Fm = score::Form<B, F>;
  constexpr int E = Fm::E;
  __shared__ _Float16 vtab[F == kSignForm ? 8 : Fm::kEntries * Fm::kHalves];
  __shared__ __align__(16) _Float16 pa[2][2][kRows][kTile];  // [buf][hi, lo][row][token]
  __shared__ float red[kWaves][kRows + 1];
  __shared__ float row_m[kRows];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t split = blockIdx.x;
  const int word = kWaves * blockIdx.y + wave;
  const int64_t grp = blockIdx.z / qchunks;
  const int64_t q0 = int64_t(blockIdx.z % qchunks) * kRows;
  const int rows = nq - q0 < kRows ? int(nq - q0) : kRows;
  const int64_t t0 = split * tps;
  const int64_t t1 = t0 + tps < n ? t0 + tps : n;
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

  // ---- pass 1: row maxima of scale * s and the largest norm over the split
  float lm[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) lm[r] = -INFINITY;
  float nmax = 0.0f;
  for (int64_t t = t0 + tid; t < t1; t += kThreads) {
    nmax = fmaxf(nmax, vnorms[t]);
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      if (r < rows) lm[r] = fmaxf(lm[r], scale * scores[r * n + t]);
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const float m = wave_max(lm[r]);
    if (lane == 0) red[wave][r] = m;
  }
  {
    const float m = wave_max(nmax);
    if (lane == 0) red[wave][kRows] = m;
  }
  __syncthreads();
  if (tid < kRows) row_m[tid] = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
  const float nm = fmaxf(fmaxf(red[0][kRows], red[1][kRows]), fmaxf(red[2][kRows], red[3][kRows]));
  // weights carry n / 2^e <= 1, so their float16 pieces cannot overflow
  int ne = 0;
  if (nm > 0.0f && nm < INFINITY) (void)frexpf(nm, &ne);
  const float nscale = ldexpf(1.0f, -ne);
  __syncthreads();

  // ---- pass 2: 32-token tiles.  Thread tid computes the weights of
  // (row tid / 32 and 8 + tid / 32, token tid % 32).
  const int wr = tid >> 5, wt = tid & 31;
  float lsum[2] = {0.0f, 0.0f};
  const int n16 = lane & 15, g16 = lane >> 4;
  uint32_t sgn_mask = 0x80008000u, sgn_one = 0x3C003C00u;
  asm volatile("" : "+v"(sgn_mask), "+v"(sgn_one));
  f32x4 acc[2] = {f32x4{}, f32x4{}};
  const bool active = word < W;
  int buf = 0;
  for (int64_t tb = t0; tb < t1; tb += kTile, buf ^= 1) {
    const int64_t tok = tb + wt;
    const bool tin = tok < t1;
    const float nv = tin ? vnorms[tok] * nscale : 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = wr + 8 * k;
      float p = 0.0f;
      if (tin && r < rows) {
        const float w = expf(scale * scores[r * n + tok] - row_m[r]);
        lsum[k] += w;
        p = w * nv;
      }
      const _Float16 hi = static_cast<_Float16>(p);
      pa[buf][0][r][wt] = hi;
      pa[buf][1][r][wt] = static_cast<_Float16>(p - float(hi));
    }
    __syncthreads();
    if (active) {
      // A: row n16, tokens 8 g16 .. 8 g16 + 7 (both pieces); B: coordinate
      // 32 word + 16 h + n16, the same tokens, from byte g16 of its words
      const f16x8 ah = *reinterpret_cast<const f16x8*>(&pa[buf][0][n16][8 * g16]);
      const f16x8 al = *reinterpret_cast<const f16x8*>(&pa[buf][1][n16][8 * g16]);
      const uint32_t* vw = vcodes + (tb / kTile) * B * dp + 32 * word + n16;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t pw[B];
#pragma unroll
        for (int p = 0; p < B; ++p) pw[p] = __builtin_amdgcn_ubfe(vw[p * dp + 16 * h], 8 * g16, 8);
        f16x8 bv, bl;
        if constexpr (F == kSignForm) {
          const uint4 s = score::expand_signs(pw[0], sgn_mask, sgn_one);
          bv = *reinterpret_cast<const f16x8*>(&s);
        } else {
#pragma unroll
          for (int k = 0; k < 8 / E; ++k) {
            uint32_t idx = 0;
#pragma unroll
            for (int p = 0; p < B; ++p) idx |= __builtin_amdgcn_ubfe(pw[p], k * E, E) << (p * E);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              bv[k * E + e] = vtab[idx * Fm::kHalves + e];
              if constexpr (F == kTwoPiece) bl[k * E + e] = vtab[idx * Fm::kHalves + E + e];
            }
          }
        }
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv, acc[h], 0, 0, 0);
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv, acc[h], 0, 0, 0);
        if constexpr (F == kTwoPiece) acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc[h], 0, 0, 0);
      }
    }
  }

  // ---- partial results of the split
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) lsum[k] += __shfl_xor(lsum[k], o);
  }
  const int64_t rowbase = grp * nq + q0;
  if (blockIdx.y == 0 && wt == 0) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = wr + 8 * k;
      if (r < rows) part_ml[(rowbase + r) * splits + split] = make_float2(row_m[r], lsum[k]);
    }
  }
  if (active) {
    // element i of acc[h]: row 4 g16 + i, coordinate 32 word + 16 h + n16
    const float f = fp.gamma * ldexpf(1.0f, ne);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g16 + i;
        if (r < rows) part_y[((rowbase + r) * splits + split) * dp + 32 * word + 16 * h + n16] = acc[h][i] * f;
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

// block per (group, query) row; dynamic LDS: d floats of the normalised sum
__global__ void __launch_bounds__(kThreads)
attn_merge_kernel(const float* __restrict__ part_y, const float2* __restrict__ part_ml, int64_t splits, int dp,
                  int d, const float* __restrict__ pi, float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float yh[];
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
  for (int c = tid; c < d; c += kThreads) {
    float a = 0.0f;
    for (int64_t s = 0; s < splits; ++s) a = fmaf(part_y[s * dp + c], wts[s], a);
    yh[c] = a * inv;
  }
  __syncthreads();
  for (int i = tid; i < d; i += kThreads) {
    float o = 0.0f;
    for (int c = 0; c < d; ++c) o = fmaf(pi[int64_t(c) * d + i], yh[c], o);
    out[row * d + i] = o;
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
  float scale;
  int64_t tps;
  int qchunks;
  ScoreForm fp;
  float* part_y;
  float2* part_ml;
  int64_t splits;
};

template <int B, int F>
hipError_t launch_pv(const PvArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_pv_kernel<B, F>), grid, dim3(kThreads), 0, s, a.scores, a.nq, a.n, a.vcodes, a.vnorms,
                     a.W, a.scale, a.tps, a.qchunks, a.fp, a.part_y, a.part_ml, a.splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_values(const tq_ctx* h, const uint32_t* codes, int64_t groups, int64_t n, uint32_t* vcodes,
                              hipStream_t stream) {
  const int64_t nb = (n + kTile - 1) / kTile;
  if (nb == 0 || groups == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_values_kernel, dim3(unsigned(nb), unsigned(groups)), dim3(kThreads), 0, stream, codes, n,
                     h->code_bits, h->words, nb, vcodes);
  return hipGetLastError();
}

// tokens per split: enough blocks to fill the GPU a few times over, at
// most kMaxSplits splits; TQ_ATTN_SPLIT=<tokens> overrides (tests use it to
// cover many splits)
int64_t attn_split_tokens(const tq_ctx* hv, int64_t groups, int64_t nq, int64_t n) {
  int64_t tps;
  if (const char* v = std::getenv("TQ_ATTN_SPLIT")) {
    tps = std::atoll(v);
  } else {
    const int64_t per = int64_t((hv->words + kWaves - 1) / kWaves) * groups * ((nq + kRows - 1) / kRows);
    const int64_t target = 4 * int64_t(hv->cus > 0 ? hv->cus : 256);
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
  const dim3 grid(unsigned(a.splits), unsigned((hv->words + kWaves - 1) / kWaves), unsigned(groups * a.qchunks));
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
  hipLaunchKernelGGL(attn_merge_kernel, dim3(unsigned(groups * nq)), dim3(kThreads), size_t(hv->d) * sizeof(float),
                     stream, a.part_y, a.part_ml, a.splits, 32 * hv->words, hv->d, hv->d_pi, out, lse);
  return hipGetLastError();
}

}  // namespace tqdev
