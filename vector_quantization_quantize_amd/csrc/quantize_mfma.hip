// Matrix-core quantize kernel for d = 128 and bf16 keys (gfx950 MFMA).
//
// Stages ("TurboQuant tutorial" (gitcode.csdn.net), PolarQuant and QJL
// sections; "TurboQuant digest" (juejin.cn) section 2):
//   n = ||k||, z = Pi k / n, idx_j = #{t_i <= z_j}, r = z - c[idx],
//   rho = ||r||, beta = [G r > 0], packed into bit planes.
//
// Both projections are dense contractions and run on the matrix cores, with
// operands split so that the float32 result is as good as a float32 dot
// product:
//   * Keys: a key is staged as float16 times 2^s, where 2^s n lies in
//     [2^14, 2^15).  A bf16 value (8 significant bits) is then exact in
//     float16 unless it falls below the float16 normal range, i.e. below
//     2^-28 n, where the rounding error is under 2^-39 n.
//   * z' = (2^12 Pi)(2^s k): 2^12 Pi is split into two float16 pieces (22
//     significant bits, 2 MFMA passes), every product is exact and only the
//     float32 accumulation rounds; the representation error is at most
//     2^-22 ||Pi_i|| ||k||, i.e. 2^-22 in units of z.
//   * p = G r: r * 2^12 is split into two float16 pieces (22 bits).  A
//     seeded G has float16-exact entries, so G * 2^10 is one exact piece and
//     G r_hi + G r_lo (2 passes) rounds only in the accumulation; a G given
//     by the caller is split too and hi*hi + hi*lo + lo*hi (3 passes) leaves
//     an error near 2^-21 sum_j |G_mj r_j|.  The power-of-two scales do not
//     change signs.
//   * n = ||k|| in float32 from the bf16 key: sixteen-term partial sums in
//     eight lanes, then a three-level tree.
//
// Bucketize: the Lloyd-Max level set is symmetric, so z is placed by its
// magnitude among the upper half (index M + j for z >= 0, M - 1 - j below,
// M = 2^(B-1)); the residual z - c[idx] equals sign(z) (|z| - c[M + j])
// exactly.  Only exact ties at -t resolve to the lower cell, which the
// tie window allows.  Plane B-1 holds [z >= 0]; plane p < B-1 holds bit p of
// j, flipped for z < 0.  A sign bit of p = +0 (only possible when G r
// cancels exactly) is stored as 1, also inside the tie window.
//
// Fractional widths (a finer level set with one more index bit on the first
// hi = 64 coordinates): the two waves that own those coordinates bucketize
// with the finer set (same symmetric form, B + 1 bits) and write the extra
// index plane to the words after the B full planes of each code row; the
// other two waves run the ordinary passes.  Both kinds of wave go through
// the same passes and barriers.
//
// Work split: a block of 4 waves takes 32 keys at a time (one 32 x 32 x 16
// MFMA tile in N); wave w owns output coordinates [32w, 32w + 32), i.e. bit
// word w of every plane, and keeps its slices of Pi and G (two float16
// pieces each) in registers for the whole run.  The host permutes the rows
// of both slices so that accumulator element r of lane l is coordinate
// 32w + 16(l/32) + r: each lane's 16 bits of a word are contiguous.  The
// residual goes through LDS to every wave as the B operand of p = G r; the
// host orders G's columns so that the K-slots of each MFMA step match the
// coordinates a lane already holds (no register shuffles).
//
// Software pipeline, one barrier per tile: while the bucketize and residual
// arithmetic of tile i runs on the vector ALU, the matrix cores work on
// p = G r of tile i-1 and z' = Pi k of tile i+1; keys of tile i+2 are
// scaled and staged in the same pass from registers loaded a pass earlier.
// The pass is written as 40 slots of one MFMA plus a slice of vector work,
// separated by scheduling fences: left alone, the compiler issues all MFMAs
// first and the vector work after them, and nothing overlaps.
//
// Outputs go through LDS: each wave writes its words of a tile's rows (code
// rows, sign rows, norms and rnorms, 16 bytes each, in their memory order)
// to a staging area, and the next pass copies the area out with one 16-byte
// store per lane.  Written directly, every wave would issue B + 3 stores of
// 4-byte words strided by the row length, all in the same slots of every
// wave on the CU, and the store path would stall the pass.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "tq_internal.h"

namespace tqdev {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQThreads = 256;
constexpr int kSteps = 8;           // K = 128 in steps of 16
constexpr float kZScale = 4096.0f;  // z, levels, thresholds and residual carry a factor 2^12

#define TQ_SLOT_END() __builtin_amdgcn_sched_barrier(0)

__device__ __forceinline__ f32x16 mfma16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// Keep a value computed in the slot that produces it, and opaque: without
// this the compiler sinks the arithmetic into the slot that consumes it, or
// recomputes it in another form there.
#define TQ_PIN(x) asm volatile("" : "+v"(x))

// Two float16 pieces of a pair: hi = f16(e), lo = f16(e - hi).  e - hi is
// exact in float32; v_fma_mix forms it from the float16 hi and rounds once.
__device__ __forceinline__ void split_f16_pair(float e0, float e1, uint32_t& hi, uint32_t& lo) {
  const f16x2 h2 = {(_Float16)e0, (_Float16)e1};
  hi = __builtin_bit_cast(uint32_t, h2);
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(lo)
      : "v"(hi), "v"(e0), "v"(e1));
}

// f16(x0 * scale), f16(x1 * scale) packed, each rounded once (v_fma_mix)
__device__ __forceinline__ uint32_t scale_to_f16_pair(float x0, float x1, float scale) {
  uint32_t h;
  asm("v_fma_mixlo_f16 %0, %1, %3, 0\n\t"
      "v_fma_mixhi_f16 %0, %2, %3, 0"
      : "=&v"(h)
      : "v"(x0), "v"(x1), "v"(scale));
  return h;
}


// Bucketize one coordinate and return the residual times 2^12.  The
// coordinate arrives unscaled as a = 2^12 2^s n z; the thresholds 2^12 t are
// multiplied by the key's 2^s n (+inf for a zero key, whose z = 0 lies in
// cell M), inv = 1 / (2^s n), and 2^12 r = a inv - sign(a) 2^12 c[M + j].
// Bits go in from the least significant end: the sign of z into sgn (1 for
// z < 0), magnitude-index bit p into jw[p].
template <int B>
struct Quantizer {
  static constexpr int M = 1 << (B - 1);
  static constexpr int NJ = B > 1 ? B - 1 : 1;
  static constexpr int NU = M > 1 ? M - 1 : 1;
  float u[NU];  // 2^12 t[M + k], k < M - 1
  float m[M];   // 2^12 c[M + j]

  __device__ __forceinline__ float operator()(float a, float inv, const float (&us)[NU], uint32_t& sgn,
                                              uint32_t (&jw)[NJ]) const {
    const float aa = __builtin_fabsf(a);
    // binary descent, written out: compare with the middle threshold of the
    // remaining candidates; the comparison at depth q gives bit B-2-q of j
    float mj;
    if constexpr (B == 1) {
      mj = m[0];
    } else if constexpr (B == 2) {
      const bool b0 = aa >= us[0];
      jw[0] = jw[0] + jw[0] + (b0 ? 1u : 0u);
      mj = b0 ? m[1] : m[0];
    } else if constexpr (B == 3) {
      const bool b1 = aa >= us[1];
      const float t = b1 ? us[2] : us[0];
      const float lo = b1 ? m[2] : m[0];
      const float hi = b1 ? m[3] : m[1];
      const bool b0 = aa >= t;
      jw[1] = jw[1] + jw[1] + (b1 ? 1u : 0u);
      jw[0] = jw[0] + jw[0] + (b0 ? 1u : 0u);
      mj = b0 ? hi : lo;
    } else {
      const bool b2 = aa >= us[3];
      const float t1 = b2 ? us[5] : us[1];
      const float ta = b2 ? us[4] : us[0];
      const float tb = b2 ? us[6] : us[2];
      const float ma = b2 ? m[4] : m[0];
      const float mb = b2 ? m[5] : m[1];
      const float mc = b2 ? m[6] : m[2];
      const float md = b2 ? m[7] : m[3];
      const bool b1 = aa >= t1;
      const float t0 = b1 ? tb : ta;
      const float me = b1 ? mc : ma;
      const float mf = b1 ? md : mb;
      const bool b0 = aa >= t0;
      jw[2] = jw[2] + jw[2] + (b2 ? 1u : 0u);
      jw[1] = jw[1] + jw[1] + (b1 ? 1u : 0u);
      jw[0] = jw[0] + jw[0] + (b0 ? 1u : 0u);
      mj = b0 ? mf : me;
    }
    sgn = __builtin_amdgcn_alignbit(sgn, as_u32(a), 31);
    // a inv - sign(a) m = sign(a) (|a| inv - m): negation does not change the
    // rounding.  The opaque copy keeps the negation on the fma's operand
    // modifier instead of an integer xor.
    float c = __builtin_copysignf(mj, a);
    asm("" : "+v"(c));
    return __builtin_fmaf(a, inv, -c);
  }
};

// G3: G needs two float16 pieces (three passes for p = G r); without it
// (G exact in float16) the G lo pass is skipped.  HW: words of the extra
// index plane of fractional widths (hi = 32 HW coordinates with the finer
// level set hch and one more index bit; waves w < HW own exactly those
// coordinates), 0 for one level set.
// Two waves per SIMD (two blocks per CU) and no more: the slices of Pi and
// G stay in registers, so the register budget is that of two waves.
template <int B, bool G3, int HW>
__global__ void __launch_bounds__(kQThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
quantize_mfma128_kernel(const uint16_t* __restrict__ keys, int64_t n, int64_t ldk,
                        const uint4* __restrict__ pi_frag, const uint4* __restrict__ g_frag, HalfCodebook hc,
                        HalfCodebook hch, uint32_t* __restrict__ codes, uint32_t* __restrict__ signs, float* __restrict__ norms,
                        float* __restrict__ rnorms, int64_t tiles, int64_t half, int64_t lead_tiles) {
  using Q = Quantizer<B>;
  // scaled float16 keys, double buffered: 32 rows of 128 halves, row stride
  // 272 bytes so that the 8 lanes of one LDS pass hit distinct banks
  __shared__ uint4 ktile[2][32][17];
  __shared__ float4 kinfo[2][32];  // (1 / (2^s n), n, 2^s n or +inf for n = 0, 0) per key
  // residual exchange [buf][piece][step][lane group][key] (8 halves each)
  __shared__ uint4 xb[2][2][kSteps][2][32];
  __shared__ float rsq[2][4][32];
  // output staging, by tile parity: the tile's code block (32 code rows of
  // CR words), the previous tile's 32 sign rows, 8 rows of this tile's
  // norms, 8 rows of the previous tile's rnorms (16 bytes each, the order
  // they have in memory)
  constexpr int CR = 4 * B + HW;  // words of a key's code row
  constexpr int kOutRows = 8 * CR + 48;
  constexpr int kRowS = 8 * CR, kRowN = kRowS + 32, kRowR = kRowN + 8;
  __shared__ uint4 ost[2][kOutRows];

  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kl = lane & 31;
  const int g = lane >> 5;

  f16x8 api[kSteps][2], ag[kSteps][2];
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      api[s][q] = __builtin_bit_cast(f16x8, pi_frag[((w * kSteps + s) * 2 + q) * 64 + lane]);
      ag[s][q] = G3 || q == 0 ? __builtin_bit_cast(f16x8, g_frag[((w * kSteps + s) * 2 + q) * 64 + lane])
                              : f16x8{};
    }
  // the finer level set (one more index bit) of the waves below HW
  using QF = Quantizer<(HW > 0 ? B + 1 : B)>;

  // staging: thread t owns bf16 elements [16 (t % 8), +16) of key t / 8.
  // Rows are fetched in tile order, one call per tile.  Rows past the end
  // re-read the last key: their outputs are never stored and a key's results
  // depend on its own row only, so no zero fill (and no branch that would
  // split the pipelined loop body) is needed.
  const int sk = threadIdx.x >> 3, sc = threadIdx.x & 7;
  // This block's tiles: tstart, tstart + tstride, ... (ntile >= 1 of them).
  // Blocks [0, half) walk the tiles [0, lead_tiles), the others the rest.
  const int64_t bid = blockIdx.x;
  const bool leads = bid < half;
  const int64_t tstart = leads ? bid : lead_tiles + (bid - half);
  const int64_t tstride = half;
  const int64_t ntile = ((leads ? lead_tiles : tiles) - tstart + tstride - 1) / tstride;
  const uint4* const row_last = reinterpret_cast<const uint4*>(keys + (n - 1) * ldk) + 2 * sc;
  const int64_t row_step = tstride * 32 * ldk / 8;  // in uint4
  const uint4* row_next = reinterpret_cast<const uint4*>(keys + (tstart * 32 + sk) * ldk) + 2 * sc;
  auto fetch = [&](uint4& a, uint4& b) {
    const uint4* src = row_next < row_last ? row_next : row_last;
    a = src[0];
    b = src[1];
    row_next += row_step;
  };
  // staging pieces: unpack + partial sum of squares, norm and scale, convert
  // Staging is one dependency chain (unpack, sum of squares, 8-lane
  // reduction, square root, scale, convert); its steps are small functions
  // so that the pipelined pass can put each in its own slot, away from the
  // step it waits for.
  struct Stage {
    float x[16];
    float part[4];  // partial sums of squares: two chains per 8 values
    float ss, nk, inv, ns, scale;
  };
  auto stage_unpack = [&](Stage& st, const uint4& v, int half) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.x[8 * half + 2 * i] = as_f32(u[i] << 16);
      st.x[8 * half + 2 * i + 1] = as_f32(u[i] & 0xFFFF0000u);
      // bf16 products are exact in float32
      const bf16x2 b2 = __builtin_bit_cast(bf16x2, u[i]);
      float& acc = st.part[2 * half + (i & 1)];
      acc = __builtin_amdgcn_fdot2_f32_bf16(b2, b2, i < 2 ? 0.0f : acc, false);
    }
  };
  auto stage_sum = [&](Stage& st) { st.ss = (st.part[0] + st.part[1]) + (st.part[2] + st.part[3]); };
  // one level of the sum over the 8 lanes of an aligned group: quad xor 1,
  // quad xor 2, then the mirror within each half row (lane i <-> 7 - i)
  auto stage_reduce = [&](Stage& st, int level) {
    const int x = static_cast<int>(as_u32(st.ss));
    const int y = level == 0   ? __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false)
                  : level == 1 ? __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false)
                               : __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
    st.ss += as_f32(static_cast<uint32_t>(y));
  };
  auto stage_norm = [&](Stage& st) {
    // 2^sh nk in [2^14, 2^15); nk == 0 gives sh = 15 and zero keys.  The
    // hardware square root and reciprocal are within 1 ulp.
    st.nk = __builtin_amdgcn_sqrtf(st.ss);
    const int sh = 15 - __builtin_amdgcn_frexp_expf(st.nk);
    st.scale = __builtin_amdgcn_ldexpf(1.0f, sh);
    st.ns = st.nk > 0.0f ? __builtin_amdgcn_ldexpf(st.nk, sh) : __builtin_inff();
    st.inv = st.nk > 0.0f ? __builtin_amdgcn_rcpf(st.ns) : 0.0f;
  };
  auto stage_store = [&](const Stage& st, int buf, int half) {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = scale_to_f16_pair(st.x[8 * half + 2 * i], st.x[8 * half + 2 * i + 1], st.scale);
    ktile[buf][sk][2 * sc + half] = make_uint4(h[0], h[1], h[2], h[3]);
    if (half == 1) kinfo[buf][sk] = make_float4(st.inv, st.nk, st.ns, 0.0f);  // the 8 lanes write the same value
  };
  auto stage_all = [&](const uint4& a, const uint4& b, int buf) {
    Stage st;
    stage_unpack(st, a, 0);
    stage_unpack(st, b, 1);
    stage_sum(st);
    stage_reduce(st, 0);
    stage_reduce(st, 1);
    stage_reduce(st, 2);
    stage_norm(st);
    stage_store(st, buf, 0);
    stage_store(st, buf, 1);
  };

  // prologue: tiles 0 and 1 staged, tile 2 in flight
  uint4 na, nb;
  {
    uint4 a0, b0, a1, b1;
    fetch(a0, b0);
    fetch(a1, b1);
    fetch(na, nb);
    stage_all(a0, b0, 0);
    stage_all(a1, b1, 1);
    // the first pass runs p = G r on buffer 1 before any residual is there
    uint4* x1 = &xb[1][0][0][0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) x1[j * kQThreads + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  float4 info = kinfo[0][kl];
  f32x16 acc1 = {};
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const f16x8 kf = __builtin_bit_cast(f16x8, ktile[0][kl][2 * s + g]);
    acc1 = mfma16(api[s][1], kf, acc1);
    acc1 = mfma16(api[s][0], kf, acc1);
  }

  // Copy-out: wave w moves rows [w R, w R + R) of a staged tile, R = kOutRows
  // / 4, one per lane (lanes past R repeat the last one: same address, same
  // value).  Code rows and norms belong to the tile of the previous pass
  // (tile c), sign rows and rnorms to the tile before it (c - 1 of this
  // block), which a lane's store pointer lags by.
  constexpr int kOutWave = kOutRows / 4;
  const int orow = w * kOutWave + (lane < kOutWave ? lane : kOutWave - 1);
  uint4* const codes4 = reinterpret_cast<uint4*>(codes);
  uint4* const signs4 = reinterpret_cast<uint4*>(signs);
  uint4* const norms4 = reinterpret_cast<uint4*>(norms);
  uint4* const rnorms4 = reinterpret_cast<uint4*>(rnorms);
  // destination of staged row r when tile c (global tile index) is the tile
  // of the code rows
  auto out_ptr = [&](int r, int64_t c) -> uint4* {
    const int64_t pc = c - tstride;
    if (r < kRowS) return codes4 + c * (8 * CR) + r;
    if (r < kRowN) return signs4 + pc * 32 + (r - kRowS);
    if (r < kRowR) return norms4 + c * 8 + (r - kRowN);
    return rnorms4 + pc * 8 + (r - kRowR);
  };
  const int64_t ostep = (orow < kRowS ? 8 * CR : orow < kRowN ? 32 : 8) * tstride;
  uint4* optr = nullptr;  // this lane's destination in the next copy-out (from the third pass on)

  // Lanes l and l ^ 32 hold the low and high 16 bits of a word; every lane
  // gets the whole word (v_permlane32_swap hands each half to both lanes).
  auto whole = [](uint32_t x) {
    const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return h[0] | (h[1] << 16);
  };
  auto both_sum = [](float x) {
    const auto h = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
    return as_f32(h[0]) + as_f32(h[1]);
  };
  auto rnorm_of = [&](int b) {
    const float* q = rsq[b][0];
    return __builtin_amdgcn_sqrtf((q[kl] + q[32 + kl]) + (q[64 + kl] + q[96 + kl])) * (1.0f / kZScale);
  };

  // One pass: tile i's vector work beside p of tile i-1 and z' of tile i+1,
  // and the copy-out of the rows staged by pass i-1.  buf = i % 2 is a
  // compile-time constant (the loop is unrolled by two), and so is the phase:
  // 0 for the first pass (no tile i-1, nothing staged), 1 for the second
  // (staged sign rows and rnorms belong to no tile: those lanes repeat a code
  // or norm row instead), 2 after.  Every tile but the last of the block is
  // full, so copy-outs need no bounds.
  auto pass = [&](int64_t i, auto bufc, auto phasec, auto finec) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    constexpr int phase = decltype(phasec)::value;
    constexpr bool fine = decltype(finec)::value;  // this wave's coordinates take the finer set
    using QP = std::conditional_t<fine, QF, Q>;
    // the wave's level set, from the kernel arguments (uniform values)
    const HalfCodebook& hq = fine ? hch : hc;
    QP qz;
#pragma unroll
    for (int k = 0; k < QP::M; ++k) qz.m[k] = hq.m[k];
#pragma unroll
    for (int k = 0; k + 1 < QP::M; ++k) qz.u[k] = hq.u[k];
    constexpr int NP = fine ? B + 1 : B;  // index planes of this wave's coordinates
    constexpr bool first = phase == 0;
    constexpr int ob = buf ^ 1;
    uint4 ov;       // staged row of this lane
    uint4* odst;    // and where it goes
    int lrow = orow;

    // ---- slot 0: operands of the first MFMAs, and while they load, the
    // thresholds scaled to the key and the first coordinate pair
    f16x8 rh = __builtin_bit_cast(f16x8, xb[ob][0][0][g][kl]);
    f16x8 rl = __builtin_bit_cast(f16x8, xb[ob][1][0][g][kl]);
    const f32x16 zt = acc1;
    const float inv = info.x, nrm = info.y;
    float us[QP::NU];
#pragma unroll
    for (int k = 0; k + 1 < QP::M; ++k) us[k] = qz.u[k] * info.z;
    uint32_t sgn = 0u, jw[QP::NJ];
#pragma unroll
    for (int p = 0; p < QP::NJ; ++p) jw[p] = 0u;
    float e[16];  // scaled residuals, coordinates processed from 15 down
    e[15] = qz(zt[15], inv, us, sgn, jw);
    e[14] = qz(zt[14], inv, us, sgn, jw);
    TQ_PIN(e[15]);
    TQ_PIN(e[14]);
    TQ_SLOT_END();

    // ---- slots 1-24: p = G r of tile i-1 (3 MFMAs per step) beside the
    // bucketize of tile i: step s quantizes pair s + 1 and packs pair s
    f32x16 acc2 = {};
    float rr = 0.0f;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int r1 = 15 - 2 * s, r0 = r1 - 1;  // pair s
      f16x8 nrh = rh, nrl = rl;
      if (s + 1 < kSteps) nrh = __builtin_bit_cast(f16x8, xb[ob][0][s + 1][g][kl]);
      if constexpr (G3) acc2 = mfma16(ag[s][1], rh, acc2);
      if (s + 1 < kSteps) {
        e[r1 - 2] = qz(zt[r1 - 2], inv, us, sgn, jw);
        TQ_PIN(e[r1 - 2]);
      }
      if constexpr (phase == 1) {
        if (s == 0) {
          // the staged tile is this block's first: no previous tile
          lrow = orow < kRowS ? orow : orow < kRowN ? orow - kRowS : orow < kRowR ? orow : orow - 8;
          odst = out_ptr(lrow, tstart);
          optr = out_ptr(orow, tstart + tstride);
        }
      } else if constexpr (phase == 2) {
        if (s == 0) {
          odst = optr;
          optr += ostep;
        }
      }
      if constexpr (!first) {
        if (s == 1) ov = ost[ob][lrow];
        if (s == 3) *odst = ov;
      }
      TQ_SLOT_END();
      if (s + 1 < kSteps) nrl = __builtin_bit_cast(f16x8, xb[ob][1][s + 1][g][kl]);
      acc2 = mfma16(ag[s][0], rl, acc2);
      if (s + 1 < kSteps) {
        e[r0 - 2] = qz(zt[r0 - 2], inv, us, sgn, jw);
        TQ_PIN(e[r0 - 2]);
      }
      TQ_SLOT_END();
      acc2 = mfma16(ag[s][0], rh, acc2);
      rr = fmaf(e[r1], e[r1], rr);
      rr = fmaf(e[r0], e[r0], rr);
      split_f16_pair(e[r0], e[r1], hi[(r0 & 7) >> 1], lo[(r0 & 7) >> 1]);
      if ((r0 & 7) == 0) {
        xb[buf][0][2 * w + (r0 >> 3)][g][kl] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        xb[buf][1][2 * w + (r0 >> 3)][g][kl] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
      TQ_SLOT_END();
      rh = nrh;
      rl = nrl;
    }

    // ---- slots 25-40: z' of tile i+1 (2 MFMAs per step) beside staging of
    // tile i+2, the sign bits of tile i-1, word assembly and the stores
    info = kinfo[ob][kl];
    f16x8 kf = __builtin_bit_cast(f16x8, ktile[ob][kl][g]);
    f32x16 a1 = {};
    Stage st;
    uint32_t sw = 0u;
    uint32_t word[NP + 1];  // index planes 0..NP-1, then the sign word of tile i-1
    float prn = 0.0f;      // rho of tile i-1
    f16x8 nkf = kf;        // next step's keys, read one step ahead
#pragma unroll
    for (int j = 0; j < 2 * kSteps; ++j) {
      const int s = j >> 1;
      if ((j & 1) == 0 && s + 1 < kSteps) nkf = __builtin_bit_cast(f16x8, ktile[ob][kl][2 * (s + 1) + g]);
      a1 = mfma16(api[s][(j & 1) ? 0 : 1], kf, a1);
      // dependent staging steps sit at least one slot apart, with independent
      // work (sign bits, word assembly, stores) between them
      switch (j) {
        case 0: stage_unpack(st, na, 0); break;
        case 1: stage_unpack(st, nb, 1); break;
        case 2:
#pragma unroll
          for (int r = 15; r >= 8; --r) sw = __builtin_amdgcn_alignbit(sw, as_u32(acc2[r]), 31);
          break;
        case 3: stage_sum(st); break;
        case 4:
#pragma unroll
          for (int r = 7; r >= 0; --r) sw = __builtin_amdgcn_alignbit(sw, as_u32(acc2[r]), 31);
          break;
        case 5: stage_reduce(st, 0); break;
        case 6:
          // 16-bit halves: plane B-1 = [z >= 0], plane p = j_p ^ [z < 0],
          // signs = [p > 0]
#pragma unroll
          for (int p = 0; p + 1 < NP; ++p) word[p] = jw[p] ^ sgn;
          word[NP - 1] = sgn ^ 0xFFFFu;
          word[NP] = sw ^ 0xFFFFu;
          if (!first) prn = rnorm_of(ob);
          break;
        case 7: stage_reduce(st, 1); break;
        case 8:
#pragma unroll
          for (int p = 0; p <= NP; ++p) word[p] = whole(word[p]);
          break;
        case 9: stage_reduce(st, 2); break;
        case 10: rsq[buf][w][kl] = both_sum(rr); break;
        case 11: stage_norm(st); break;
        case 12: {
          // word w of this tile's code rows (planes 0..B-1 at 4 p + w, the
          // extra plane of the finer coordinates at 4 B + w) and of the
          // previous tile's sign rows (lane group g takes every other word;
          // with an even count the last word goes twice), this tile's norm
          // (g = 0) and the previous tile's rho (g = 1)
          uint32_t* o32 = reinterpret_cast<uint32_t*>(ost[buf]);
          auto addr = [&](int p) {
            return p < B ? kl * CR + 4 * p + w : p < NP ? kl * CR + 4 * B + w : (kRowS + kl) * 4 + w;
          };
#pragma unroll
          for (int q = 0; 2 * q <= NP; ++q) {
            const int p0 = 2 * q, p1 = 2 * q + 1 <= NP ? 2 * q + 1 : NP;
            o32[g ? addr(p1) : addr(p0)] = g ? word[p1] : word[p0];
          }
          reinterpret_cast<float*>(&ost[buf][kRowN])[32 * g + kl] = g ? prn : nrm;
          break;
        }
        case 13: stage_store(st, buf, 0); break;
        case 14: stage_store(st, buf, 1); break;
        case 15: fetch(na, nb); break;  // tile i + 3
        default: break;
      }
      TQ_SLOT_END();
      if (j & 1) kf = nkf;
    }
    acc1 = a1;
    __syncthreads();
  };
  // After the last pass (tile i): the rows it staged, bounded by n since its
  // tile may be the ragged last one, then p of tile i and its sign words and
  // rho, written directly (rows past the end go to key n - 1, same value).
  auto finish = [&](int64_t i, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int64_t c = tstart + i * tstride;
    const int64_t left = n - c * 32;
    const int vk = left < 32 ? static_cast<int>(left) : 32;  // keys of tile c
    const uint4 v = ost[buf][orow];
    if (orow < kRowS) {
      // the code words of the tile's vk keys (a row may end inside one)
      const int vw = vk * CR;
      if (4 * orow + 4 <= vw) {
        *out_ptr(orow, c) = v;
      } else if (4 * orow < vw) {
        uint32_t* d32 = reinterpret_cast<uint32_t*>(out_ptr(orow, c));
        const int left = vw - 4 * orow;  // 1 .. 3
        d32[0] = v.x;
        if (left > 1) d32[1] = v.y;
        if (left > 2) d32[2] = v.z;
      }
    } else if (orow < kRowN || orow >= kRowR) {
      if (i > 0) *out_ptr(orow, c) = v;  // the tile before c, if any
    } else {
      const int k0 = 4 * (orow - kRowN);
      float* dn = norms + c * 32 + k0;
      const float nv[4] = {as_f32(v.x), as_f32(v.y), as_f32(v.z), as_f32(v.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k0 + e < vk) dn[e] = nv[e];
    }
    const int64_t key = c * 32 + kl;
    const int64_t kc = key < n ? key : n - 1;
    f32x16 acc2 = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const f16x8 rh = __builtin_bit_cast(f16x8, xb[buf][0][s][g][kl]);
      const f16x8 rl = __builtin_bit_cast(f16x8, xb[buf][1][s][g][kl]);
      if constexpr (G3) acc2 = mfma16(ag[s][1], rh, acc2);
      acc2 = mfma16(ag[s][0], rl, acc2);
      acc2 = mfma16(ag[s][0], rh, acc2);
    }
    uint32_t sw = 0u;
#pragma unroll
    for (int r = 15; r >= 0; --r) sw = __builtin_amdgcn_alignbit(sw, as_u32(acc2[r]), 31);
    signs[kc * 4 + w] = whole(sw ^ 0xFFFFu);
    rnorms[kc] = rnorm_of(buf);
  };
  constexpr std::integral_constant<int, 0> kBuf0{};
  constexpr std::integral_constant<int, 1> kBuf1{};
  constexpr std::integral_constant<int, 0> kFirst{};
  constexpr std::integral_constant<int, 1> kSecond{};
  constexpr std::integral_constant<int, 2> kLater{};
  // the same sequence of passes and barriers for every wave; waves whose
  // coordinates take the finer level set run the passes built for it
  auto run = [&](auto finec) __attribute__((always_inline)) {
    pass(0, kBuf0, kFirst, finec);
    if (ntile == 1) {
      finish(0, kBuf0);
      return;
    }
    pass(1, kBuf1, kSecond, finec);
    int64_t i = 2;
    for (; i + 1 < ntile; i += 2) {
      pass(i, kBuf0, kLater, finec);
      pass(i + 1, kBuf1, kLater, finec);
    }
    if (i < ntile) {
      pass(i, kBuf0, kLater, finec);
      finish(i, kBuf0);
    } else {
      finish(i - 1, kBuf1);
    }
  };
  if constexpr (HW > 0) {
    if (__builtin_amdgcn_readfirstlane(w) < HW)
      run(std::true_type{});
    else
      run(std::false_type{});
  } else {
    run(std::false_type{});
  }
}

// share of the tiles taken by the first-dispatched half of the grid, by B
constexpr double kLeadShare[4] = {0.65, 0.65, 0.65, 0.65};

template <int B>
hipError_t launch_b(const tq_ctx* h, const void* keys, int64_t n, int64_t ldk, uint32_t* codes, uint32_t* signs,
                    float* norms, float* rnorms, hipStream_t stream) {
  const int64_t tiles = (n + 31) / 32;
  // Two blocks fit on a CU, and the grid is one resident wave of them.  The
  // CU's wave arbiter favours older waves, so the block dispatched first to a
  // CU (the grid's first half, one per CU) runs well ahead of its partner;
  // with equal shares the partner finishes long after it, alone on the CU.
  // The first half therefore takes a fixed larger share of the tiles (the
  // front range), the second half the rest.  The split only moves work
  // between blocks; any dispatch order gives the same results.
  const int64_t slots = 2 * static_cast<int64_t>(h->cus);
  int64_t blocks, half, lead;
  if (tiles >= 4 * slots) {
    blocks = slots;
    half = slots / 2;
    lead = static_cast<int64_t>(static_cast<double>(tiles) * kLeadShare[B - 1] + 0.5);
    lead = lead < half ? half : lead > tiles - half ? tiles - half : lead;
  } else {  // few tiles per block: equal shares, one sequence
    blocks = tiles < slots ? tiles : slots;
    half = blocks;
    lead = tiles;
  }
  auto kernel = h->g_f16 ? quantize_mfma128_kernel<B, false, 0> : quantize_mfma128_kernel<B, true, 0>;
  if (h->hi > 0) {
    // fractional widths: hi = 64, seeded G (checked by the caller)
    if constexpr (B <= 3)
      kernel = quantize_mfma128_kernel<B, false, 2>;
    else
      return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kQThreads), 0, stream,
                     static_cast<const uint16_t*>(keys), n, ldk, reinterpret_cast<const uint4*>(h->d_pi_frag),
                     reinterpret_cast<const uint4*>(h->d_g_frag), h->half, h->half_hi, codes, signs, norms, rnorms,
                     tiles, half, lead);
  return hipGetLastError();
}

}  // namespace

bool quantize_mfma128_supported(const tq_ctx* h, const void* keys, int key_dtype, int64_t ldk,
                                const void* codes, const void* signs, const void* norms, const void* rnorms) {
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  // fractional widths: the finer set on the first 64 coordinates (two waves'
  // words), symmetric too, B + 1 <= 4 index bits there, seeded G
  const bool widths = h->hi == 0 || (h->hi == 64 && h->symmetric_hi && h->g_f16 && h->code_bits <= 3);
  return h->d == 128 && widths && key_dtype == TQ_BF16 && h->d_pi_frag && h->d_g_frag && h->symmetric && ldk >= 128 &&
         (ldk % 8) == 0 && a16(keys) && a16(codes) && a16(signs) && a16(norms) && a16(rnorms) &&
         h->code_bits >= 1 && h->code_bits <= 4;
}

hipError_t launch_quantize_mfma128(const tq_ctx* h, const void* keys, int64_t n, int64_t ldk, uint32_t* codes,
                                   uint32_t* signs, float* norms, float* rnorms, hipStream_t stream) {
  switch (h->code_bits) {
    case 1: return launch_b<1>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    case 2: return launch_b<2>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    case 3: return launch_b<3>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    case 4: return launch_b<4>(h, keys, n, ldk, codes, signs, norms, rnorms, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqdev
