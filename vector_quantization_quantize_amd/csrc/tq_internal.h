// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/tq.h"

namespace tqdev {

constexpr int kMaxLevels = 16;  // bits <= 5  ->  B <= 4  ->  L <= 16

// Codebook passed by value to kernels; copied to LDS before use.
struct Codebook {
  float c[kMaxLevels];  // ascending levels
  float t[kMaxLevels];  // t[0 .. L-2] thresholds, rest +inf
  int levels;
};

// Coefficients of the level as a multilinear function of the plane signs.
// With s_p = 2 b_p - 1 (b_p = bit p of the index), a symmetric level set
// satisfies c[idx] = sum over odd-size plane subsets S of alpha_S prod s_p.
// For B <= 4 the odd subsets are: the B singletons and the C(B,3) triples.
struct PlaneExpansion {
  int count;            // number of terms
  uint32_t mask[8];     // plane subset of each term (bit p = plane p)
  float alpha[8];       // coefficient of each term
};

// Upper half of a level set that is exactly symmetric (c[L-1-i] = -c[i],
// t[L-2-i] = -t[i], middle threshold 0), times 2^12: index M + j holds
// m[j] and is chosen for z >= 0 with j = #{u_k <= z}; M = L / 2.
struct HalfCodebook {
  float u[kMaxLevels / 2];  // u[k] = 2^12 t[M + k], k < M - 1
  float m[kMaxLevels / 2];  // m[j] = 2^12 c[M + j],  j < M
};

// Level values the reconstruction's lookup table holds.  When the level set
// has at most two distinct magnitudes, a scale sigma (found at init) makes
// sigma c[level] a float16 number for every level, to within 2^-19 relative:
// one float16 piece per value is then enough and k_hat takes two matrix-core
// passes instead of three.
struct DequantTable {
  float v[kMaxLevels];  // sigma c[level], exactly representable in float16
  float out_scale;      // 1 / (sigma 2^12)
  int two_pass;         // 1 when v is in use
};

}  // namespace tqdev

struct tq_ctx {
  int d = 0, bits = 0, code_bits = 0, levels = 0, words = 0;
  int device = -1;
  int cus = 0;  // compute units of the device
  int lds_per_block = 0;  // bytes of LDS one workgroup may use
  // host copies (float32), row-major d x d
  std::vector<float> pi, g, centroids, thresholds;
  // device tables
  float* d_pi = nullptr;   // Pi  row-major: d_pi[j*d + i] = Pi[j][i]
  float* d_piT = nullptr;  // Pi^T row-major: d_piT[i*d + j] = Pi[j][i]
  float* d_g = nullptr;    // G   row-major
  float* d_gT = nullptr;   // G^T row-major
  float* d_piT128 = nullptr;  // Pi^T zero-padded to 128 x 128, d <= 128 only
  float* d_sT128 = nullptr;   // (G Pi)^T zero-padded to 128 x 128, d <= 128 only
  // d = 128 only: register fragments of the matrix-core quantize kernel
  uint16_t* d_pi_frag = nullptr;  // [word 4][step 8][piece 2][lane 64][8] f16 pieces of 2^12 Pi
  uint16_t* d_g_frag = nullptr;   // [word 4][step 8][piece 2][lane 64][8] f16 pieces of 2^10 G
  uint16_t* d_dq_frag = nullptr;  // [word 4][step 8][piece 2][lane 64][8] f16 pieces of 2^12 Pi (B operand)
  uint16_t* d_ds_frag = nullptr;  // the same for 2^10 S, S = G Pi (corrected reconstruction)
  tqdev::Codebook cb{};
  // fractional widths: rotated coordinates 0 .. hi-1 use cbh (2^(B+1)
  // levels); their extra index bit is one more plane of hi_words words
  // after the B full planes.  hi = hi_words = 0 for a plain handle.
  int hi = 0, hi_words = 0;
  std::vector<float> centroids_hi, thresholds_hi;
  tqdev::Codebook cbh{};
  tqdev::PlaneExpansion planes{};
  bool symmetric = false;  // level set exactly symmetric in float32
  tqdev::HalfCodebook half{};
  tqdev::HalfCodebook half_hi{};  // the finer set of coordinates below hi
  tqdev::PlaneExpansion planes_hi{};
  bool symmetric_hi = false;
  tqdev::DequantTable dqt{};
  // randomized Hadamard rotation (tq_init_hadamard): Pi = H diag(sigma) c
  // with c = float32(1 / sqrt(d)); d_hsigma holds sigma (float +-1)
  bool g_f16 = false;  // every entry of G is exact in float16
  int hadamard = 0;
  float hscale = 0.0f;
  float* d_hsigma = nullptr;
  // polar stage 1 (tq_init_polar): log2 d recursion levels; per level
  // (0-based) 48 floats: thresholds (+inf past L - 1), cos and sin of the
  // levels (float32 of the float64 values of the float32 levels)
  int polar = 0, polar_levels = 0;
  std::vector<float> polar_tab;
  float* d_polar_tab = nullptr;
  // general matrix-core quantizer (quantize_gemm.hip), d >= 16: operand
  // tiles of 2^12 Pi and 2^10 G as two float16 pieces,
  // [coord tile][K step][row 128][piece 2][16 halves]
  uint16_t* d_qpi_tiles = nullptr;
  uint16_t* d_qg_tiles = nullptr;
  // its scratch (residual pieces and rho^2 partials of one chunk of keys),
  // allocated at first use; a call on another stream waits for the event of
  // the last call that used it
  void* qscratch = nullptr;
  size_t qscratch_bytes = 0;
  hipEvent_t qscratch_done = nullptr;
  hipStream_t qscratch_stream = nullptr;
  bool qscratch_used = false;
  std::mutex qscratch_mu;
};

namespace tqdev {

// launchers (return hipError_t of the launch)
hipError_t launch_quantize_v1(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                              uint32_t* codes, uint32_t* signs, float* norms, float* rnorms,
                              hipStream_t stream);

hipError_t launch_query_prep(const tq_ctx* h, const float* queries, int64_t count, float* vw,
                             hipStream_t stream);

hipError_t launch_logits_v1(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq,
                            const uint32_t* codes, const uint32_t* signs, const float* norms,
                            const float* rnorms, int64_t n, float* scores, hipStream_t stream);

bool logits_lut128_supported(const tq_ctx* h);
hipError_t launch_logits_lut128(const tq_ctx* h, const float* queries, int64_t groups, int64_t nq,
                                const uint32_t* codes, const uint32_t* signs, const float* norms,
                                const float* rnorms, int64_t n, float* scores, hipStream_t stream);

// also requires 16-byte aligned keys and outputs (outputs are written as
// whole 16-byte rows)
// matrix-core scorer for many queries (d <= 256; one index bit needs a
// symmetric level set); vw from launch_query_prep
bool score_mfma_supported(const tq_ctx* h);
constexpr int64_t kScoreMfmaMinQueries = 16;  // below this the lookup-table scorer is used
hipError_t launch_score_mfma(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                             const uint32_t* signs, const float* norms, const float* rnorms, int64_t n,
                             float* scores, hipStream_t stream);

// General matrix-core quantizer (quantize_gemm.hip): any d >= kQGemmMinD,
// float32 or bfloat16 keys, plain or fractional-width handles.
constexpr int kQGemmMinD = 16;
bool quantize_gemm_supported(const tq_ctx* h);
// the operand tiles for tq_init (host, float64 products where needed)
int build_quantize_gemm_tiles(tq_ctx* h);
hipError_t launch_quantize_gemm(tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk, uint32_t* codes,
                                uint32_t* signs, float* norms, float* rnorms, hipStream_t stream);
void free_quantize_gemm(tq_ctx* h);

bool quantize_mfma128_supported(const tq_ctx* h, const void* keys, int key_dtype, int64_t ldk,
                                const void* codes, const void* signs, const void* norms, const void* rnorms);
hipError_t launch_quantize_mfma128(const tq_ctx* h, const void* keys, int64_t n, int64_t ldk, uint32_t* codes,
                                   uint32_t* signs, float* norms, float* rnorms, hipStream_t stream);

bool dequant_mfma128_supported(const tq_ctx* h);
hipError_t launch_dequant_mfma128(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n,
                                  float* khat, hipStream_t stream);

// TQ_KERNELS=ref selects the straightforward kernels everywhere (A/B checks)
bool force_reference_kernels();
// TQ_QUANTIZER=tiled: plain handles at 16 <= d <= 208 take the tiled general
// quantizer instead of the one-kernel form (A/B comparisons, tests of both)
bool force_tiled_quantizer();

// tq_logits after its argument checks (tq_api.cpp): check_logits_args
// returns TQ_OK for valid arguments (also for an empty request);
// run_logits launches with a workspace of tq_logits_workspace_size bytes
int check_logits_args(const tq_ctx* h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
                      const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores);
int run_logits(const tq_ctx* h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
               const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores,
               void* workspace, hipStream_t s);
// the static scratch of the allocation-free entry points (noalloc.hip):
// looks up its address on `device` (which must be current) once; TQ_OK or
// TQ_EHIP
int noalloc_prepare(int device);

// search: merge one chunk of scores ([nq][csize], keys c0 .. or, with
// chunk_i, the keys chunk_i holds; INT64_MAX marks an empty entry) into the
// running lists of the k best keys per query ([nq][k]); the last chunk writes
// the outputs instead (index -1, score -inf past the keys seen)
constexpr int kTopkMax = 64;
hipError_t launch_topk_merge(const float* chunk, const int64_t* chunk_i, int64_t nq, int64_t csize, int64_t c0,
                             int k, float* list_s, int64_t* list_i, bool last, float* out_s, int64_t* out_i,
                             hipStream_t stream);

// Forms of the level values in the matrix-core scorer: sign (one index bit,
// symmetric levels: c[1] times +-1), one float16 piece (sigma c[level], at
// most two magnitudes), two float16 pieces (2^10 c[level], hi and lo).
enum { kSignForm = 0, kOnePiece = 1, kTwoPiece = 2 };
struct ScoreForm {
  float val[kMaxLevels];  // one piece: sigma c[level]; two pieces: 2^10 c[level]
  float lambda;           // w rows are scaled lambda times the v rows
  float gamma;            // score = gamma / s_R * u for the row scale s_R
};
// one launch of the matrix-core scorer (scores form, or search form with topk)
struct ScoreArgs {
  const tq_ctx* h;
  const float* vw;
  int64_t groups, nq;
  const uint32_t* codes;
  const uint32_t* signs;
  const float* norms;
  const float* rnorms;
  int64_t n;           // keys scored per group
  int64_t key_stride;  // keys between groups in the packed arrays
  float* scores;       // scores form: [groups][nq][n]
  bool topk;         // search form
  float* part_s;     // search form: [groups][nq][splits][k]
  int64_t* part_i;
  int k;
  unsigned int* bound;  // search form, optional: [groups][nq] shared bounds, set to kBoundEmpty first
  void* qa;             // d > 256: float16 query rows [groups * nq][2 kp] (kp = d rounded up to 16)
  float* row_f;         // d > 256: score factor per query row
  ScoreForm form;
  int64_t qtiles, splits, tiles_per_block;  // grid (qtiles, splits, groups)
  hipStream_t stream;
};
inline size_t score_list_bytes(int k) { return size_t(128) * size_t(k) * (sizeof(float) + sizeof(int)); }
// per form (one translation unit each): launch, and the search kernel's
// static LDS bytes for dimension d
hipError_t score_launch_sign(const ScoreArgs& a);
hipError_t score_launch_one2(const ScoreArgs& a);
hipError_t score_launch_two2(const ScoreArgs& a);
hipError_t score_launch_two3(const ScoreArgs& a);
hipError_t score_launch_two4(const ScoreArgs& a);
size_t score_lds_sign(int d);
size_t score_lds_one2(int d);
size_t score_lds_two2(int d);
size_t score_lds_two3(int d);
size_t score_lds_two4(int d);
// d > 256: the tiled form (both operands through LDS), same forms
hipError_t score_gemm_launch_sign(const ScoreArgs& a);
hipError_t score_gemm_launch_one2(const ScoreArgs& a);
hipError_t score_gemm_launch_two2(const ScoreArgs& a);
hipError_t score_gemm_launch_two3(const ScoreArgs& a);
hipError_t score_gemm_launch_two4(const ScoreArgs& a);
size_t score_gemm_lds_sign();
size_t score_gemm_lds_one2();
size_t score_gemm_lds_two2();
size_t score_gemm_lds_two3();
size_t score_gemm_lds_two4();
constexpr int kScoreGemmMinD = 257;  // from this d on the tiled form runs

// search form of the matrix-core scorer: per block, the k best keys of each
// of its rows ([groups][nq][splits][k] scores and keys); merged afterwards
// with launch_topk_merge (csize = splits * k)
// Keys n of each group are scored (groups key_stride apart).  bound, when
// given ([groups][nq], each set to kBoundEmpty beforehand), lets the blocks
// that walk one row's keys share the best k-th score found so far.
constexpr unsigned int kBoundEmpty = 0x007FFFFFu;  // -inf in the order-preserving encoding
bool score_topk_mfma_supported(const tq_ctx* h, int64_t n, int k);
int64_t score_topk_mfma_splits(const tq_ctx* h, int64_t groups, int64_t nq, int64_t n);
hipError_t launch_score_topk_mfma(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq,
                                  const uint32_t* codes, const uint32_t* signs, const float* norms,
                                  const float* rnorms, int64_t n, int64_t key_stride, int k, unsigned int* bound,
                                  float* part_s, int64_t* part_i, hipStream_t stream);
// fill n words with a value (stream-ordered; no memset node in graphs)
hipError_t launch_fill_u32(unsigned int* p, int64_t n, unsigned int v, hipStream_t stream);

hipError_t launch_dequant_v1(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n,
                             float* khat, hipStream_t stream);

// polar handles (kernels_ref.hip): quantize, scores (vw from
// launch_query_prep) and the stage-1 reconstruction with the composed
// z_hat in place of c[idx]
constexpr int kPolarTab = 48;  // floats per level: thresholds, cos, sin (16 each)
hipError_t launch_quantize_polar(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                                 uint32_t* codes, uint32_t* signs, float* norms, float* rnorms, hipStream_t stream);
hipError_t launch_logits_polar(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                               const uint32_t* signs, const float* norms, const float* rnorms, int64_t n,
                               float* scores, hipStream_t stream);
hipError_t launch_dequant_polar(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n, float* khat,
                                hipStream_t stream);
// polar handles at d = 128 with one or two index bits per angle: the
// byte-table decode scorer (logits_polar.hip)
bool logits_polar128_supported(const tq_ctx* h);
// ... and its stage-1 reconstruction on the matrix cores (dequant_mfma.hip)
bool dequant_polar128_supported(const tq_ctx* h);
// plain handles with 16 <= d <= 208, d % 8 == 0, a seeded G, float32 or
// bf16 keys in 16-byte aligned rows: the one-kernel matrix-core quantizer
// (quantize_fused.hip)
bool quantize_fused_supported(const tq_ctx* h, const void* keys, int key_dtype, int64_t ldk);
hipError_t launch_quantize_fused(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                                 uint32_t* codes, uint32_t* signs, float* norms, float* rnorms, hipStream_t stream);
// polar handles at d = 128 with a seeded (float16-exact) G, float32 or
// bf16 keys in 16-byte aligned rows: the matrix-core quantizer
// (quantize_polar128.hip)
bool quantize_polar128_supported(const tq_ctx* h, const void* keys, int key_dtype, int64_t ldk);
hipError_t launch_quantize_polar128(const tq_ctx* h, const void* keys, int key_dtype, int64_t n, int64_t ldk,
                                    uint32_t* codes, uint32_t* signs, float* norms, float* rnorms,
                                    hipStream_t stream);
hipError_t launch_dequant_polar128(const tq_ctx* h, const uint32_t* codes, const float* norms, int64_t n, float* khat,
                                   hipStream_t stream);
hipError_t launch_logits_polar128(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                                  const uint32_t* signs, const float* norms, const float* rnorms, int64_t n,
                                  float* scores, hipStream_t stream);
// k_tilde = n Pi^T (c[idx] + rho sqrt(pi/2)/d G^T (2 beta - 1)); d = 128 on
// the matrix cores (dequant_mfma.hip), float32 otherwise (kernels_ref.hip)
hipError_t launch_dequant_prod_mfma128(const tq_ctx* h, const uint32_t* codes, const uint32_t* signs,
                                       const float* norms, const float* rnorms, int64_t n, float* out,
                                       hipStream_t stream);
hipError_t launch_dequant_prod_v1(const tq_ctx* h, const uint32_t* codes, const uint32_t* signs,
                                  const float* norms, const float* rnorms, int64_t n, float* out,
                                  hipStream_t stream);

// float offset between a query's v and w vectors in the workspace, and the
// stride between queries: v at q*vw_stride, w at q*vw_stride + vw_half
inline int64_t vw_half(int d) { return (int64_t(d) + 63) / 64 * 64; }
inline int64_t vw_stride(int d) { return 2 * vw_half(d); }

// Workspace of the query transform for `rows` query rows: the vw rows, then
// (d > 256, for the tiled matrix-core scorer) float16 query rows and one
// score factor per row.
inline size_t ws_align(size_t x) { return (x + 255) / 256 * 256; }
inline size_t score_vw_bytes(int d, int64_t rows) { return ws_align(size_t(rows) * size_t(vw_stride(d)) * 4); }
// float16 rows for `groups` groups of nq queries, padded to 128-row tiles
inline size_t score_qa_bytes(int d, int64_t groups, int64_t nq) {
  return ws_align(size_t(groups) * size_t((nq + 127) / 128 * 128) * size_t(2 * ((d + 15) / 16 * 16)) * 2);
}
inline size_t score_prep_bytes(int d, int64_t groups, int64_t nq) {
  const int64_t rows = groups * nq;
  return score_vw_bytes(d, rows) +
         (d >= kScoreGemmMinD ? score_qa_bytes(d, groups, nq) + ws_align(size_t(rows) * 4) : 0);
}

// Inner products with unquantized float32 (key_dtype 0) or bfloat16 (1)
// keys (dense_logits.hip)
hipError_t launch_dense_logits(const float* queries, int64_t groups, int64_t nq, const void* keys, int key_dtype,
                               int64_t n, int d, int64_t ldk, float* scores, hipStream_t stream);

// Decode attention (attention.hip).  Values in token blocks:
// vcodes[group][ceil(n/32)][B][32 W], bit i of word (b, p, j) = bit p of the
// index of coordinate j of token 32 b + i.
hipError_t launch_pack_values(const tq_ctx* h, const uint32_t* codes, int64_t groups, int64_t n, uint32_t* vcodes,
                              hipStream_t stream);
// tokens per key split of the value pass, and the bytes of its partial sums
int64_t attn_split_tokens(const tq_ctx* hv, int64_t groups, int64_t nq, int64_t n);
// one-kernel decode attention (scores by the byte tables and the value pass
// together) for a lookup-table key handle with up to 3 index bits and value
// codes of up to 3 bits at d in (96, 128]; TQ_ATTN_FUSED=0 turns it off.
// Its partials (one split per chunk, attn_fused_partial_bytes) take the
// place of the two-kernel form's; the caller checks that they fit.
bool attention_fused_supported(const tq_ctx* hk, const tq_ctx* hv);
size_t attn_fused_partial_bytes(const tq_ctx* hk, int64_t groups, int64_t nq, int64_t n);
hipError_t launch_attention_fused(const tq_ctx* hk, const tq_ctx* hv, const float* queries, int64_t groups,
                                  int64_t nq, const uint32_t* kcodes, const uint32_t* ksigns, const float* knorms,
                                  const float* krnorms, int64_t n, const uint32_t* vcodes, const float* vnorms,
                                  float scale, void* partials, float* out, float* lse, hipStream_t stream);
size_t attn_partial_bytes(const tq_ctx* hv, int64_t groups, int64_t nq, int64_t n);
// from scores [groups][nq][n]: softmax(scale s) over each row, weighted sum
// of the value reconstructions into out [groups][nq][d] and, if lse is not
// null, log sum exp(scale s) into lse [groups][nq]; n >= 1
hipError_t launch_attention_values(const tq_ctx* hv, const float* scores, int64_t groups, int64_t nq, int64_t n,
                                   const uint32_t* vcodes, const float* vnorms, float scale, void* partials,
                                   float* out, float* lse, hipStream_t stream);

}  // namespace tqdev
