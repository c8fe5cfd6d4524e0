/*
 * tq.h - C ABI of libtq, a gfx950 (AMD Instinct MI355X) implementation of the
 * TurboQuant quantize / score path.
 *
 * The method (sources are web pages about TurboQuant, cited by title and
 * section):
 *   - "TurboQuant digest" (juejin.cn), section 2: a key is randomly rotated so
 *     that a scalar quantizer suits every coordinate; this stage spends most
 *     of the bits.  About one more bit per coordinate is a QJL sign sketch of
 *     the residual, read back by an asymmetric estimator that pairs the
 *     low-bit key with a high-precision query.
 *   - "TurboQuant tutorial" (gitcode.csdn.net), sections PolarQuant and QJL:
 *     the length is kept at higher precision; each rotated coordinate is
 *     replaced by the nearest allowed value; the residual is multiplied by a
 *     Gaussian JL matrix with as many outputs as inputs and only the signs
 *     are kept (positive -> 1, negative -> 0); a 2-bit (3-bit) first stage
 *     makes 3 (4) bits in all, one of them the QJL bit.
 *   - "TurboQuant deep review" (freelamp.com), breakthrough and error
 *     compensation sections: random orthogonal preconditioning, no per-block
 *     scale constants, and a zero-bias estimate of the attention score.
 *
 * Concretely, with B = bits - 1 codebook bits, L = 2^B levels, a key k in R^d
 * and W = ceil(d / 32):
 *   n    = ||k||_2,  u = k / n  (u = 0 when n = 0)
 *   z    = Pi u                      Pi: d x d Haar rotation from the seed
 *   idx  = #{ i : t_i <= z_j }       t: L-1 float32 thresholds (midpoints of
 *                                    the float32 Lloyd-Max levels c for the
 *                                    law of one coordinate of a uniform unit
 *                                    vector in R^d)
 *   r    = z - c[idx],  rho = ||r||_2
 *   p    = G r,  beta_j = [p_j > 0]  G: d x d iid N(0,1) from the seed
 *   score(q) = n * ( <Pi q, c[idx]> + rho * sqrt(pi/2) / d * <G Pi q, 2 beta - 1> )
 *   k_hat    = n * Pi^T c[idx]       (stage-1 reconstruction)
 *
 * Seeded draws: SplitMix64 (Steele, Lea & Flood 2014) with golden gamma
 * g = 0x9E3779B97F4A7C15.  Stream s (0 = Pi, 1 = G) of seed x starts from
 * state fmix(x + (s+1) g); its counter c (0-based) is fmix(state + (c+1) g).
 * Normal pair i of a stream uses counters 2i, 2i+1 in Box-Muller form
 * (u1 = ((a>>11)+1) 2^-53, u2 = (b>>11) 2^-53, R = sqrt(-2 ln u1); element
 * 2i = R cos(2 pi u2), 2i+1 = R sin(2 pi u2)), filling a d x d matrix in row
 * order.  Pi = Q diag(sign(diag R)) from the Householder QR of the stream-0
 * matrix, in float64, then rounded to float32; G is the stream-1 matrix
 * rounded to float16 precision (11 significant bits, round to nearest even,
 * held as float32), so that the matrix cores multiply by it exactly.
 *
 * Packed layout (format version 1), all arrays dense and 4-byte aligned:
 *   codes [n][B][W] uint32   bit p of idx_j at plane p, word j/32, bit j%32
 *   signs [n][W]    uint32   beta_j at word j/32, bit j%32
 *   norms [n]       float32  n
 *   rnorms[n]       float32  rho
 * Bits past d in the last word are 0.
 *
 * Conventions for every entry point:
 *   - Return 0 (TQ_OK) or a negative TQ_E* code; nothing aborts and no C++
 *     exception crosses the ABI.  tq_strerror() names a code.
 *   - "device" pointers are HIP device memory of the device the handle was
 *     created on (hipGetDevice() at tq_init); "host" pointers are ordinary
 *     host memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device work is
 *     enqueued asynchronously on it; launch errors are returned, faults
 *     surface at the caller's synchronisation.
 *   - The caller owns every buffer passed in; the library owns only what
 *     tq_init allocates (the rotation, projection and codebook tables) and
 *     frees it in tq_destroy.  A handle is read-only after tq_init, so calls
 *     on different streams may share it.
 *   - n = 0 (or groups = 0, nq = 0) is a successful no-op.  NaN or Inf in
 *     inputs gives unspecified codes and scores.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define TQ_API __attribute__((visibility("default")))
#else
#define TQ_API
#endif

#define TQ_OK 0
#define TQ_EINVAL (-1)       /* bad argument (null pointer, size, range)   */
#define TQ_EUNSUPPORTED (-2) /* valid but not implemented                  */
#define TQ_EHIP (-3)         /* a HIP runtime call or kernel launch failed */
#define TQ_ENOMEM (-4)       /* host or device allocation failed           */
#define TQ_ESCRATCH (-5)     /* request larger than the static scratch     */

#define TQ_FORMAT_VERSION 1

/* element type of the keys given to tq_quantize */
#define TQ_F32 0
#define TQ_BF16 1

typedef struct tq_ctx* tq_handle;

typedef struct {
  int32_t d;              /* vector dimension                                 */
  int32_t bits;           /* total bits per coordinate (B + 1)                */
  int32_t code_bits;      /* B                                                */
  int32_t levels;         /* L = 2^B                                          */
  int32_t words;          /* W = ceil(d / 32)                                 */
  int32_t format_version; /* TQ_FORMAT_VERSION                                */
  int64_t code_bytes;     /* bytes of codes per key  = 4 (B W + hi_words)     */
  int64_t sign_bytes;     /* bytes of signs per key  = 4 W                    */
  int64_t key_bytes;      /* code_bytes + sign_bytes + 8 (norm and rnorm)     */
  int32_t hi;             /* coordinates with one more index bit (0: plain)   */
  int32_t hi_words;       /* ceil(hi / 32): words of the extra plane          */
  int32_t polar;          /* 1 for a tq_init_polar handle                     */
} tq_layout;

/* Build the method for (d, bits, seed) on the current HIP device: rotation,
 * projection and codebook as described above.  2 <= d <= 4096,
 * 2 <= bits <= 5.  Synchronous.  *out receives the handle. */
TQ_API int tq_init(int32_t d, int32_t bits, uint64_t seed, tq_handle* out);

/* Fractional widths ("TurboQuant digest", section 4 quotes 2.5 and 3.5
 * bits per channel as operating points; the pages give no mechanism, so
 * this is a reading): tq_init(d, bits, seed) whose rotated coordinates
 * 0 .. hi-1 are quantized with the Lloyd-Max set of 2^bits levels (one more
 * index bit, the codebook tq_init(d, bits + 1, .) uses) and the rest with the
 * 2^(bits-1) levels of tq_init(d, bits, .).  Budget: bits + hi / d bits per
 * coordinate with the sign bit (d = 128, hi = 64: 2.5 from bits = 2, 3.5
 * from bits = 3).  Codes per key: the B = bits - 1 planes of W words as
 * usual, then one plane of hi_words = ceil(hi / 32) words holding bit B of
 * the indices of coordinates 0 .. hi-1 (bit j mod 32 of word j div 32,
 * padding 0); tq_layout gives code_bytes.  2 <= bits <= 4, 0 <= hi <= d
 * (hi = 0 is tq_init).  tq_quantize, tq_logits, tq_logits_topk,
 * tq_dequant_mse, tq_dequant_prod and the key side of tq_attention take such
 * handles (general kernels; the two reconstructions run on the matrix cores
 * when d = 128 and hi = 64); tq_pack_values and the value side of
 * tq_attention return TQ_EUNSUPPORTED. */
TQ_API int tq_init_split(int32_t d, int32_t bits, int32_t hi, uint64_t seed, tq_handle* out);

/* As tq_init but with caller-given float32 matrices (host, row-major d x d):
 * `pi` is used as the rotation, `g` as the projection; the codebook still
 * depends only on (d, bits).  For tests that need a known rotation, e.g. the
 * tutorial page's 4-D example.  Orthogonality of `pi` is not checked. */
TQ_API int tq_init_explicit(int32_t d, int32_t bits, const float* pi, const float* g, tq_handle* out);

/* As tq_init with a randomized Hadamard rotation in place of the Haar one
 * ("TurboQuant tutorial", PolarQuant section: its 4-D example rotates with
 * a +-1/2 matrix, the Hadamard matrix of order 4 over 2):
 *   Pi = H diag(sigma) / sqrt(d),  H[i][j] = (-1)^popcount(i & j)
 * (Sylvester order), sigma_j = -1 when bit 63 of counter j of stream 2 of
 * the seed is set, else +1; entries rounded to float32.  G and the codebook
 * are tq_init's.  d a power of two in [2, 4096]; every entry point then
 * works as for a tq_init handle (the rotation is applied as a dense matrix). */
TQ_API int tq_init_hadamard(int32_t d, int32_t bits, uint64_t seed, tq_handle* out);

/* Recursive polar-angle stage 1 in place of the scalar codebook ("TurboQuant
 * tutorial", section on turning Cartesian into polar coordinates: one length
 * kept at high precision and d - 1 angles of 2 or 3 bits; "TurboQuant deep
 * review", breakthrough section: a recursive polar transform after the random
 * rotation, angles with a concentrated law of analytic form; the pages leave
 * the recursion open, this is a reading).  With z = Pi u (u = k / ||k||) and
 * d a power of two: level 1 takes the pairs (z_2i, z_2i+1) to a radius and an
 * angle atan2(z_2i+1, z_2i) in [0, 2 pi); level l >= 2 takes pairs of level
 * l-1 radii (a, b) to sqrt(a^2 + b^2) and atan2(b, a) in [0, pi/2]; after
 * log2 d levels one radius (1) and d - 1 angles remain.  Each angle gets
 * bits - 1 index bits: level 1 the uniform quantizer of the circle (level
 * (k + 1/2) 2 pi / L), level l the Lloyd-Max quantizer of the law of
 * atan2(|b|, |a|) for two independent 2^(l-1)-dimensional Gaussian blocks
 * (density proportional to sin^(m-1) psi cos^(m-1) psi); tq_polar_codebook
 * gives them.  z_hat composes the level values back from radius 1, and the
 * QJL stage, the score and the stage-1 reconstruction use z_hat where a
 * plain handle uses c[idx]: r = z - z_hat, rho = ||r||, beta = [G r > 0],
 * score = n (<Pi q, z_hat> + rho sqrt(pi/2)/d <G Pi q, 2 beta - 1>),
 * k_hat = n Pi^T z_hat.  Codes: the d - 1 angle indices in level order
 * (level 1's d/2 angles, then level 2's d/4, ..., the top angle) in slots
 * 0 .. d-2 of the usual bit planes, slot d-1 zero; tq_layout reports
 * polar = 1.  Pi and G are tq_init's for the seed.  d a power of two in
 * [2, 4096], 2 <= bits <= 5.  tq_quantize, tq_logits and tq_dequant_mse take
 * such handles (float32 kernels); tq_logits_topk, tq_dequant_prod,
 * tq_pack_values and tq_attention return TQ_EUNSUPPORTED. */
TQ_API int tq_init_polar(int32_t d, int32_t bits, uint64_t seed, tq_handle* out);

/* Host only, no HIP call: the angle codebook of recursion level `level`
 * (1 .. log2 d) of tq_init_polar(d, bits, .): levels float[2^(bits-1)]
 * ascending, thresholds float[2^(bits-1) - 1] (either may be NULL). */
TQ_API int tq_polar_codebook(int32_t d, int32_t bits, int32_t level, float* levels, float* thresholds);

/* Host only, no HIP call: the rotation tq_init_hadamard(d, ., seed) uses,
 * float[d*d] row-major into pi. */
TQ_API int tq_hadamard_rotation(int32_t d, uint64_t seed, float* pi);

/* Release the handle and its device tables.  NULL is accepted. */
TQ_API int tq_destroy(tq_handle h);

/* Sizes of the packed layout for this handle (host struct). */
TQ_API int tq_get_layout(tq_handle h, tq_layout* out);

/* Host only, no HIP call: the parameters tq_init(d, bits, seed) uses.
 * pi, g: host float[d*d] row-major (either may be NULL to skip it);
 * centroids: host float[2^(bits-1)] ascending; thresholds: host
 * float[2^(bits-1) - 1] ascending (either may be NULL). */
TQ_API int tq_host_params(int32_t d, int32_t bits, uint64_t seed, float* pi, float* g,
                   float* centroids, float* thresholds);

/* FNV-1a 64 hash of the handle's float32 Pi, G and centroids (host copies);
 * equal handles on different processes or GPUs hash equal.  0 on a NULL
 * handle. */
TQ_API uint64_t tq_params_hash(tq_handle h);

/* Quantize n keys.  keys: device, n rows of d elements of type key_dtype
 * (TQ_F32 or TQ_BF16), row i at keys + i*ldk elements (ldk >= d).
 * Outputs (device): codes [n][B][W], signs [n][W], norms [n], rnorms [n] as
 * in the packed layout, 4-byte aligned.  Asynchronous on `stream`.  Norms
 * are computed in float32: a key whose squared norm overflows float32
 * (||k|| above about 1.8e19) gives an infinite norm; NaN/Inf inputs are
 * undefined.  The fast d = 128 path for bf16 keys needs keys and all four
 * outputs 16-byte aligned and ldk a multiple of 8; other calls take the
 * general kernels (same results within the parity bounds). */
TQ_API int tq_quantize(tq_handle h, const void* keys, int32_t key_dtype, int64_t n, int64_t ldk,
                uint32_t* codes, uint32_t* signs, float* norms, float* rnorms, void* stream);

/* Bytes of device workspace tq_logits needs for `groups` x `nq` queries. */
TQ_API size_t tq_logits_workspace_size(tq_handle h, int64_t groups, int64_t nq);

/* Asymmetric scores of full-precision queries against packed keys.
 * queries: device float [groups][nq][d]; the packed arrays hold groups*n keys
 * ordered [groups][n] (key t of group g is key g*n + t); group g's queries
 * score only group g's keys (grouped-query attention: the nq query heads
 * that share one key head form a group).  scores: device float
 * [groups][nq][n].  workspace: device, at least
 * tq_logits_workspace_size(h, groups, nq) bytes, 256-byte aligned.  Raw
 * inner products, no 1/sqrt(d) scaling.  Asynchronous on `stream`. */
TQ_API int tq_logits(tq_handle h, const float* queries, int64_t groups, int64_t nq,
              const uint32_t* codes, const uint32_t* signs, const float* norms,
              const float* rnorms, int64_t n, float* scores, void* workspace,
              size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): tq_logits
 * with the workspace taken from a static scratch array of the library
 * instead of an argument.  Same arguments otherwise, same kernels, and the
 * same scores bit for bit.  No allocation happens in the call (nor any
 * hipMalloc / hipFree); the caller still provides queries, packed keys and
 * scores.  Returns TQ_ESCRATCH when tq_logits_workspace_size(h, groups, nq)
 * exceeds tq_noalloc_scratch_bytes() (16 MiB: query rows of d = 128 up to
 * 16384 per call).  The array is one per GPU, held until the process ends
 * and shared by every call on that GPU: calls that overlap in time on one
 * GPU (other streams or host threads) race on it and must be serialised by
 * the caller. */
TQ_API int tq_logits_noalloc(tq_handle h, const float* queries, int64_t groups, int64_t nq,
                             const uint32_t* codes, const uint32_t* signs, const float* norms,
                             const float* rnorms, int64_t n, float* scores, void* stream);

/* Bytes of the static scratch array tq_logits_noalloc uses (per GPU). */
TQ_API size_t tq_noalloc_scratch_bytes(void);

/* Bytes of device workspace tq_logits_topk needs for `groups` x `nq`
 * queries against n keys per group, k best keys per query. */
TQ_API size_t tq_logits_topk_workspace_size(tq_handle h, int64_t groups, int64_t nq, int64_t n, int32_t k);

/* Search ("TurboQuant digest", section 3: brute-force scores compared by
 * recall): the k best keys per query by the asymmetric score of tq_logits,
 * without materialising the score matrix.  queries, packed arrays, groups,
 * nq and n as for tq_logits; 1 <= k <= 64.  top_idx: device int64
 * [groups][nq][k], key index within the group; top_scores: device float
 * [groups][nq][k], best first, equal scores in ascending key index.  When
 * k > n the entries past n hold index -1 and score -inf.  workspace: device,
 * at least tq_logits_topk_workspace_size(h, groups, nq, n, k) bytes,
 * 256-byte aligned; its contents are scratch.  Scores are computed exactly
 * as tq_logits computes them, a chunk of keys at a time.  Asynchronous on
 * `stream`. */
TQ_API int tq_logits_topk(tq_handle h, const float* queries, int64_t groups, int64_t nq,
                          const uint32_t* codes, const uint32_t* signs, const float* norms,
                          const float* rnorms, int64_t n, int32_t k, int64_t* top_idx,
                          float* top_scores, void* workspace, size_t workspace_bytes, void* stream);

/* Stage-1 reconstruction k_hat = n * Pi^T c[idx] of n packed keys.
 * codes, norms: device as in the packed layout; khat: device float [n][d].
 * Asynchronous on `stream`. */
TQ_API int tq_dequant_mse(tq_handle h, const uint32_t* codes, const float* norms, int64_t n,
                   float* khat, void* stream);

/* Reconstruction with the QJL correction ("TurboQuant deep review", error
 * compensation section: the corrected estimate is unbiased):
 *   k_tilde = n * Pi^T ( c[idx] + rho * sqrt(pi/2) / d * G^T (2 beta - 1) ),
 * the vector whose inner product with any query q equals the asymmetric
 * score tq_logits estimates (the score is linear in q).  codes, signs,
 * norms, rnorms: device, n packed keys; ktilde: device float [n][d].
 * Float32 arithmetic.  Asynchronous on `stream`. */
TQ_API int tq_dequant_prod(tq_handle h, const uint32_t* codes, const uint32_t* signs, const float* norms,
                           const float* rnorms, int64_t n, float* ktilde, void* stream);

/* The uncompressed comparison: raw inner products of float32 queries with
 * unquantized keys, the operation whose time the pages compare 4-bit keys
 * against ("TurboQuant digest", section 3: attention logits against 32-bit
 * keys).  No handle.  queries: device float [groups][nq][d]; keys: device,
 * groups * n rows of d elements of key_dtype (TQ_F32 or TQ_BF16), row i at
 * keys + i*ldk elements (ldk >= d), group g's keys are rows g*n ..
 * g*n + n - 1; scores: device float [groups][nq][n].  1 <= d <= 4096.
 * Summation in float32 (order unspecified).  Asynchronous on `stream`. */
TQ_API int tq_dense_logits(const float* queries, int64_t groups, int64_t nq, const void* keys,
                           int32_t key_dtype, int64_t n, int32_t d, int64_t ldk, float* scores,
                           void* stream);

/* Value cache layout for tq_attention.  Values are quantized like keys
 * (tq_quantize with the value handle; only codes and norms are kept: the
 * attention reads values back through the stage-1 reconstruction) and their
 * codes are regrouped into token blocks of 32 tokens:
 *   vcodes [groups][ceil(n/32)][B][32 W] uint32, i.e. 128 B W bytes per
 *   block, read as little-endian bytes (tokens past n and coordinates past
 *   d give index 0).
 * Within a block the 32 tokens form 4 octets o (tokens 32 b + 8 o .. + 7).
 * For coordinate c and octet o, one B-byte little-endian integer X holds
 * the B index bits of the octet's 8 tokens: bit p of the index of token
 * 8 o + t sits at bit (t div E) B E + p E + (t mod E) of X, with E = 8, 4,
 * 2, 2 tokens for B = 1, 2, 3, 4.  So each run of B E bits of X is the
 * packed index of E consecutive tokens, which the attention's value pass
 * looks up in one table read.  Coordinates come in groups of 128 (the last
 * group holds G = W mod 4 words of the key layout when that is not 0, else
 * G = 4); group g's 512 B G bytes start at byte 512 B g of the block, and
 * for coordinate c = 128 g + r (r < 32 G) the integer X of octet o starts at
 * byte ((r mod 16) + 16 o) * 2 G B + (r div 16) * B of the group.  That puts
 * the integers one lane of the value pass reads (one octet, coordinates
 * r mod 16 + 16 j) side by side.
 * codes: device, groups * n packed keys' codes [groups][n][B][W]; vcodes:
 * device, 16-byte aligned, as above.  Asynchronous on `stream`. */
TQ_API int tq_pack_values(tq_handle h, const uint32_t* codes, int64_t groups, int64_t n, uint32_t* vcodes,
                          void* stream);

/* Bytes of device workspace tq_attention needs. */
TQ_API size_t tq_attention_workspace_size(tq_handle hk, tq_handle hv, int64_t groups, int64_t nq, int64_t n);

/* Decode attention over a compressed KV cache ("Why KV-cache compression
 * works", section 2: the method compresses the key-value cache; "TurboQuant
 * tutorial", glossary: queries, keys and values).  For each query of group
 * g against the group's n stored tokens:
 *   o   = sum_t softmax_t(scale * s_t) * v_hat_t,
 *   lse = log sum_t exp(scale * s_t),
 * s_t the asymmetric score of the query against key t (exactly as
 * tq_logits computes it, with handle hk) and v_hat_t = n_t Pi^T c[idx_t] the
 * stage-1 reconstruction of value t (handle hv: its rotation and levels;
 * same d as hk, any bit width).  Every stored token is visible; `scale` is
 * the caller's (1/sqrt(d) in the usual attention), any finite value.
 * queries: device float [groups][nq][d]; kcodes, ksigns, knorms, krnorms:
 * groups * n packed keys as for tq_logits; vcodes: token blocks from
 * tq_pack_values; vnorms: device float [groups][n].  out: device float
 * [groups][nq][d]; lse: device float [groups][nq] or NULL.  n = 0 gives
 * o = 0 and lse = -inf.  workspace: device, at least
 * tq_attention_workspace_size(hk, hv, groups, nq, n) bytes (room for the
 * score matrix and the per-split partial sums; when the key handle takes
 * the byte-table scorer, d in (96, 128] with at most 3 index bits, and the
 * values have at most 3 index bits, the scores stay on chip and only the
 * partials are used), 256-byte aligned.  Asynchronous on `stream`. */
TQ_API int tq_attention(tq_handle hk, tq_handle hv, const float* queries, int64_t groups, int64_t nq,
                        const uint32_t* kcodes, const uint32_t* ksigns, const float* knorms,
                        const float* krnorms, const uint32_t* vcodes, const float* vnorms, int64_t n,
                        float scale, float* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Static string naming an error code. */
TQ_API const char* tq_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
