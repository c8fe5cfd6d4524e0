// Matrix-core scorer: choice of form, grid shape and per-form dispatch (the
// kernels are in score_mfma.h, d <= 256, and score_gemm.h, d > 256,
// instantiated by score_mfma_<form>.hip).
#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

constexpr int kTileKeys = 32;
// resident blocks per CU: the register form runs 2 of 4 waves, the tiled
// form 1 of 8
int blocks_per_cu(const tq_ctx* h) { return h->d >= kScoreGemmMinD ? 1 : 2; }
constexpr float kCScale = 1024.0f;

// Blocks of key tiles per query tile: enough blocks to fill the resident
// slots, with the total a close fit to a whole number of rounds of slots (a
// last round that holds a few blocks costs as much as a full one).
int64_t pick_splits(int64_t slots, int64_t qtiles, int64_t groups, int64_t ntiles) {
  const int64_t per = qtiles * groups;
  int64_t lo = (slots + per - 1) / per;
  lo = lo < ntiles ? lo : ntiles;
  lo = lo < 1 ? 1 : lo;
  int64_t best = lo;
  double best_eff = -1.0;
  for (int64_t s = lo; s <= 8 * lo + 8 && s <= ntiles; ++s) {
    const int64_t blocks = per * s;
    const int64_t rounds = (blocks + slots - 1) / slots;
    const double eff = double(blocks) / double(rounds * slots);
    if (eff > best_eff + 0.02) {  // fewer splits unless clearly better
      best = s;
      best_eff = eff;
    }
  }
  // whole tiles per block
  const int64_t tpb = (ntiles + best - 1) / best;
  return (ntiles + tpb - 1) / tpb;
}

// keys per tile: 32 in the register form, 128 in the tiled form
int64_t tile_keys(const tq_ctx* h) { return h->d >= kScoreGemmMinD ? 128 : kTileKeys; }

int form_of(const tq_ctx* h) {
  if (h->code_bits == 1) return kSignForm;  // symmetric: checked by score_mfma_supported
  if (h->code_bits == 2 && h->dqt.two_pass) return kOnePiece;
  return kTwoPiece;
}

ScoreForm form_params(const tq_ctx* h) {
  ScoreForm fp{};
  const double kappa = 1.2533141373155002512 / double(h->d);  // sqrt(pi/2) / d
  switch (form_of(h)) {
    case kSignForm: {
      const double a = h->cb.c[1];
      fp.lambda = float(kappa / a);
      fp.gamma = float(a);
      break;
    }
    case kOnePiece: {
      // out_scale = 1 / (sigma 2^12)
      const double inv_sigma = double(h->dqt.out_scale) * 4096.0;
      for (int i = 0; i < kMaxLevels; ++i) fp.val[i] = h->dqt.v[i];
      fp.lambda = float(kappa / inv_sigma);
      fp.gamma = float(inv_sigma);
      break;
    }
    default:
      for (int i = 0; i < kMaxLevels; ++i) fp.val[i] = h->cb.c[i] * kCScale;
      fp.lambda = float(kappa * kCScale);
      fp.gamma = 1.0f / kCScale;
  }
  return fp;
}

hipError_t dispatch(const ScoreArgs& a) {
  if (a.h->d >= kScoreGemmMinD) {
    switch (a.h->code_bits) {
      case 1: return score_gemm_launch_sign(a);
      case 2: return form_of(a.h) == kOnePiece ? score_gemm_launch_one2(a) : score_gemm_launch_two2(a);
      case 3: return score_gemm_launch_two3(a);
      case 4: return score_gemm_launch_two4(a);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.h->code_bits) {
    case 1: return score_launch_sign(a);
    case 2: return form_of(a.h) == kOnePiece ? score_launch_one2(a) : score_launch_two2(a);
    case 3: return score_launch_two3(a);
    case 4: return score_launch_two4(a);
    default: return hipErrorInvalidValue;
  }
}

size_t static_lds(const tq_ctx* h) {
  if (h->d >= kScoreGemmMinD) {
    switch (h->code_bits) {
      case 1: return score_gemm_lds_sign();
      case 2: return form_of(h) == kOnePiece ? score_gemm_lds_one2() : score_gemm_lds_two2();
      case 3: return score_gemm_lds_two3();
      case 4: return score_gemm_lds_two4();
      default: return SIZE_MAX;
    }
  }
  switch (h->code_bits) {
    case 1: return score_lds_sign(h->d);
    case 2: return form_of(h) == kOnePiece ? score_lds_one2(h->d) : score_lds_two2(h->d);
    case 3: return score_lds_two3(h->d);
    case 4: return score_lds_two4(h->d);
    default: return SIZE_MAX;
  }
}

ScoreArgs make_args(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                    const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, hipStream_t stream) {
  ScoreArgs a{};
  a.h = h;
  a.vw = vw;
  a.groups = groups;
  a.nq = nq;
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.rnorms = rnorms;
  a.n = n;
  a.key_stride = n;
  a.form = form_params(h);
  a.qtiles = (nq + 127) / 128;
  const int64_t tk = tile_keys(h);
  const int64_t ntiles = (n + tk - 1) / tk;
  a.splits = pick_splits(int64_t(blocks_per_cu(h)) * h->cus, a.qtiles, groups, ntiles);
  a.tiles_per_block = (ntiles + a.splits - 1) / a.splits;
  a.stream = stream;
  if (h->d >= kScoreGemmMinD) {
    // float16 query rows and row factors follow the vw rows
    const int64_t rows = groups * nq;
    char* base = reinterpret_cast<char*>(const_cast<float*>(vw)) + score_vw_bytes(h->d, rows);
    a.qa = base;
    a.row_f = reinterpret_cast<float*>(base + score_qa_bytes(h->d, groups, nq));
  }
  return a;
}

}  // namespace

bool score_mfma_supported(const tq_ctx* h) {
  if (h->hi != 0 || h->code_bits < 1 || h->code_bits > 4) return false;
  return h->code_bits > 1 || h->symmetric;
}

hipError_t launch_score_mfma(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq, const uint32_t* codes,
                             const uint32_t* signs, const float* norms, const float* rnorms, int64_t n,
                             float* scores, hipStream_t stream) {
  if (n <= 0 || nq <= 0 || groups <= 0) return hipSuccess;
  if (!score_mfma_supported(h)) return hipErrorInvalidValue;
  ScoreArgs a = make_args(h, vw, groups, nq, codes, signs, norms, rnorms, n, stream);
  if (a.qtiles > 0x7FFFFFFF || a.splits > 65535 || groups > 65535) return hipErrorInvalidConfiguration;
  a.scores = scores;
  return dispatch(a);
}

bool score_topk_mfma_supported(const tq_ctx* h, int64_t n, int k) {
  if (!score_mfma_supported(h) || k < 1 || k > kTopkMax || n <= 0 || n > INT32_MAX) return false;
  const size_t st = static_lds(h);
  return st != SIZE_MAX && st + score_list_bytes(k) <= size_t(h->lds_per_block);
}

int64_t score_topk_mfma_splits(const tq_ctx* h, int64_t groups, int64_t nq, int64_t n) {
  const int64_t qtiles = (nq + 127) / 128;
  const int64_t tk = tile_keys(h);
  const int64_t ntiles = (n + tk - 1) / tk;
  return pick_splits(int64_t(blocks_per_cu(h)) * h->cus, qtiles, groups, ntiles);
}

hipError_t launch_score_topk_mfma(const tq_ctx* h, const float* vw, int64_t groups, int64_t nq,
                                  const uint32_t* codes, const uint32_t* signs, const float* norms,
                                  const float* rnorms, int64_t n, int64_t key_stride, int k, unsigned int* bound,
                                  float* part_s, int64_t* part_i, hipStream_t stream) {
  if (n <= 0 || nq <= 0 || groups <= 0) return hipSuccess;
  if (!score_topk_mfma_supported(h, n, k) || key_stride < n) return hipErrorInvalidValue;
  ScoreArgs a = make_args(h, vw, groups, nq, codes, signs, norms, rnorms, n, stream);
  if (a.qtiles > 0x7FFFFFFF || a.splits > 65535 || groups > 65535) return hipErrorInvalidConfiguration;
  a.key_stride = key_stride;
  a.bound = bound;
  a.topk = true;
  a.part_s = part_s;
  a.part_i = part_i;
  a.k = k;
  return dispatch(a);
}

}  // namespace tqdev
