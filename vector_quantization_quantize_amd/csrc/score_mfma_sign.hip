// Matrix-core scorer instantiations, one index bit, symmetric level set (sign form):
// every K-step count of the register form (d <= 256) and the tiled form (d > 256).
#include "score_gemm.h"
#include "score_mfma.h"

namespace tqdev {

hipError_t score_launch_sign(const ScoreArgs& a) { return score::launch_form<1, kSignForm>(a); }

size_t score_lds_sign(int d) { return score::static_lds_form<1, kSignForm>(d); }

hipError_t score_gemm_launch_sign(const ScoreArgs& a) { return gemm::launch_form<1, kSignForm>(a); }

size_t score_gemm_lds_sign() { return gemm::static_lds<1, kSignForm>(); }

}  // namespace tqdev
