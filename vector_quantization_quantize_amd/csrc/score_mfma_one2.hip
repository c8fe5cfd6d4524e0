// Matrix-core scorer instantiations, two index bits, one float16 piece per level:
// every K-step count of the register form (d <= 256) and the tiled form (d > 256).
#include "score_gemm.h"
#include "score_mfma.h"

namespace tqdev {

hipError_t score_launch_one2(const ScoreArgs& a) { return score::launch_form<2, kOnePiece>(a); }

size_t score_lds_one2(int d) { return score::static_lds_form<2, kOnePiece>(d); }

hipError_t score_gemm_launch_one2(const ScoreArgs& a) { return gemm::launch_form<2, kOnePiece>(a); }

size_t score_gemm_lds_one2() { return gemm::static_lds<2, kOnePiece>(); }

}  // namespace tqdev
