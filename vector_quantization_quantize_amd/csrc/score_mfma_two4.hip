// Matrix-core scorer instantiations, four index bits, two float16 pieces per level:
// every K-step count of the register form (d <= 256) and the tiled form (d > 256).
#include "score_gemm.h"
#include "score_mfma.h"

namespace tqdev {

hipError_t score_launch_two4(const ScoreArgs& a) { return score::launch_form<4, kTwoPiece>(a); }

size_t score_lds_two4(int d) { return score::static_lds_form<4, kTwoPiece>(d); }

hipError_t score_gemm_launch_two4(const ScoreArgs& a) { return gemm::launch_form<4, kTwoPiece>(a); }

size_t score_gemm_lds_two4() { return gemm::static_lds<4, kTwoPiece>(); }

}  // namespace tqdev
