// Matrix-core scorer instantiations: three index bits, two float16 pieces per level, every K-step count.
#include "score_mfma.h"

namespace tqdev {

hipError_t score_launch_two3(const ScoreArgs& a) { return score::launch_form<3, kTwoPiece>(a); }

size_t score_lds_two3(int d) { return score::static_lds_form<3, kTwoPiece>(d); }

}  // namespace tqdev
