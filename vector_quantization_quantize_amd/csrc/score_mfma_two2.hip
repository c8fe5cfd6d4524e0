// Matrix-core scorer instantiations: two index bits, two float16 pieces per level, every K-step count.
#include "score_mfma.h"

namespace tqdev {

hipError_t score_launch_two2(const ScoreArgs& a) { return score::launch_form<2, kTwoPiece>(a); }

size_t score_lds_two2(int d) { return score::static_lds_form<2, kTwoPiece>(d); }

}  // namespace tqdev
