// Matrix-core scorer instantiations: two index bits, one float16 piece per level, every K-step count.
#include "score_mfma.h"

namespace tqdev {

hipError_t score_launch_one2(const ScoreArgs& a) { return score::launch_form<2, kOnePiece>(a); }

size_t score_lds_one2(int d) { return score::static_lds_form<2, kOnePiece>(d); }

}  // namespace tqdev
