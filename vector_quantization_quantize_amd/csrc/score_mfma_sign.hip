// Matrix-core scorer instantiations: one index bit, symmetric level set (sign form), every K-step count.
#include "score_mfma.h"

namespace tqdev {

hipError_t score_launch_sign(const ScoreArgs& a) { return score::launch_form<1, kSignForm>(a); }

size_t score_lds_sign(int d) { return score::static_lds_form<1, kSignForm>(d); }

}  // namespace tqdev
