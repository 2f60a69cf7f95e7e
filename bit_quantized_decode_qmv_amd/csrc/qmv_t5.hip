// Decode kernel instances of one weight format.
#include "qmv_launch.hpp"

namespace bq {

QmvLauncher pick_qmv_t5(int gs, int M, bool implied) {
  if (gs == 64) return implied ? pick_m<FMT_T5, 64, true>(M) : pick_m<FMT_T5, 64, false>(M);
  return implied ? pick_m<FMT_T5, 128, true>(M) : pick_m<FMT_T5, 128, false>(M);
}

}  // namespace bq
