// Prefill product instances of one weight format.
#include "qmm_launch.hpp"

namespace bq {

int launch_qmm_u2(const QmmParams& p, int gs, bool implied, void* stream) {
  return launch_qmm_bits<2>(p, gs, implied, stream);
}

}  // namespace bq
