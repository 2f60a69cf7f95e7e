// Prefill product instances of one weight format.
#include "qmm_launch.hpp"

namespace bq {

int launch_qmm_t5(const QmmParams& p, int gs, bool implied, void* stream) {
  return launch_qmm_bits<BQ_BITS_T5>(p, gs, implied, stream);
}

}  // namespace bq
