// gemv_ternary.hip -- GEMV instantiations for the ternary format (see gemv_impl.hpp).
#include "gemv_impl.hpp"

namespace qmoe {

hipError_t launch_gemv_ternary(const GemvArgs &a, int epilogue, int in_f16, int mmax, int waves,
                          int grid_slots, hipStream_t s) {
  return launch_gemv_qt<QMOE_QTYPE_TERNARY>(a, epilogue, in_f16, mmax, waves, grid_slots, s);
}

}  // namespace qmoe
