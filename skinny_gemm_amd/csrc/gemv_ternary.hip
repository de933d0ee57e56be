// gemv_ternary.hip -- GEMV instantiations for the ternary format (see gemv_impl.hpp).
#include "gemv_impl.hpp"

namespace qmoe {

const void *gemv_ptr_ternary(int epilogue, int in_f16, int rows, int block, int tn, int ext) {
  return gemv_ptr_qt<QMOE_QTYPE_TERNARY>(epilogue, in_f16, rows, block, tn, ext);
}

}  // namespace qmoe
