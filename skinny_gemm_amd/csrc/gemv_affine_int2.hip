// gemv_affine_int2.hip -- GEMV instantiations for the affine_int2 format (see gemv_impl.hpp).
#include "gemv_impl.hpp"

namespace qmoe {

const void *gemv_ptr_affine_int2(int epilogue, int in_f16, int rows, int block, int tn, int ext) {
  return gemv_ptr_qt<QMOE_QTYPE_AFFINE_INT2>(epilogue, in_f16, rows, block, tn, ext);
}

}  // namespace qmoe
