// gemv_affine_int4.hip -- GEMV instantiations for the affine_int4 format (see gemv_impl.hpp).
#include "gemv_impl.hpp"

namespace qmoe {

const void *gemv_ptr_affine_int4(int epilogue, int in_f16, int rows, int block, int tn, int ext) {
  return gemv_ptr_qt<QMOE_QTYPE_AFFINE_INT4>(epilogue, in_f16, rows, block, tn, ext);
}

}  // namespace qmoe
