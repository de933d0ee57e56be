// grouped_swiglu.hip -- grouped MFMA kernel instances of FC1 with the SwiGLU / ReLU epilogue (see grouped_impl.hpp).
#include "grouped_impl.hpp"

namespace qmoe {

hipError_t launch_grouped_swiglu(const GroupedArgs &a, int grid, hipStream_t s) {
  return launch_grouped_epi<kGEpiSwiGLU>(a, grid, s);
}

}  // namespace qmoe
