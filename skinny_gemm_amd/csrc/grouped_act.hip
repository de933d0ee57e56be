// grouped_act.hip -- grouped MFMA kernel instances of the dense matrix with 16-bit outputs (see grouped_impl.hpp).
#include "grouped_impl.hpp"

namespace qmoe {

hipError_t launch_grouped_act(const GroupedArgs &a, int grid, hipStream_t s) {
  return launch_grouped_epi<kGEpiStoreAct>(a, grid, s);
}

}  // namespace qmoe
