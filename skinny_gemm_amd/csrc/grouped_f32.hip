// grouped_f32.hip -- grouped MFMA kernel instances of FC2 with fp32 per-slot outputs (see grouped_impl.hpp).
#include "grouped_impl.hpp"

namespace qmoe {

hipError_t launch_grouped_f32(const GroupedArgs &a, int grid, hipStream_t s) {
  return launch_grouped_epi<kGEpiStoreF32>(a, grid, s);
}

}  // namespace qmoe
