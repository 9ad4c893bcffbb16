// Instantiations of the chunked kernels: bf16 activations, decay kind 1
// (0 none, 1 per head, 2 per key channel).
#include "chunked_impl.h"

namespace kda {
namespace chunked {

hipError_t launch_bf16_d1(int DK, int DVS, int C, const PrepParams& pp, int nwg_prep,
                          const StateParams& sp, int nwg_state, hipStream_t s) {
  return launch_any<bf16_t, 1>(DK, DVS, C, pp, nwg_prep, sp, nwg_state, s);
}

}  // namespace chunked
}  // namespace kda
