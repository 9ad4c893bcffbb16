// Instantiations of the fused chunked kernel: f32 activations, decay kind 0
// (0 none, 1 per head, 2 per key channel).
#include "chunked_impl.h"

namespace kda {
namespace chunked {

hipError_t launch_f32_d0(int DK, int DVS, int C, const ChunkParams& cp, int nwg, hipStream_t s) {
  return launch_any<float, 0>(DK, DVS, C, cp, nwg, s);
}

}  // namespace chunked
}  // namespace kda
