// Instantiations of the fused chunked kernel for fp32 activations.
#include "chunked_impl.h"

namespace kda {
namespace chunked {

hipError_t launch_f32(int DK, int DVS, int C, const ChunkParams& cp, int nwg, bool chan,
                      hipStream_t s) {
  return launch_any<float>(DK, DVS, C, cp, nwg, chan, s);
}

}  // namespace chunked
}  // namespace kda
