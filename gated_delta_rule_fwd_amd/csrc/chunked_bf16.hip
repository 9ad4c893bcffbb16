// Instantiations of the fused chunked kernel for bf16 activations.
#include "chunked_impl.h"

namespace kda {
namespace chunked {

hipError_t launch_bf16(int DK, int DVS, int C, const ChunkParams& cp, int nwg, bool chan,
                       hipStream_t s) {
  return launch_any<bf16_t>(DK, DVS, C, cp, nwg, chan, s);
}

}  // namespace chunked
}  // namespace kda
