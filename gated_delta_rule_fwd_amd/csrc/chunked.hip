// Host planning of the fused chunked forward: value-slice width, grid, and
// dispatch to the bf16 / fp32 instantiations (chunked_impl.h).
#include "chunked_impl.h"

namespace kda {
namespace {

using chunked::ChunkParams;

// Pick the value-slice width: enough workgroups to cover the 256 CUs, no
// wider than 64 columns, and an LDS plan that fits one CU.
struct Plan { int dvs; size_t lds; };

Plan plan_for(int B, int H, int DK, int DV, int C, int dtype, bool chan) {
  int dvs = DV < 64 ? DV : 64;
  while (dvs > 16 && static_cast<long>(B) * H * (DV / dvs) < 256) dvs /= 2;
  while (dvs >= 16) {
    const size_t l = dtype == 0 ? chunked::lds_bytes<4>(DK, dvs, C, chan)
                                : chunked::lds_bytes<2>(DK, dvs, C, chan);
    if (l != 0 && l <= kMaxLds) return Plan{dvs, l};
    dvs /= 2;
  }
  return Plan{0, 0};
}

}  // namespace

size_t chunked_lds_bytes(int DK, int DV, int chunk, int dtype) {
  // the largest plan over decay kinds at the smallest grid (B = H = 1)
  const Plan a = plan_for(1, 1, DK, DV, chunk, dtype, true);
  const Plan b = plan_for(1, 1, DK, DV, chunk, dtype, false);
  if (a.dvs == 0 || b.dvs == 0) return 0;
  return a.lds > b.lds ? a.lds : b.lds;
}

hipError_t launch_chunked(const FwdArgs& a, hipStream_t s) {
  const bool chan = a.decay_kind == DECAY_CHANNEL;
  const Plan pl = plan_for(a.B, a.H, a.DK, a.DV, a.chunk, a.dtype, chan);
  if (pl.dvs == 0) return hipErrorInvalidConfiguration;
  ChunkParams cp;
  cp.q = a.q; cp.k = a.k; cp.v = a.v; cp.beta = a.beta; cp.decay = a.decay;
  cp.init = a.init; cp.o = a.o; cp.state = a.state;
  cp.T = a.T; cp.H = a.H; cp.DV = a.DV;
  cp.nsl = a.DV / pl.dvs;
  cp.decay_kind = a.decay_kind;
  cp.l2norm = a.l2norm;
  cp.scale = a.scale;
  const int nheads = a.B * a.H;
  cp.xcd_map = (nheads % 8 == 0) ? 1 : 0;
  const int nwg = nheads * cp.nsl;
  using LaunchFn = hipError_t (*)(int, int, int, const ChunkParams&, int, hipStream_t);
  static const LaunchFn table[2][3] = {
      {chunked::launch_f32_d0, chunked::launch_f32_d1, chunked::launch_f32_d2},
      {chunked::launch_bf16_d0, chunked::launch_bf16_d1, chunked::launch_bf16_d2}};
  return table[a.dtype == 0 ? 0 : 1][a.decay_kind](a.DK, pl.dvs, a.chunk, cp, nwg, s);
}

}  // namespace kda
