// Host planning of the chunked forward: value-slice width, grids, the
// segments of chunks that the caller's workspace holds the records of (the
// prep kernel writes one record per chunk, the state kernel reads it), and
// dispatch to the bf16 / fp32 instantiations (chunked_impl.h).
#include <mutex>

#include "../../include/kda.h"
#include "chunked_impl.h"

namespace kda {
namespace {

// Fixed device scratch of kda_fwd_chunked_noalloc: the per-chunk records of
// callers that cannot allocate.  Each device the library runs on holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress (noalloc_scratch below) and only that is passed on.
__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_WORKSPACE_BYTES];

using chunked::PrepParams;
using chunked::StateParams;

// Pick the value-slice width of the state kernel: enough workgroups to cover
// the 256 CUs, no wider than 64 columns, and LDS plans that fit one CU.
struct Plan { int dvs; size_t lds; };

Plan plan_for(int B, int H, int DK, int DV, int C, int dtype, bool chan) {
  int dvs = DV < 64 ? DV : 64;
  while (dvs > 16 && static_cast<long>(B) * H * (DV / dvs) < 256) dvs /= 2;
  while (dvs >= 16) {
    const size_t l = dtype == 0 ? chunked::lds_bytes<4, 4>(DK, dvs, C, chan)
                                : chunked::lds_bytes<2, 2>(DK, dvs, C, chan);
    if (l != 0 && l <= kMaxLds) return Plan{dvs, l};
    dvs /= 2;
  }
  return Plan{0, 0};
}

}  // namespace

size_t chunked_lds_bytes(int DK, int DV, int chunk, int dtype, int decay_kind) {
  // the plan at the smallest grid (B = H = 1) is the widest slice
  const Plan a = plan_for(1, 1, DK, DV, chunk, dtype, decay_kind == DECAY_CHANNEL);
  return a.dvs == 0 ? 0 : a.lds;
}

// The device address of this device's `scratch`, looked up once per device
// with that device current (the caller's current device).
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t chunked_record_bytes(int DK, int chunk, int dtype, int decay_kind) {
  const bool chan = decay_kind == DECAY_CHANNEL;
  return dtype == 0 ? chunked::record_bytes<4>(DK, chunk, chan) : chunked::record_bytes<2>(DK, chunk, chan);
}

// Chunks per launch pair: as many as the workspace holds the records of
// (every head of a chunk index takes one record), at least 1, at most all.
// Long inputs with a small workspace are processed in segments of chunks; the
// state kernel of one segment hands its final state to the next.
int segment_chunks(int nchunks, int nheads, size_t rec, size_t ws_bytes) {
  const size_t per = rec * static_cast<size_t>(nheads);
  size_t seg = per ? ws_bytes / per : 0;
  if (seg < 1) seg = 1;
  if (seg > static_cast<size_t>(nchunks)) seg = nchunks;
  return static_cast<int>(seg);
}

hipError_t launch_chunked(const FwdArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  const bool chan = a.decay_kind == DECAY_CHANNEL;
  const Plan pl = plan_for(a.B, a.H, a.DK, a.DV, a.chunk, a.dtype, chan);
  if (pl.dvs == 0) return hipErrorInvalidConfiguration;
  const int nchunks = (a.T + a.chunk - 1) / a.chunk;
  const int nheads = a.B * a.H;
  const size_t rec = a.dtype == 0 ? chunked::record_bytes<4>(a.DK, a.chunk, chan)
                                  : chunked::record_bytes<2>(a.DK, a.chunk, chan);
  if (rec == 0) return hipErrorInvalidConfiguration;
  const int seg = segment_chunks(nchunks, nheads, rec, ws_bytes);
  hipError_t e = hipSuccess;

  PrepParams pp;
  pp.cu = nullptr; pp.cb = nullptr; pp.nseq = a.B;
  pp.q = a.q; pp.k = a.k; pp.beta = a.beta; pp.decay = a.decay;
  pp.ws = static_cast<unsigned char*>(ws);
  pp.T = a.T; pp.H = a.H; pp.l2norm = a.l2norm; pp.scale = a.scale;
  pp.tf = a.tf;
  pp.Hk = a.Hk;
  pp.hk_magic = ((1ULL << 32) + a.H / a.Hk - 1) / (a.H / a.Hk);

  StateParams sp;
  sp.cu = nullptr; sp.cb = nullptr;
  sp.q = a.q; sp.k = a.k;
  sp.l2norm = a.l2norm; sp.scale = a.scale;
  sp.v = a.v; sp.ws = static_cast<const unsigned char*>(ws);
  sp.o = a.o; sp.state = a.state;
  sp.T = a.T; sp.H = a.H; sp.DV = a.DV;
  sp.Hk = a.Hk; sp.vfirst = a.vfirst; sp.hk_magic = pp.hk_magic;
  sp.nsl = a.DV / pl.dvs;
  sp.xcd_map = (nheads % 8 == 0) ? 1 : 0;

  using LaunchFn = hipError_t (*)(int, int, int, const PrepParams&, int, const StateParams&, int,
                                  hipStream_t);
  static const LaunchFn table[2][3] = {
      {chunked::launch_f32_d0, chunked::launch_f32_d1, chunked::launch_f32_d2},
      {chunked::launch_bf16_d0, chunked::launch_bf16_d1, chunked::launch_bf16_d2}};
  const LaunchFn fn = table[a.dtype == 0 ? 0 : 1][a.decay_kind];
  for (int c0 = 0; c0 < nchunks; c0 += seg) {
    const int n = nchunks - c0 < seg ? nchunks - c0 : seg;
    pp.c0 = c0; pp.nchunks = n;
    sp.c0 = c0; sp.nchunks = n;
    // the state entering a later segment is the one the previous segment left
    sp.init = c0 == 0 ? a.init : a.state;
    e = fn(a.DK, pl.dvs, a.chunk, pp, nheads * n, sp, nheads * sp.nsl, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {

// cb[0] = 0, cb[n + 1] = cb[n] + ceil((cu[n + 1] - cu[n]) / C): one wave,
// an inclusive lane scan per 64 sequences.
__global__ void chunk_offsets_kernel(const int* __restrict__ cu, int* __restrict__ cb, int nseq, int C) {
  const int lane = threadIdx.x;
  int carry = 0;
  if (lane == 0) cb[0] = 0;
  for (int base = 0; base < nseq; base += 64) {
    const int n = base + lane;
    int x = n < nseq ? (cu[n + 1] - cu[n] + C - 1) / C : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (n < nseq) cb[n + 1] = carry + x;
    carry += __shfl(x, 63, 64);
  }
}

}  // namespace

hipError_t launch_chunked_varlen(const FwdArgs& a, const int* cu_dev, const int* cu_host, int nseq,
                                 void* ws, hipStream_t s) {
  const bool chan = a.decay_kind == DECAY_CHANNEL;
  const Plan pl = plan_for(nseq, a.H, a.DK, a.DV, a.chunk, a.dtype, chan);
  if (pl.dvs == 0) return hipErrorInvalidConfiguration;
  long total = 0;   // chunks of all sequences
  for (int n = 0; n < nseq; ++n) total += (cu_host[n + 1] - cu_host[n] + a.chunk - 1) / a.chunk;
  const size_t rec = a.dtype == 0 ? chunked::record_bytes<4>(a.DK, a.chunk, chan)
                                  : chunked::record_bytes<2>(a.DK, a.chunk, chan);
  if (rec == 0) return hipErrorInvalidConfiguration;
  const size_t recs = rec * static_cast<size_t>(total) * a.H;
  hipError_t e = hipSuccess;
  int* cb = reinterpret_cast<int*>(static_cast<unsigned char*>(ws) + recs);
  chunk_offsets_kernel<<<dim3(1), dim3(64), 0, s>>>(cu_dev, cb, nseq, a.chunk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (total == 0) {
    // every sequence is empty: the final states are the initial ones
    return launch_state_copy(a.init, a.state, static_cast<long>(nseq) * a.H * a.DK * a.DV, s);
  }

  PrepParams pp;
  pp.cu = cu_dev; pp.cb = cb; pp.nseq = nseq;
  pp.q = a.q; pp.k = a.k; pp.beta = a.beta; pp.decay = a.decay;
  pp.ws = static_cast<unsigned char*>(ws);
  pp.T = a.T; pp.H = a.H; pp.l2norm = a.l2norm; pp.scale = a.scale;
  pp.tf = a.tf;
  pp.Hk = a.Hk;
  pp.hk_magic = ((1ULL << 32) + a.H / a.Hk - 1) / (a.H / a.Hk);
  pp.c0 = 0; pp.nchunks = static_cast<int>(total);

  StateParams sp;
  sp.cu = cu_dev; sp.cb = cb;
  sp.q = a.q; sp.k = a.k;
  sp.l2norm = a.l2norm; sp.scale = a.scale;
  sp.v = a.v; sp.ws = static_cast<const unsigned char*>(ws);
  sp.o = a.o; sp.state = a.state; sp.init = a.init;
  sp.T = a.T; sp.H = a.H; sp.DV = a.DV;
  sp.Hk = a.Hk; sp.vfirst = a.vfirst; sp.hk_magic = pp.hk_magic;
  sp.nsl = a.DV / pl.dvs;
  const int nheads = nseq * a.H;
  sp.xcd_map = (nheads % 8 == 0) ? 1 : 0;
  sp.c0 = 0; sp.nchunks = static_cast<int>(total);

  using LaunchFn = hipError_t (*)(int, int, int, const PrepParams&, int, const StateParams&, int,
                                  hipStream_t);
  static const LaunchFn table[2][3] = {
      {chunked::launch_f32_d0, chunked::launch_f32_d1, chunked::launch_f32_d2},
      {chunked::launch_bf16_d0, chunked::launch_bf16_d1, chunked::launch_bf16_d2}};
  const LaunchFn fn = table[a.dtype == 0 ? 0 : 1][a.decay_kind];
  return fn(a.DK, pl.dvs, a.chunk, pp, a.H * static_cast<int>(total), sp, nheads * sp.nsl, s);
}

}  // namespace kda
