// Streaming-read probe (measurement harness, not a step of the method).
//
// Reads a device buffer once, as fast as this part allows, so that the
// HBM-bound kernels (sparse draft, dense verify) can be reported against
// the bandwidth a plain sweep actually attains beside the nominal 8 TB/s.
//
// A fixed grid of one workgroup per CU walks the buffer in 16 KB tiles,
// tile t going to workgroup t mod grid; each lane issues four 16-byte
// non-temporal loads per tile (the hint reads a once-read stream faster),
// two tiles in flight.  The loaded words are folded into an XOR
// digest (one word per lane) so the loads cannot be dropped; its value has
// no meaning beyond that.

#include "common.hpp"
#include "stdspec.h"

namespace stdspec {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeGrid = STD_PROBE_SINK_WORDS / kProbeThreads;   // one digest word per lane
constexpr int kProbeLoads = 4;                              // 16-byte loads per lane per tile
constexpr int kProbeTile16 = kProbeThreads * kProbeLoads;   // 16-byte elements per tile

__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe(const u32x4_t* __restrict__ p,
                                                                size_t n16,
                                                                uint32_t* __restrict__ sink) {
  const size_t ntiles = (n16 + kProbeTile16 - 1) / kProbeTile16;
  const size_t full = n16 / kProbeTile16;                  // tiles with every element present
  u32x4_t acc = {0u, 0u, 0u, 0u};
  size_t t = blockIdx.x;
#pragma unroll 2
  for (; t < full; t += gridDim.x) {
    const u32x4_t* src = p + t * kProbeTile16 + threadIdx.x;
    u32x4_t x[kProbeLoads];
#pragma unroll
    for (int i = 0; i < kProbeLoads; ++i) x[i] = __builtin_nontemporal_load(src + i * kProbeThreads);
#pragma unroll
    for (int i = 0; i < kProbeLoads; ++i) acc ^= x[i];
  }
  if (t < ntiles) {                                         // the ragged last tile
    for (int i = 0; i < kProbeLoads; ++i) {
      const size_t e = t * kProbeTile16 + (size_t)i * kProbeThreads + threadIdx.x;
      if (e < n16) acc ^= p[e];
    }
  }
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                 hipStream_t stream) {
  hbm_read_probe<<<kProbeGrid, kProbeThreads, 0, stream>>>(static_cast<const u32x4_t*>(buf),
                                                          bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace stdspec
