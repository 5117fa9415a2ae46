// Device-side check of a selected index list (debug aid).
//
// The sparse draft call takes, per KV head, positions inside the visual
// span in ascending order without repeats (the form the selection call
// returns them in).  The attention kernels do not verify that; they only
// clamp each position into the span.  This kernel counts the entries that
// break the preconditions, so a caller can test a list it built itself.
//
// One workgroup walks every head's list with coalesced loads; entry j of a
// head is bad when it lies outside [vis_start, vis_end) or is not larger
// than entry j-1 of the same head (an unsorted list or a repeat).  The
// count is reduced in LDS and written with one plain store.

#include "common.hpp"

namespace stdspec {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_idx_kernel(
    const int32_t* __restrict__ idx, int n_kv_heads, int topk, int vis_start, int vis_end,
    int32_t* __restrict__ bad_out) {
  __shared__ int part[kCheckThreads / 64];
  const int tid = threadIdx.x;
  int bad = 0;
  const long long n = (long long)n_kv_heads * topk;
  for (long long e = tid; e < n; e += kCheckThreads) {
    const int j = (int)(e % topk);
    const int x = idx[e];
    const bool out_of_span = x < vis_start || x >= vis_end;
    const bool not_ascending = j > 0 && x <= idx[e - 1];
    bad += (out_of_span || not_ascending) ? 1 : 0;
  }
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_down(bad, off, 64);
  if ((tid & 63) == 0) part[tid >> 6] = bad;
  __syncthreads();
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < kCheckThreads / 64; ++w) total += part[w];
    *bad_out = total;
  }
}

}  // namespace

hipError_t launch_check_idx(const int32_t* idx, int n_kv_heads, int topk, int vis_start,
                            int vis_len, int32_t* bad_out, hipStream_t stream) {
  check_idx_kernel<<<1, kCheckThreads, 0, stream>>>(idx, n_kv_heads, topk, vis_start,
                                                    vis_start + vis_len, bad_out);
  return hipGetLastError();
}

}  // namespace stdspec
