// Index lists of the streaming-attention comparator (gfx950).
//
// The pages compare StD against a streaming-attention draft (technical
// summary, Experimental results), a KV policy that keeps a few initial
// "sink" positions and a window of recent positions instead of ranking them
// by attention.  Applied to the visual span only (text KV is kept whole, as
// for the StD draft), it is a fixed index list, so it runs through the same
// sparse draft call: for every KV head, the first s = min(sink, topk) visual
// positions followed by the last topk - s, in ascending order.  The two
// parts are disjoint because topk <= vis_len.
//
// One thread per list entry; entries are independent.

#include "common.hpp"

namespace stdspec {
namespace {

constexpr int kWindowThreads = 256;

__global__ __launch_bounds__(kWindowThreads) void static_window_kernel(
    int vis_start, int vis_len, int sink, int topk, long long n, int32_t* __restrict__ idx_out) {
  const long long e = (long long)blockIdx.x * kWindowThreads + threadIdx.x;
  if (e >= n) return;
  const int j = (int)(e % topk);                      // entry within its head's list
  const int s = min(sink, topk);
  idx_out[e] = j < s ? vis_start + j : vis_start + vis_len - (topk - j);
}

}  // namespace

hipError_t launch_static_window_idx(int n_kv_heads, int vis_start, int vis_len, int sink,
                                    int topk, int32_t* idx_out, hipStream_t stream) {
  const long long n = (long long)n_kv_heads * topk;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + kWindowThreads - 1) / kWindowThreads);
  static_window_kernel<<<blocks, kWindowThreads, 0, stream>>>(vis_start, vis_len, sink, topk, n,
                                                              idx_out);
  return hipGetLastError();
}

}  // namespace stdspec
