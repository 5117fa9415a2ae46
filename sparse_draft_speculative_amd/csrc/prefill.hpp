// Host-side declarations of the prefill text-row attention (prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace stdspec {

// Keys per workgroup chunk; the chunks' partials are merged by a second kernel.
constexpr int kPfChunk = 16384;

struct PrefillArgs {
  const void* q_text;   // [Hq][n_text][D] bf16
  const void* k;        // [Hkv][capacity][D] bf16
  const void* v;
  void* out;            // [Hq][n_text][D] bf16
  float* lse_out;       // [Hq][n_text] natural log, or null
  int hq, hkv, d, capacity, text_start, n_text;
  float scale;
  void* ws;             // prefill_workspace_bytes(hq, d, text_start, n_text)
};

size_t prefill_workspace_bytes(int hq, int d, int text_start, int n_text);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace stdspec
