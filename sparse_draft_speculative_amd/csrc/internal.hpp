// Host-side declarations shared by the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace stdspec {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int pow2_floor(long long x) {
  int p = 1;
  while ((long long)p * 2 <= x) p *= 2;
  return p;
}

// ---------------------------------------------------------------------------
// Split-K geometry.
//
// Dense verify: the len keys form ceil(len/64) tiles of 64 keys; split s of
// S takes tiles s, s+S, s+2S, ...  S depends only on (len, n_kv_heads),
// never on n_q, so a query row sees the same splits and the same reduction
// order whatever the number of rows in the call.  S is sized so one layer
// launches about 208 workgroups, one round at one per CU.  Measured on the
// 140k-key layer: 208 workgroups with two tiles in flight each stream the
// cache faster than 256 with three (52.9 against 54.0 us per call with
// non-temporal copies, 56.8 against 59.1 without); past about 13 MB in
// flight the HBM requests contend, below about 160 workgroups too few are
// in flight.
constexpr int kDenseWorkgroups = 208;
inline int dense_split_count(int len, int n_kv_heads) {
  const int tiles = (len + 63) / 64;
  const int target = n_kv_heads >= kDenseWorkgroups ? 1 : kDenseWorkgroups / n_kv_heads;
  return tiles < target ? tiles : target;
}

// Sparse decode: the per-head key list (prefix + selected + tail) is cut
// into splits of kSparseChunk entries, kSparseEntriesPerWave per wave
// (16, 32 or 64: one to four 16-key MFMA blocks).
constexpr int kSparseEntriesPerWave = 32;
constexpr int kSparseChunk = 128;

inline int sparse_list_len(int len, int vis_start, int vis_len, int topk) {
  return vis_start + topk + (len - (vis_start + vis_len));
}

// Split-K workspace: [ml: splits x rows x float2][o: splits x rows x
// head_dim floats]; scratch, no initialisation needed.
struct SplitWorkspace {
  int splits;     // number of key splits
  int rows;       // query rows = n_q * n_q_heads
  int head_dim;
  size_t ml_bytes, o_bytes;
  size_t bytes() const { return align256(ml_bytes) + align256(o_bytes); }
};

inline SplitWorkspace split_workspace(int splits, int rows, int head_dim) {
  SplitWorkspace w;
  w.splits = splits;
  w.rows = rows;
  w.head_dim = head_dim;
  w.ml_bytes = (size_t)splits * rows * 2 * sizeof(float);
  w.o_bytes = (size_t)splits * rows * head_dim * sizeof(float);
  return w;
}

// ---------------------------------------------------------------------------
// Kernel launchers (attention.hip).  All return the hipError_t of the launch.

struct AttnArgs {
  const void* q;        // dense: [n_q][Hq][D]; sparse: [Hq][D]
  const void* k;
  const void* v;
  void* out;
  int hq, hkv, d;
  float scale;
  int capacity, len, n_q;
  // device-resident length (null: use len); valid length min(*len_dev + len_off, len)
  // (sparse batch: len_dev[b] for sequence b)
  const int32_t* len_dev;
  int len_off;
  int len_lo;           // shortest valid length a device value resolves to
  // per-sequence draft lengths (sparse batch only, else null): sequence b
  // takes part in draft step `step` only while step < gamma_dev[b]
  const int32_t* gamma_dev;
  int step;
  // independent sequences laid out back to back (q, out [batch][n_q][Hq][D],
  // K and V [batch][Hkv][capacity][D], sparse idx [batch][Hkv][topk],
  // len_dev[b]); 0 or 1: one sequence
  int batch;
  bool bf16;
  // sparse key list; for dense, sparse == false
  bool sparse;
  const int32_t* idx;
  int vis_start, vis_len, topk;
  // workspace
  float* ml;            // [splits][rows][2]
  float* o;             // [splits][rows][D]
  int splits;
  int chunk;            // keys (dense) or list entries (sparse) per split
  int passes;           // sparse MFMA path: kSparseChunk-entry passes per split (1 or 2)
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

// Selection (select.hip).
struct SelectArgs {
  const void* q_text;   // [Hq][n_text][D]
  const void* k;        // [Hkv][capacity][D]
  int hq, hkv, d;
  float scale;
  int capacity;
  int text_start, n_text;
  int vis_start, vis_len, topk;
  bool bf16;
  const float* lse_in;  // optional natural-log LSE [Hq][n_text]
  int32_t* idx_out;
  float* scores_out;    // [Hkv][vis_len] (caller's or workspace)
  void* ws;
};

size_t select_workspace_bytes(int hq, int hkv, int d, int n_text, int vis_len,
                              int text_start, bool scores_in_ws);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

// Acceptance (accept.hip).
// gamma is the row stride ([batch][gamma] drafts, [batch][gamma+1] logit
// rows); gamma_dev (null: every sequence uses gamma) holds each sequence's
// own draft length, clamped into [0, gamma].
hipError_t launch_accept(const int32_t* draft, int gamma, int batch, const int32_t* gamma_dev,
                         const void* logits, int vocab, bool bf16, int32_t* out_tokens,
                         int32_t* n_out, float* margins, int32_t* seq_len, hipStream_t stream);

// Streaming-baseline index lists (check.hip): [n_kv_heads][topk] positions,
// the first min(sink, topk) of the span then its last topk - min(sink, topk).
hipError_t launch_static_window_idx(int n_kv_heads, int vis_start, int vis_len, int sink,
                                    int topk, int32_t* idx_out, hipStream_t stream);

}  // namespace stdspec
