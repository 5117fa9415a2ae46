// Greedy acceptance plus the bonus token (gfx950, wave64).
//
// Technical summary, Methodology item 3 ("decoding procedure"): verification
// finds the longest prefix of drafted tokens matching the dense model's
// predictions (n tokens) and accepts one extra bonus token; the accepted
// tokens are appended to the context.
//
//  argmax_rows  -- one 1024-thread workgroup per logit row: argmax (ties to
//                  the lowest id) and margin = top1 - top2.  The prediction
//                  is written straight into out_tokens[row].
//  accept_commit -- one wave per sequence: n = length of the agreeing
//                  prefix, n_out = n+1, slots after the bonus set to -1,
//                  optional seq_len += n+1.
// A batch may give each sequence its own draft length gamma_b <= gamma (the
// row stride): rows past gamma_b + 1 are not read.

#include "common.hpp"
#include "internal.hpp"

namespace stdspec {
namespace {

struct Best {
  float v;     // best value
  int i;       // its id (lowest on ties)
  float v2;    // best value among all other ids
};

__device__ __forceinline__ Best merge(Best a, Best b) {
  const bool a_wins = a.v > b.v || (a.v == b.v && a.i < b.i);
  Best r;
  if (a_wins) { r.v = a.v; r.i = a.i; r.v2 = fmaxf(a.v2, b.v); }
  else        { r.v = b.v; r.i = b.i; r.v2 = fmaxf(b.v2, a.v); }
  return r;
}

constexpr int kArgmaxThreads = 1024;

// Draft length of sequence b: gamma_dev[b] clamped into [0, gamma], or gamma.
__device__ __forceinline__ int seq_gamma(const int32_t* gamma_dev, int b, int gamma) {
  return gamma_dev ? min(max(gamma_dev[b], 0), gamma) : gamma;
}

// Elements reach a thread in increasing id order, so only a strictly larger
// value takes over (the first maximum wins); the runner-up is the larger of
// the old runner-up and the smaller of (best, x).
__device__ __forceinline__ void consider(Best& b, float x, int j) {
  b.i = x > b.v ? j : b.i;
  b.v2 = fmaxf(b.v2, fminf(b.v, x));
  b.v = fmaxf(b.v, x);
}

// The ids of one 16-byte chunk of a row as fp32 values.
template <typename T>
__device__ __forceinline__ void chunk_values(const uint4& u, float (&x)[16 / sizeof(T)]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      x[e] = __uint_as_float((e & 1) ? (w[e / 2] & 0xffff0000u) : (w[e / 2] << 16));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
  }
}

// One workgroup per logit row.  Rows whose length is a multiple of 8 are read
// with 16-byte loads (8 bf16 or 4 fp32 ids per thread per step), others
// element by element.  On the 16-byte path a thread keeps its best value and
// the first chunk that holds it (a chunk takes over only with a strictly
// larger maximum, so the earliest chunk wins ties); the id inside that chunk
// is found once at the end by reading the chunk again.  The runner-up value
// is tracked element by element only when margins are asked for.
template <typename T, bool MARGIN>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_rows(const T* __restrict__ logits,
                                                              int vocab, int gamma,
                                                              const int32_t* __restrict__ gamma_dev,
                                                              int32_t* __restrict__ pred,
                                                              float* __restrict__ margins) {
  __shared__ Best sh[kArgmaxThreads / kWave];
  const int row = blockIdx.x, tid = threadIdx.x;
  // row i of sequence b; rows past the sequence's own gamma_b + 1 are unused
  if (gamma_dev && row % (gamma + 1) > seq_gamma(gamma_dev, row / (gamma + 1), gamma)) {
    if (tid == 0) {
      pred[row] = -1;
      if (MARGIN) margins[row] = __builtin_nanf("");
    }
    return;
  }
  const T* lr = logits + (size_t)row * vocab;
  constexpr int kVec = 16 / sizeof(T);                 // ids per 16-byte load
  const bool vec = (vocab % 8) == 0 && (reinterpret_cast<uintptr_t>(lr) & 15) == 0;
  // a thread that sees no id keeps the sentinel id and -inf, which loses
  // every merge against a thread that saw one
  Best b{-INFINITY, 0x7fffffff, -INFINITY};
  if (vec) {
    const int nchunk = vocab / kVec;
    int cb = tid < nchunk ? tid : -1;                  // chunk holding the best so far
#pragma unroll 4
    for (int c = tid; c < nchunk; c += kArgmaxThreads) {
      float x[kVec];
      chunk_values<T>(*reinterpret_cast<const uint4*>(lr + (size_t)c * kVec), x);
      float m = x[0];
#pragma unroll
      for (int e = 1; e < kVec; ++e) m = fmaxf(m, x[e]);
      if constexpr (MARGIN) {
        float v = b.v;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          b.v2 = fmaxf(b.v2, fminf(v, x[e]));
          v = fmaxf(v, x[e]);
        }
      }
      cb = m > b.v ? c : cb;
      b.v = fmaxf(b.v, m);
    }
    if (cb >= 0) {                                     // the best's id inside its chunk
      float x[kVec];
      chunk_values<T>(*reinterpret_cast<const uint4*>(lr + (size_t)cb * kVec), x);
      int e0 = kVec - 1;
#pragma unroll
      for (int e = kVec - 1; e >= 0; --e) e0 = x[e] == b.v ? e : e0;
      b.i = cb * kVec + e0;
    }
  } else {
    for (int j = tid; j < vocab; j += kArgmaxThreads) consider(b, Elem<T>::load(lr, j), j);
    if (tid < vocab && b.i == 0x7fffffff) b.i = tid;   // every value it saw was -inf
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    Best other;
    other.v = __shfl_xor(b.v, o, kWave);
    other.i = __shfl_xor(b.i, o, kWave);
    other.v2 = __shfl_xor(b.v2, o, kWave);
    b = merge(b, other);
  }
  if ((tid & 63) == 0) sh[tid >> 6] = b;
  __syncthreads();
  if (tid == 0) {
    Best r = sh[0];
    for (int w = 1; w < kArgmaxThreads / kWave; ++w) r = merge(r, sh[w]);
    pred[row] = r.i;
    if (MARGIN) margins[row] = vocab > 1 ? r.v - r.v2 : INFINITY;
  }
}

__global__ __launch_bounds__(64) void accept_commit(const int32_t* __restrict__ draft, int gamma,
                                                    const int32_t* __restrict__ gamma_dev,
                                                    int32_t* __restrict__ out_tokens,
                                                    int32_t* __restrict__ n_out,
                                                    int32_t* __restrict__ seq_len) {
  // workgroup b: sequence b of a batch ([b][gamma] drafts, [b][gamma+1] tokens)
  const int b = blockIdx.x;
  draft += (size_t)b * gamma;
  out_tokens += (size_t)b * (gamma + 1);
  n_out += b;
  if (seq_len) seq_len += b;
  __shared__ int sh_n;
  const int lane = threadIdx.x;
  const int gb = seq_gamma(gamma_dev, b, gamma);     // this sequence's drafts
  if (lane == 0) sh_n = gb;
  __syncthreads();
  // first j with draft[j] != pred[j] (pred lives in out_tokens)
  for (int base = 0; base < gb; base += 64) {
    const int j = base + lane;
    const bool miss = j < gb && draft[j] != out_tokens[j];
    const unsigned long long mask = __ballot(miss);
    if (mask) {
      if (lane == 0) sh_n = base + __ffsll((long long)mask) - 1;
      break;
    }
  }
  __syncthreads();
  const int n = sh_n;
  for (int j = n + 1 + lane; j <= gamma; j += 64) out_tokens[j] = -1;
  if (lane == 0) {
    n_out[0] = n + 1;
    if (seq_len) seq_len[0] += n + 1;
  }
}

}  // namespace

hipError_t launch_accept(const int32_t* draft, int gamma, int batch, const int32_t* gamma_dev,
                         const void* logits, int vocab, bool bf16, int32_t* out_tokens,
                         int32_t* n_out, float* margins, int32_t* seq_len, hipStream_t st) {
  // one argmax workgroup per logit row of every sequence ([batch][gamma+1]
  // rows back to back), then one commit wave per sequence
  const int rows = batch * (gamma + 1);
  const auto* lb = static_cast<const uint16_t*>(logits);
  const auto* lf = static_cast<const float*>(logits);
  if (bf16 && margins)
    argmax_rows<uint16_t, true><<<rows, kArgmaxThreads, 0, st>>>(lb, vocab, gamma, gamma_dev,
                                                                 out_tokens, margins);
  else if (bf16)
    argmax_rows<uint16_t, false><<<rows, kArgmaxThreads, 0, st>>>(lb, vocab, gamma, gamma_dev,
                                                                  out_tokens, margins);
  else if (margins)
    argmax_rows<float, true><<<rows, kArgmaxThreads, 0, st>>>(lf, vocab, gamma, gamma_dev,
                                                              out_tokens, margins);
  else
    argmax_rows<float, false><<<rows, kArgmaxThreads, 0, st>>>(lf, vocab, gamma, gamma_dev,
                                                               out_tokens, margins);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  accept_commit<<<batch, 64, 0, st>>>(draft, gamma, gamma_dev, out_tokens, n_out, seq_len);
  return hipGetLastError();
}

}  // namespace stdspec
