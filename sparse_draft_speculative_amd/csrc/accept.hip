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

__device__ __forceinline__ void consider(Best& b, float x, int j) {
  // elements reach a thread in increasing id order: the first maximum wins
  if (x > b.v || b.i == 0x7fffffff) { b.v2 = fmaxf(b.v2, b.v); b.v = x; b.i = j; }
  else b.v2 = fmaxf(b.v2, x);
}

// One workgroup per logit row.  Rows whose length is a multiple of 8 are read
// with 16-byte loads (8 ids per thread per step), others element by element.
template <typename T>
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
      if (margins) margins[row] = __builtin_nanf("");
    }
    return;
  }
  const T* lr = logits + (size_t)row * vocab;
  Best b{-INFINITY, 0x7fffffff, -INFINITY};
  constexpr int kVec = 16 / sizeof(T);                 // ids per 16-byte load
  const bool vec = (vocab % 8) == 0 && (reinterpret_cast<uintptr_t>(lr) & 15) == 0;
  if (vec) {
    const int nchunk = vocab / kVec;
#pragma unroll 4
    for (int c = tid; c < nchunk; c += kArgmaxThreads) {
      const uint4 u = *reinterpret_cast<const uint4*>(lr + (size_t)c * kVec);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          consider(b, bf16_bits_to_f32((w[e / 2] >> (16 * (e & 1))) & 0xffffu), c * 8 + e);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) consider(b, __uint_as_float(w[e]), c * 4 + e);
      }
    }
  } else {
    for (int j = tid; j < vocab; j += kArgmaxThreads) consider(b, Elem<T>::load(lr, j), j);
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
    if (margins) margins[row] = vocab > 1 ? r.v - r.v2 : INFINITY;
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
  if (bf16)
    argmax_rows<uint16_t><<<rows, kArgmaxThreads, 0, st>>>(
        static_cast<const uint16_t*>(logits), vocab, gamma, gamma_dev, out_tokens, margins);
  else
    argmax_rows<float><<<rows, kArgmaxThreads, 0, st>>>(static_cast<const float*>(logits), vocab,
                                                       gamma, gamma_dev, out_tokens, margins);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  accept_commit<<<batch, 64, 0, st>>>(draft, gamma, gamma_dev, out_tokens, n_out, seq_len);
  return hipGetLastError();
}

}  // namespace stdspec
