// Prefill-time top-K visual KV selection (gfx950, wave64).
//
// Technical summary, Methodology item 4 ("KV cache selection"): the top-K
// visual KV are chosen at prefill from the average attention score that
// text tokens direct at visual tokens, separately per layer and per head.
// Three steps:
//   1. row normaliser  lse2[h][i] = log2 sum_{j <= pos_i} 2^(c * q_hi . k_j)
//      (c = scale * log2 e), over every key text row i sees;
//   2. column score    score[g][j] = 1/(G n_text) sum_{h in g, i}
//                                    2^(c q_hi . k_j - lse2[h][i]),  j visual;
//   3. top-K           radix select of the K largest fp32 scores per KV head,
//                      ties to the lower position, emitted in ascending
//                      position order by a stable compaction.
// Steps 1-2 run on MFMA for bf16 (the text rows x visual keys product is a
// real GEMM) and on the vector ALU for fp32.  Cross-tile sums accumulate in
// fp64; every reduction has a fixed order (no atomics), so results are
// bitwise reproducible and two identical key rows get identical scores.

#include "common.hpp"
#include "internal.hpp"
#include "tile.hpp"

namespace stdspec {
namespace {

constexpr int kLseChunk = 8192;     // keys per workgroup in step 1 (MFMA)
constexpr int kRowsPerLseWg = 128;  // text rows per workgroup in step 1
constexpr int kColsPerScoreWg = 256;  // visual keys per workgroup in step 2
constexpr int kXcds = 8;

// Workgroup ids are dispatched round-robin over the 8 XCDs (each with its
// own L2).  Map them so that each XCD receives a contiguous run of work
// items: items that share an operand (a key chunk in step 1, a head's text
// queries in step 2) then meet in the same L2.
__device__ __forceinline__ int xcd_item(int bid, int n_items) {
  const int per = (n_items + kXcds - 1) / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

struct Geo {
  int hq, hkv, G, D, capacity;
  int text_start, n_text;
  int vis_start, vis_len;
  float c;  // scale * log2 e
};

// Stage one 64-row tile of a [rows][D] bf16 tensor: global -> registers
// (rows clamped to ``last``, so every load is in bounds) and registers ->
// LDS in the K-swizzled layout of Tile<D>.
template <int D, int KPT>
__device__ __forceinline__ void tile_load(u32x4_t (&r)[KPT], const uint16_t* base, int row0,
                                          int last, const int (&rrow)[KPT],
                                          const int (&rslot)[KPT]) {
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const size_t off = (size_t)min(row0 + rrow[u], last) * D;
    r[u] = *reinterpret_cast<const u32x4_t*>(base + off + (Tile<D>::slot_k(rrow[u], rslot[u]) << 3));
  }
}
template <int D, int KPT>
__device__ __forceinline__ void tile_store(const u32x4_t (&r)[KPT], uint16_t* lds,
                                           const int (&rrow)[KPT], const int (&rslot)[KPT]) {
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    *reinterpret_cast<u32x4_t*>(lds + rrow[u] * D + (rslot[u] << 3)) = r[u];
}

// ---------------------------------------------------------------------------
// Step 1 (bf16, MFMA): partial (max, sum) of each text row over one key chunk.
// Work item = (KV head, key chunk, 128-row block); 4 waves x 32 rows.  Keys
// are staged in LDS (64 per tile, double buffered, the next tiles' loads in
// flight in two register buffers) and are the M side of S^T = K Q^T, rows
// the N side.  Each lane keeps its own running (max, fp64 sum) over the keys
// it sees; the max moves only when a score exceeds it by 2^8 (exact: it is
// only the shift of the exponent), and the four lanes of a column are merged
// once at the end.  Only tiles that reach the causal (text) part or the
// chunk end are masked.
template <int D>
__device__ __forceinline__ void lse_tile(const uint16_t* Ks, const bf16x8_t (*qb)[D / 32],
                                         int t0, int key1, int text_start, const int* rpos,
                                         float c, int col, int grp, float* m, double* l) {
  constexpr int KST = D / 32;
  floatx4_t sacc[4][2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    u32x4_t a[KST];
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      a[kk] = *reinterpret_cast<const u32x4_t*>(Ks + Tile<D>::off_k(kb * 16 + col, KST * grp + kk));
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) acc = mfma_bf16(as_bf16x8(a[kk]), qb[nb][kk], acc);
      sacc[kb][nb] = acc;
    }
  }
  const bool masked = t0 + 64 > text_start || t0 + 64 > key1;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = sacc[j >> 2][nb][j & 3];
    if (masked) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = t0 + (j >> 2) * 16 + 4 * grp + (j & 3);
        if (!(key < key1 && key <= rpos[nb])) v[j] = -INFINITY;
      }
    }
    float tmax = v[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) tmax = fmaxf(tmax, v[j]);
    if (tmax == -INFINITY) continue;
    const float ts = tmax * c;                       // c > 0: max then scale
    if (ts > m[nb] + 8.f) {
      if (m[nb] != -INFINITY) l[nb] *= exp2((double)m[nb] - (double)ts);
      m[nb] = ts;
    }
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ps += fast_exp2(fmaf(v[j], c, -m[nb]));
    l[nb] += (double)ps;
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void lse_partial_mfma(const uint16_t* __restrict__ qt,
                                                           const uint16_t* __restrict__ k, Geo geo,
                                                           int n_chunks, int n_rb,
                                                           float* __restrict__ m_part,
                                                           double* __restrict__ l_part) {
  constexpr int KST = D / 32, CPR = D / 8, KPT = 64 * CPR / 256;
  __shared__ __align__(16) uint16_t Ks0[64 * D];
  __shared__ __align__(16) uint16_t Ks1[64 * D];
  const int n_items = geo.hkv * n_chunks * n_rb;
  const int item = xcd_item(blockIdx.x, n_items);
  if (item >= n_items) return;
  const int rb = item % n_rb;
  const int ch = (item / n_rb) % n_chunks;
  const int g = item / (n_rb * n_chunks);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int R = geo.G * geo.n_text;
  const int n_keys = geo.text_start + geo.n_text;
  const int key0 = ch * kLseChunk, key1 = min(n_keys, key0 + kLseChunk);

  bf16x8_t qb[2][KST];
  int rpos[2];
  bool rok[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int rho = rb * kRowsPerLseWg + wave * 32 + nb * 16 + col;
    rok[nb] = rho < R;
    rpos[nb] = geo.text_start + (rok[nb] ? rho % geo.n_text : 0);
    const uint16_t* qrow = qt + ((size_t)g * R + (rok[nb] ? rho : 0)) * D + (D / 4) * grp;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (rok[nb]) u = *reinterpret_cast<const uint4*>(qrow + 8 * kk);
      qb[nb][kk] = as_bf16x8(u);
    }
  }
  float m[2] = {-INFINITY, -INFINITY};
  double l[2] = {0.0, 0.0};

  const uint16_t* kh = k + (size_t)g * geo.capacity * D;
  int rrow[KPT], rslot[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int cl = tid + 256 * u;
    rrow[u] = cl / CPR;
    rslot[u] = cl % CPR;
  }
  const int ntiles = (key1 - key0 + 63) / 64;
  u32x4_t ra[KPT], rb_[KPT];
  tile_load<D, KPT>(ra, kh, key0, key1 - 1, rrow, rslot);
  tile_store<D, KPT>(ra, Ks0, rrow, rslot);
  tile_load<D, KPT>(ra, kh, key0 + 64, key1 - 1, rrow, rslot);
  tile_load<D, KPT>(rb_, kh, key0 + 128, key1 - 1, rrow, rslot);
  for (int t = 0; t < ntiles; t += 2) {
    __syncthreads();
    tile_store<D, KPT>(ra, Ks1, rrow, rslot);
    tile_load<D, KPT>(ra, kh, key0 + (t + 3) * 64, key1 - 1, rrow, rslot);
    lse_tile<D>(Ks0, qb, key0 + t * 64, key1, geo.text_start, rpos, geo.c, col, grp, m, l);
    __syncthreads();
    tile_store<D, KPT>(rb_, Ks0, rrow, rslot);
    tile_load<D, KPT>(rb_, kh, key0 + (t + 4) * 64, key1 - 1, rrow, rslot);
    if (t + 1 < ntiles)
      lse_tile<D>(Ks1, qb, key0 + (t + 1) * 64, key1, geo.text_start, rpos, geo.c, col, grp, m,
                  l);
  }
  // merge the four lanes of each column, then write this chunk's partial
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float mm = max_over_groups(m[nb]);
    double ll = (m[nb] == -INFINITY) ? 0.0 : l[nb] * exp2((double)m[nb] - (double)mm);
    ll += __shfl_xor(ll, 16, kWave);
    ll += __shfl_xor(ll, 32, kWave);
    const int rho = rb * kRowsPerLseWg + wave * 32 + nb * 16 + col;
    if (grp == 0 && rok[nb]) {
      const size_t slot = (size_t)ch * geo.hq * geo.n_text + (size_t)g * R + rho;
      m_part[slot] = mm;
      l_part[slot] = ll;
    }
  }
}

// Step 1 merge: lse2 = M + log2(sum_c l_c 2^(m_c - M)), one thread per row.
__global__ void lse_finalize(const float* __restrict__ m_part, const double* __restrict__ l_part,
                             int n_chunks, int rows, float* __restrict__ lse2) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float M = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, m_part[(size_t)c * rows + r]);
  double L = 0.0;
  for (int c = 0; c < n_chunks; ++c) {
    const float mc = m_part[(size_t)c * rows + r];
    if (mc != -INFINITY) L += l_part[(size_t)c * rows + r] * exp2((double)mc - (double)M);
  }
  lse2[r] = (float)((double)M + log2(L));
}

// Step 1 (vector ALU): one wave per text row over all its keys.
template <typename T, int D>
__global__ __launch_bounds__(64) void lse_valu(const T* __restrict__ qt, const T* __restrict__ k,
                                               Geo geo, float* __restrict__ lse2) {
  __shared__ float qs[D];
  const int r = blockIdx.x;  // row = h * n_text + i
  const int lane = threadIdx.x;
  const int h = r / geo.n_text, i = r % geo.n_text;
  const int g = h / geo.G;
  for (int d = lane; d < D; d += 64) qs[d] = Elem<T>::load(qt, (size_t)r * D + d);
  __syncthreads();
  const T* kh = k + (size_t)g * geo.capacity * D;
  const int last = geo.text_start + i;
  float m = -INFINITY;
  double l = 0.0;
  for (int t0 = 0; t0 <= last; t0 += 64) {
    const int key = t0 + lane;
    float x = -INFINITY;
    if (key <= last) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], Elem<T>::load(kh, (size_t)key * D + d), acc);
      x = acc * geo.c;
    }
    const float mnew = fmaxf(m, wave_max(x));
    if (m != -INFINITY && mnew > m) l *= exp2((double)m - (double)mnew);
    m = mnew;
    const float p = key <= last ? fast_exp2(x - m) : 0.f;
    l += wave_sum((double)p);
  }
  if (lane == 0) lse2[r] = (float)((double)m + log2(l));
}

// ---------------------------------------------------------------------------
// Step 2 (bf16, MFMA): column sums over all text rows of the group for 256
// visual keys.  S = Q K^T with rows on the M side (streamed through LDS, 64
// per tile, double buffered) and keys on the N side (4 blocks of 16 per
// wave, held in registers).  Each lane owns one key per block and sums its
// rows; partial sums of a tile are fp32 and are added into fp64
// accumulators; the four lanes of a key are merged at the end in fp64.
template <int D>
__global__ __launch_bounds__(256, 2) void colscore_mfma(const uint16_t* __restrict__ qt,
                                                        const uint16_t* __restrict__ k, Geo geo,
                                                        const float* __restrict__ lse,
                                                        float lse_factor, int n_ct,
                                                        float* __restrict__ scores) {
  constexpr int KST = D / 32, CPR = D / 8, KPT = 64 * CPR / 256;
  __shared__ __align__(16) uint16_t Qs0[64 * D];
  __shared__ __align__(16) uint16_t Qs1[64 * D];
  __shared__ float Ls[2][64];
  const int n_items = geo.hkv * n_ct;
  const int item = xcd_item(blockIdx.x, n_items);
  if (item >= n_items) return;
  const int ct = item % n_ct, g = item / n_ct;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int R = geo.G * geo.n_text;

  // key operands: B[k = d][n = key], key = base + kb*16 + col (clamped)
  bf16x8_t kbop[4][KST];
  const uint16_t* kh = k + (size_t)g * geo.capacity * D;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int j = min(ct * kColsPerScoreWg + wave * 64 + kb * 16 + col, geo.vis_len - 1);
    const uint16_t* krow = kh + (size_t)(geo.vis_start + j) * D + (D / 4) * grp;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      kbop[kb][kk] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(krow + 8 * kk));
  }
  double acc[4] = {0.0, 0.0, 0.0, 0.0};

  const uint16_t* qg = qt + (size_t)g * R * D;
  const float* lg = lse + (size_t)g * R;
  int rrow[KPT], rslot[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int cl = tid + 256 * u;
    rrow[u] = cl / CPR;
    rslot[u] = cl % CPR;
  }
  // row normalisers: rows past the end get +inf (probability 0)
  auto lse_of = [&](int row) { return row < R ? lg[row] * lse_factor : INFINITY; };

  // one 64-row tile: four 16-row blocks; a block's 16 MFMAs are issued
  // before the previous block's exponentials are summed
  auto tile = [&](const uint16_t* Qs, const float* L) {
    float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      u32x4_t a[KST];
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        a[kk] = *reinterpret_cast<const u32x4_t*>(Qs + Tile<D>::off_k(qb * 16 + col, KST * grp + kk));
      float lrow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) lrow[i] = L[qb * 16 + 4 * grp + i];
      floatx4_t sv[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        floatx4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) x = mfma_bf16(as_bf16x8(a[kk]), kbop[kb][kk], x);
        sv[kb] = x;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[kb] += fast_exp2(fmaf(sv[kb][i], geo.c, -lrow[i]));
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] += (double)cs[kb];
  };

  const int ntiles = (R + 63) / 64;
  u32x4_t ra[KPT], rb_[KPT];
  float la = 0.f, lb = 0.f;
  tile_load<D, KPT>(ra, qg, 0, R - 1, rrow, rslot);
  tile_store<D, KPT>(ra, Qs0, rrow, rslot);
  if (tid < 64) Ls[0][tid] = lse_of(tid);
  tile_load<D, KPT>(ra, qg, 64, R - 1, rrow, rslot);
  tile_load<D, KPT>(rb_, qg, 128, R - 1, rrow, rslot);
  if (tid < 64) { la = lse_of(64 + tid); lb = lse_of(128 + tid); }
  for (int t = 0; t < ntiles; t += 2) {
    __syncthreads();
    tile_store<D, KPT>(ra, Qs1, rrow, rslot);
    if (tid < 64) { Ls[1][tid] = la; la = lse_of((t + 3) * 64 + tid); }
    tile_load<D, KPT>(ra, qg, (t + 3) * 64, R - 1, rrow, rslot);
    tile(Qs0, Ls[0]);
    __syncthreads();
    tile_store<D, KPT>(rb_, Qs0, rrow, rslot);
    if (tid < 64) { Ls[0][tid] = lb; lb = lse_of((t + 4) * 64 + tid); }
    tile_load<D, KPT>(rb_, qg, (t + 4) * 64, R - 1, rrow, rslot);
    if (t + 1 < ntiles) tile(Qs1, Ls[1]);
  }
  const double inv = 1.0 / ((double)geo.G * (double)geo.n_text);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    double a = acc[kb];
    a += __shfl_xor(a, 16, kWave);
    a += __shfl_xor(a, 32, kWave);
    const int j = ct * kColsPerScoreWg + wave * 64 + kb * 16 + col;
    if (grp == 0 && j < geo.vis_len) scores[(size_t)g * geo.vis_len + j] = (float)(a * inv);
  }
}

// Step 2 (vector ALU): one wave per 64 visual keys; lane j keeps key j in
// registers and walks every text row of the group.
template <typename T, int D>
__global__ __launch_bounds__(64) void colscore_valu(const T* __restrict__ qt,
                                                    const T* __restrict__ k, Geo geo,
                                                    const float* __restrict__ lse,
                                                    float lse_factor, float* __restrict__ scores) {
  __shared__ float qs[64][D + 1];
  __shared__ float ls[64];
  const int ct = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x;
  const int j = ct * 64 + lane;
  const bool ok = j < geo.vis_len;
  const int R = geo.G * geo.n_text;
  float kr[D];
  const T* krow = k + ((size_t)g * geo.capacity + geo.vis_start + (ok ? j : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) kr[d] = Elem<T>::load(krow, d);
  const T* qg = qt + (size_t)g * R * D;
  double acc = 0.0;
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int nr = min(64, R - r0);
    __syncthreads();
    for (int e = lane; e < nr * D; e += 64) qs[e / D][e % D] = Elem<T>::load(qg, (size_t)r0 * D + e);
    if (lane < nr) ls[lane] = lse[(size_t)g * R + r0 + lane] * lse_factor;
    __syncthreads();
    float cs = 0.f;
    for (int r = 0; r < nr; ++r) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qs[r][d], kr[d], s);
      cs += fast_exp2(fmaf(s, geo.c, -ls[r]));
    }
    acc += (double)cs;
  }
  if (ok) scores[(size_t)g * geo.vis_len + j] = (float)(acc / ((double)geo.G * geo.n_text));
}

// ---------------------------------------------------------------------------
// Step 3: top-K per KV head.  One 1024-thread workgroup per head.
// Radix select on the fp32 bit patterns (non-negative floats order like
// their bits), 8 bits per pass from the top, finds the exact K-th largest
// value T and how many copies of T to keep; a stable compaction in position
// order then emits every score > T plus the lowest-positioned copies of T.

constexpr int kTopkThreads = 1024;

__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kTopkThreads / 64 ? red[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(w, o, kWave);
      if (lane >= o) w += y;
    }
    if (lane < kTopkThreads / 64) red[lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  total = red[kTopkThreads / 64 - 1];
  const int before = wave > 0 ? red[wave - 1] : 0;
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kTopkThreads) void radix_topk(const float* __restrict__ scores,
                                                           int vis_len, int vis_start, int topk,
                                                           int32_t* __restrict__ idx_out) {
  __shared__ unsigned hist[256];
  __shared__ int red[kTopkThreads / 64];
  __shared__ unsigned sh_prefix;
  __shared__ int sh_remaining;
  const int g = blockIdx.x;
  const unsigned* bits = reinterpret_cast<const unsigned*>(scores + (size_t)g * vis_len);
  const int tid = threadIdx.x;

  unsigned prefix = 0, pmask = 0;
  int remaining = topk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for (int j = tid; j < vis_len; j += kTopkThreads) {
      const unsigned b = bits[j];
      if ((b & pmask) == prefix) atomicAdd(&hist[(b >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, dgt = 0;
      for (int b = 255; b >= 0; --b) {
        if (cum + (int)hist[b] >= remaining) { dgt = b; break; }
        cum += hist[b];
      }
      sh_prefix = prefix | ((unsigned)dgt << shift);
      sh_remaining = remaining - cum;
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const unsigned T = prefix;
  const int need_eq = remaining;  // copies of T to keep, >= 1

  // stable compaction over contiguous per-thread segments
  const int per = (vis_len + kTopkThreads - 1) / kTopkThreads;
  const int j0 = min(vis_len, tid * per), j1 = min(vis_len, j0 + per);
  int n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    const unsigned b = bits[j];
    n_gt += b > T;
    n_eq += b == T;
  }
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, red, tot);
  const int take_eq = max(0, min(n_eq, need_eq - eq_before));
  const int off = block_exclusive_scan(n_gt + take_eq, red, tot);
  int32_t* dst = idx_out + (size_t)g * topk + off;
  int w = 0, eq_used = 0;
  for (int j = j0; j < j1; ++j) {
    const unsigned b = bits[j];
    const bool take = b > T || (b == T && eq_used < take_eq);
    eq_used += b == T;
    if (take) dst[w++] = vis_start + j;
  }
}

template <int D>
hipError_t launch_mfma_select(const SelectArgs& a, const Geo& geo, float* lse2, float* m_part,
                              double* l_part, hipStream_t st) {
  const auto* qt = static_cast<const uint16_t*>(a.q_text);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const float* lse = lse2;
  float factor = 1.f;
  if (a.lse_in) {
    lse = a.lse_in;
    factor = kLog2e;
  } else {
    const int n_keys = a.text_start + a.n_text;
    const int n_chunks = (n_keys + kLseChunk - 1) / kLseChunk;
    const int R = geo.G * a.n_text;
    const int n_rb = (R + kRowsPerLseWg - 1) / kRowsPerLseWg;
    const int n_items = a.hkv * n_chunks * n_rb;
    const int grid = ((n_items + kXcds - 1) / kXcds) * kXcds;
    lse_partial_mfma<D><<<grid, 256, 0, st>>>(qt, k, geo, n_chunks, n_rb, m_part, l_part);
    const int rows = a.hq * a.n_text;
    lse_finalize<<<(rows + 255) / 256, 256, 0, st>>>(m_part, l_part, n_chunks, rows, lse2);
  }
  const int n_ct = (a.vis_len + kColsPerScoreWg - 1) / kColsPerScoreWg;
  const int n_items = a.hkv * n_ct;
  const int grid = ((n_items + kXcds - 1) / kXcds) * kXcds;
  colscore_mfma<D><<<grid, 256, 0, st>>>(qt, k, geo, lse, factor, n_ct, a.scores_out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu_select(const SelectArgs& a, const Geo& geo, float* lse2, hipStream_t st) {
  const auto* qt = static_cast<const T*>(a.q_text);
  const auto* k = static_cast<const T*>(a.k);
  const float* lse = lse2;
  float factor = 1.f;
  if (a.lse_in) {
    lse = a.lse_in;
    factor = kLog2e;
  } else {
    lse_valu<T, D><<<a.hq * a.n_text, 64, 0, st>>>(qt, k, geo, lse2);
  }
  colscore_valu<T, D><<<dim3((a.vis_len + 63) / 64, a.hkv), 64, 0, st>>>(qt, k, geo, lse, factor,
                                                                        a.scores_out);
  return hipGetLastError();
}

struct SelectLayout {
  size_t lse2, m_part, l_part, scores, total;
};

SelectLayout select_layout(int hq, int hkv, int n_text, int vis_len, int text_start,
                           bool scores_in_ws) {
  SelectLayout L;
  const size_t rows = (size_t)hq * n_text;
  const int n_chunks = (text_start + n_text + kLseChunk - 1) / kLseChunk;
  size_t off = 0;
  L.lse2 = off;
  off += align256(rows * sizeof(float));
  L.m_part = off;
  off += align256((size_t)n_chunks * rows * sizeof(float));
  L.l_part = off;
  off += align256((size_t)n_chunks * rows * sizeof(double));
  L.scores = off;
  if (scores_in_ws) off += align256((size_t)hkv * vis_len * sizeof(float));
  L.total = off;
  return L;
}

}  // namespace

size_t select_workspace_bytes(int hq, int hkv, int /*d*/, int n_text, int vis_len, int text_start,
                              bool scores_in_ws) {
  return select_layout(hq, hkv, n_text, vis_len, text_start, scores_in_ws).total;
}

hipError_t launch_select(const SelectArgs& a0, hipStream_t st) {
  SelectArgs a = a0;
  const SelectLayout L =
      select_layout(a.hq, a.hkv, a.n_text, a.vis_len, a.text_start, a.scores_out == nullptr);
  char* ws = static_cast<char*>(a.ws);
  float* lse2 = reinterpret_cast<float*>(ws + L.lse2);
  float* m_part = reinterpret_cast<float*>(ws + L.m_part);
  double* l_part = reinterpret_cast<double*>(ws + L.l_part);
  if (!a.scores_out) a.scores_out = reinterpret_cast<float*>(ws + L.scores);
  Geo geo{a.hq, a.hkv, a.hq / a.hkv, a.d, a.capacity, a.text_start, a.n_text,
          a.vis_start, a.vis_len, a.scale * kLog2e};
  hipError_t err;
  if (a.bf16)
    err = a.d == 128 ? launch_mfma_select<128>(a, geo, lse2, m_part, l_part, st)
                     : launch_mfma_select<64>(a, geo, lse2, m_part, l_part, st);
  else
    err = a.d == 128 ? launch_valu_select<float, 128>(a, geo, lse2, st)
                     : launch_valu_select<float, 64>(a, geo, lse2, st);
  if (err != hipSuccess) return err;
  radix_topk<<<a.hkv, kTopkThreads, 0, st>>>(a.scores_out, a.vis_len, a.vis_start, a.topk,
                                             a.idx_out);
  return hipGetLastError();
}

}  // namespace stdspec
