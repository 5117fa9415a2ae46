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
constexpr int kColKB = 3;            // 16-key blocks per wave in step 2
constexpr int kColWaves = 8;         // waves per workgroup in step 2
constexpr int kColOcc = 2;           // step-2 workgroups per CU
constexpr int kColBufs = 4;          // LDS tile buffers in step 2 (a power of two)
constexpr int kColThreads = 64 * kColWaves;
constexpr int kColsPerScoreWg = kColWaves * 16 * kColKB;  // visual keys per workgroup in step 2
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

// ---------------------------------------------------------------------------
// Step 1 (bf16, MFMA): partial (max, sum) of each text row over one key chunk.
//
// Work item = (KV head, key chunk, kLseRowsWg-row block).  Each wave keeps
// kLseRB blocks of 16 text rows as MFMA operands in registers; the
// workgroup streams the chunk's keys through LDS in 64-key tiles by
// direct-to-LDS copies (kLseBufs buffers, kLseBufs - 1 tiles in flight).
// Scores are S^T = K Q^T (keys on the M side), so each key fragment read
// from LDS feeds kLseRB MFMA column blocks and lane (col, grp) gets keys
// 4 grp + i of every 16-key block for row col.  Each lane keeps a running
// (max, sum) per row block over the keys it sees; the max moves only when
// a score exceeds it by 2^8 (exact: it only shifts the exponent).  The sum
// of a tile is fp32, the running sum fp64.  The four lanes of a row are
// merged once at the end.  Only tiles that reach the causal (text) part or
// the chunk end are masked.
constexpr int kLseRB = 2;                          // 16-row blocks per wave
constexpr int kLseWaves = 8;                       // waves per workgroup
constexpr int kLseThreads = 64 * kLseWaves;
constexpr int kLseOcc = 2;                         // workgroups per CU (the launch bound
                                                   // asks for the matching waves per SIMD)
constexpr int kLseBufs = 4;                        // LDS key-tile buffers (a power of two)
constexpr int kLseRowsWg = kLseWaves * 16 * kLseRB;   // text rows per workgroup

struct LseState {
  float m[kLseRB];      // running max (base-2 units) per row block
  double l[kLseRB];     // sum relative to m
};

// Where a tile reaches the chunk end or the causal part, the scores of keys
// at or past key1 or after the row's own position are -inf.  Row rho of the
// group is text row rho % n_text (the G heads' rows are stacked).
struct LseMask {
  int key1, R, n_text, text_start;
  __device__ __forceinline__ void apply(floatx4_t& v, int rho, int key_base) const {
    const int rpos = text_start + (rho < R ? rho % n_text : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key_base + i;
      if (!(key < key1 && key <= rpos)) v[i] = -INFINITY;
    }
  }
};

// The scores of one 16-key block (LDS rows kb*16 ..) against the wave's row
// blocks: v[rb] holds keys 4 grp + i for row col of block rb.
template <int D, bool MASK>
__device__ __forceinline__ void lse_block(const uint16_t* Kt, const bf16x8_t (*qb)[D / 32], int kb,
                                          int col, int grp, const LseMask& mk, int row0,
                                          int key_base, floatx4_t (&v)[kLseRB]) {
  constexpr int KST = D / 32;
  u32x4_t a[KST];
#pragma unroll
  for (int kk = 0; kk < KST; ++kk)
    a[kk] = *reinterpret_cast<const u32x4_t*>(Kt + Tile<D>::off_k(kb * 16 + col, KST * grp + kk));
#pragma unroll
  for (int rb = 0; rb < kLseRB; ++rb) {
    floatx4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) x = mfma_bf16(as_bf16x8(a[kk]), qb[rb][kk], x);
    if constexpr (MASK) mk.apply(x, row0 + rb * 16 + col, key_base);
    v[rb] = x;
  }
}

// One 64-key tile.  Fast path: the probabilities relative to the running
// max are summed directly; each is at most 2^8 while the max invariant
// holds, so a tile sum above 2^8 (or NaN: an unset max against a masked
// score) flags a lane whose max may have to move.  Then the whole wave (the
// MFMAs cover every lane, so none may sit under a lane-dependent branch)
// takes the slow path: it recomputes the tile's scores block by block and,
// for the flagged lanes, moves the max to a block's max where that exceeds
// max + 8 (rescaling the running and the partial tile sum) before adding
// the block; all with selects.
template <int D, bool MASK>
__device__ __forceinline__ void lse_tile(const uint16_t* Kt, const bf16x8_t (*qb)[D / 32], int t0,
                                         const LseMask& mk, int row0, float c, int col, int grp,
                                         LseState& st) {
  float tot[kLseRB];
#pragma unroll
  for (int rb = 0; rb < kLseRB; ++rb) tot[rb] = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    floatx4_t v[kLseRB];
    lse_block<D, MASK>(Kt, qb, kb, col, grp, mk, row0, t0 + kb * 16 + 4 * grp, v);
#pragma unroll
    for (int rb = 0; rb < kLseRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[rb] += fast_exp2(fmaf(v[rb][i], c, -st.m[rb]));
  }
  bool ok = true;
#pragma unroll
  for (int rb = 0; rb < kLseRB; ++rb) ok = ok && (tot[rb] <= 256.f);
  if (__any(!ok)) {                    // wave-uniform
    bool need[kLseRB];
    float t2[kLseRB];
#pragma unroll
    for (int rb = 0; rb < kLseRB; ++rb) {
      need[rb] = !(tot[rb] <= 256.f);
      t2[rb] = 0.f;
    }
#pragma unroll 1
    for (int kb = 0; kb < 4; ++kb) {
      floatx4_t v[kLseRB];
      lse_block<D, MASK>(Kt, qb, kb, col, grp, mk, row0, t0 + kb * 16 + 4 * grp, v);
#pragma unroll
      for (int rb = 0; rb < kLseRB; ++rb) {
        const float bm = fmaxf(fmaxf(v[rb][0], v[rb][1]), fmaxf(v[rb][2], v[rb][3]));
        const float ts = bm * c;       // c > 0: max then scale
        const bool move = need[rb] && bm != -INFINITY && ts > st.m[rb] + 8.f;
        const bool had = st.m[rb] != -INFINITY;
        const double scale = exp2((double)(had ? st.m[rb] : ts) - (double)ts);
        st.l[rb] = move ? st.l[rb] * scale : st.l[rb];
        t2[rb] = move ? (float)((double)t2[rb] * scale) : t2[rb];
        st.m[rb] = move ? ts : st.m[rb];
        float b = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) b += fast_exp2(fmaf(v[rb][i], c, -st.m[rb]));
        t2[rb] += bm == -INFINITY ? 0.f : b;
      }
    }
#pragma unroll
    for (int rb = 0; rb < kLseRB; ++rb) tot[rb] = need[rb] ? t2[rb] : tot[rb];
  }
#pragma unroll
  for (int rb = 0; rb < kLseRB; ++rb) st.l[rb] += (double)tot[rb];
}

template <int D>
__global__ __launch_bounds__(kLseThreads, kLseOcc * kLseWaves / 4) void lse_partial_mfma(
    const uint16_t* __restrict__ qt, const uint16_t* __restrict__ k, Geo geo, int n_chunks,
    int n_rb, float* __restrict__ m_part, double* __restrict__ l_part) {
  constexpr int KST = D / 32, CPR = D / 8;
  constexpr int LPT = 64 * CPR / kLseThreads;   // direct-to-LDS copies per thread and tile
  static_assert(LPT * kLseThreads == 64 * CPR, "a tile is a whole number of copies per thread");
  constexpr int NB = kLseBufs;
  constexpr int TILE = 64 * D;
  __shared__ __align__(16) uint16_t Kbuf[NB * TILE];
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
  const int row0 = rb * kLseRowsWg + wave * 16 * kLseRB;   // first row of the wave

  // Q operands: B[k = d][n = row] (rows past R read as zero; never stored)
  bf16x8_t qb[kLseRB][KST];
#pragma unroll
  for (int r = 0; r < kLseRB; ++r) {
    const int rho = row0 + r * 16 + col;
    const bool ok = rho < R;
    const uint16_t* qrow = qt + ((size_t)g * R + (ok ? rho : 0)) * D + (D / 4) * grp;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      u32x4_t u = {0u, 0u, 0u, 0u};
      if (ok) u = *reinterpret_cast<const u32x4_t*>(qrow + 8 * kk);
      qb[r][kk] = as_bf16x8(u);
    }
  }
  LseState st;
#pragma unroll
  for (int r = 0; r < kLseRB; ++r) {
    st.m[r] = -INFINITY;
    st.l[r] = 0.0;
  }

  const uint16_t* khp = k + (size_t)g * geo.capacity * D;
  const int ntiles = (key1 - key0 + 63) / 64;
  const int last = key1 - 1;
  const LseMask mk{key1, R, geo.n_text, geo.text_start};
  const float c = geo.c;

  // Direct-to-LDS copies of tile tt of the chunk into buffer tt % NB, rows
  // clamped to the chunk's last key, K-swizzled (thread tid fills 16-byte
  // slots kLseThreads*u + tid; a slot's row and physical chunk give the
  // logical chunk through the self-inverse XOR swizzle).
  auto issue = [&](int tt) {
    uint16_t* buf = Kbuf + (tt & (NB - 1)) * TILE;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int slot = kLseThreads * u + tid;
      const int row = slot / CPR, phys = slot % CPR;
      const uint16_t* src =
          khp + (size_t)min(key0 + tt * 64 + row, last) * D + (Tile<D>::slot_k(row, phys) << 3);
      dma16(src, lds_addr(buf) + (kLseThreads * u + 64 * wave) * 16);
    }
  };

  // the Q operands land before any copy is issued (the empty asm takes them
  // as operands): the compiler does not count the copies, so a wait it
  // placed for these loads inside the loop would also wait for every copy
  // in flight
#pragma unroll
  for (int r = 0; r < kLseRB; ++r)
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) asm volatile("" : "+v"(qb[r][kk]));
  // Step t waits for its own copies of tile t (the NB - 2 newer tiles may
  // stay in flight); after the barrier every copy of tile t has landed and
  // every wave is done with the buffer of tile t - 1, which is refilled with
  // tile t + NB - 1.  A copy is issued at every step (tiles past the chunk
  // re-read its last key), so the count in flight is the same at every wait.
#pragma unroll
  for (int tt = 0; tt < NB - 1; ++tt) issue(tt);
  for (int t = 0; t < ntiles; ++t) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 2) * LPT));
    __syncthreads();
    issue(t + NB - 1);
    const uint16_t* Kt = Kbuf + (t & (NB - 1)) * TILE;
    const int t0 = key0 + t * 64;
    if (t0 + 64 <= mk.text_start && t0 + 64 <= mk.key1)
      lse_tile<D, false>(Kt, qb, t0, mk, row0, c, col, grp, st);
    else
      lse_tile<D, true>(Kt, qb, t0, mk, row0, c, col, grp, st);
  }
  // no copy may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // merge the four lane groups of each row (they saw different keys)
#pragma unroll
  for (int r = 0; r < kLseRB; ++r) {
    const float mm = max_over_groups(st.m[r]);
    double ll = (st.m[r] == -INFINITY) ? 0.0 : st.l[r] * exp2((double)st.m[r] - (double)mm);
    ll += __shfl_xor(ll, 16, kWave);
    ll += __shfl_xor(ll, 32, kWave);
    const int rho = row0 + r * 16 + col;
    if (grp == 0 && rho < R) {
      const size_t slot = (size_t)ch * geo.hq * geo.n_text + (size_t)g * R + rho;
      m_part[slot] = mm;
      l_part[slot] = ll;
    }
  }
}

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
// Step 2 (bf16, MFMA): column sums over the text rows of the group for
// kColsPerScoreWg visual keys.  S = Q K^T with rows on the M side and keys
// on the N side: each wave keeps kColKB blocks of 16 keys as MFMA operands
// in registers, and the workgroup streams the group's text-query rows and
// their normalisers through LDS in 64-row tiles by direct-to-LDS copies
// (kColBufs buffers, kColBufs - 1 tiles in flight, so the copies hide the
// L2 latency).  Each lane owns one key per block and sums its rows: fp32
// within a tile, fp64 across tiles, the four lanes of a key merged at the
// end in fp64.  Few registers per wave let four waves share each SIMD, so
// one wave's exponentials run while another's MFMAs do.
//
// The normalisers come from col_prep: per head group, scaled to base 2 and
// padded with +inf (probability 0) to whole tiles.
//
// The rows of a head group may be cut into n_split contiguous ranges of
// tiles (work item = KV head, row range, key block) so that the grid fills
// whole rounds of the machine; each range then writes fp64 partial sums and
// col_finalize adds the ranges in order.
constexpr int kColMaxSplit = 4;      // row ranges per head group, at most
constexpr int kColSlots = 256 * kColOcc;   // step-2 workgroups resident at once (256 CUs)

// lsep[g][rho] = factor * lse[g * R + rho] for rho < R, +inf up to R_pad.
__global__ void col_prep(const float* __restrict__ lse, float factor, int R, int R_pad, int n,
                         float* __restrict__ lsep) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int g = i / R_pad, rho = i % R_pad;
  lsep[i] = rho < R ? lse[(size_t)g * R + rho] * factor : INFINITY;
}

template <int D>
__global__ __launch_bounds__(kColThreads, kColOcc * kColWaves / 4) void colscore_mfma(
    const uint16_t* __restrict__ qt, const uint16_t* __restrict__ k, Geo geo,
    const float* __restrict__ lsep, int n_ct, int n_split, float* __restrict__ scores,
    double* __restrict__ part) {
  constexpr int KST = D / 32, CPR = D / 8, LPT = 64 * CPR / kColThreads;
  static_assert(LPT * kColThreads == 64 * CPR, "a tile is a whole number of copies per thread");
  constexpr int KB = kColKB, NB = kColBufs;
  constexpr int TILE = 64 * D;
  constexpr int OPS = LPT + 1;         // copies per thread and tile (rows + normalisers)
  __shared__ __align__(16) uint16_t Qs[NB * TILE];
  __shared__ __align__(16) float Ls[NB * 64];
  const int n_items = geo.hkv * n_split * n_ct;
  const int item = xcd_item(blockIdx.x, n_items);
  if (item >= n_items) return;
  const int ct = item % n_ct, sp = (item / n_ct) % n_split, g = item / (n_ct * n_split);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int R = geo.G * geo.n_text;
  const int n_rt = (R + 63) / 64;
  const int R_pad = n_rt * 64;
  const int rt0 = (int)((long)sp * n_rt / n_split), rt1 = (int)((long)(sp + 1) * n_rt / n_split);

  // key operands: B[k = d][n = key], key = base + kb*16 + col (clamped)
  bf16x8_t kbop[KB][KST];
  const uint16_t* kh = k + (size_t)g * geo.capacity * D;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = min(ct * kColsPerScoreWg + wave * 16 * KB + kb * 16 + col, geo.vis_len - 1);
    const uint16_t* krow = kh + (size_t)(geo.vis_start + j) * D + (D / 4) * grp;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      kbop[kb][kk] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(krow + 8 * kk));
  }
  double acc[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) acc[kb] = 0.0;

  const uint16_t* qg = qt + (size_t)g * R * D;
  const float* lg = lsep + (size_t)g * R_pad;
  const float c = geo.c;
  const int r0 = rt0 * 64;

  // Direct-to-LDS copies of tile tt of the range into buffer tt % NB:
  // rows clamped to R - 1, K-swizzled (thread tid fills 16-byte slots
  // kColThreads*u + tid; a slot's row and physical chunk give the logical
  // chunk through the self-inverse XOR swizzle), and the tile's 64
  // normalisers (every wave copies them, so all threads count the same
  // number of copies; tiles past the range re-read the last one).
  auto issue = [&](int tt) {
    const int buf = tt & (NB - 1);
    const int row0 = r0 + tt * 64;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int slot = kColThreads * u + tid;
      const int row = slot / CPR, phys = slot % CPR;
      const uint16_t* src =
          qg + (size_t)min(row0 + row, R - 1) * D + (Tile<D>::slot_k(row, phys) << 3);
      dma16(src, lds_addr(Qs + buf * TILE) + (kColThreads * u + 64 * wave) * 16);
    }
    dma4(lg + min(row0, R_pad - 64) + lane, lds_addr(Ls + buf * 64));
  };

  auto tile = [&](const uint16_t* Qt, const float* L) {
    float cs[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) cs[kb] = 0.f;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      u32x4_t a[KST];
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        a[kk] = *reinterpret_cast<const u32x4_t*>(Qt + Tile<D>::off_k(qb * 16 + col, KST * grp + kk));
      const floatx4_t lrow = *reinterpret_cast<const floatx4_t*>(L + qb * 16 + 4 * grp);
      floatx4_t sv[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        floatx4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) x = mfma_bf16(as_bf16x8(a[kk]), kbop[kb][kk], x);
        sv[kb] = x;
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[kb] += fast_exp2(fmaf(sv[kb][i], c, -lrow[i]));
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[kb] += (double)cs[kb];
  };

  // Step t waits for its own copies of tile t (the NB - 2 newer tiles may
  // stay in flight), then after the barrier -- all copies of tile t have
  // landed and every wave is done with the buffer of tile t - 1 -- refills
  // that buffer with tile t + NB - 1.  A copy is issued at every step, so
  // the count in flight is the same at every wait.
  const int ntiles = rt1 - rt0;
  // the key operands land before any copy is issued (the empty asm takes
  // them as operands, so their loads complete here and stay here): the
  // compiler does not count the copies, so a wait it placed for these loads
  // inside the loop would also wait for every copy in flight
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) asm volatile("" : "+v"(kbop[kb][kk]));
#pragma unroll
  for (int tt = 0; tt < NB - 1; ++tt) issue(tt);
  for (int t = 0; t < ntiles; ++t) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 2) * OPS));
    __syncthreads();
    issue(t + NB - 1);
    const int buf = t & (NB - 1);
    tile(Qs + buf * TILE, Ls + buf * 64);
  }
  // no copy may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  const double inv = 1.0 / ((double)geo.G * (double)geo.n_text);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    double a = acc[kb];
    a += __shfl_xor(a, 16, kWave);
    a += __shfl_xor(a, 32, kWave);
    const int j = ct * kColsPerScoreWg + wave * 16 * KB + kb * 16 + col;
    if (grp == 0 && j < geo.vis_len) {
      if (n_split == 1)
        scores[(size_t)g * geo.vis_len + j] = (float)(a * inv);
      else
        part[((size_t)sp * geo.hkv + g) * geo.vis_len + j] = a;
    }
  }
}

// Adds the n_split fp64 partial column sums of each key in range order.
__global__ void col_finalize(const double* __restrict__ part, int n_split, int n, double inv,
                             float* __restrict__ scores) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  double a = 0.0;
  for (int s = 0; s < n_split; ++s) a += part[(size_t)s * n + j];
  scores[j] = (float)(a * inv);
}

// Row ranges for step 2: the count with the least time, in units of one
// tile per workgroup, when the grid runs in rounds of kColSlots workgroups.
int col_splits(int n_items, int n_rt) {
  int best = 1;
  long best_cost = -1;
  for (int s = 1; s <= kColMaxSplit && s <= n_rt; ++s) {
    const long rounds = ((long)n_items * s + kColSlots - 1) / kColSlots;
    const long cost = rounds * ((n_rt + s - 1) / s);
    if (best_cost < 0 || cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
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
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkBatch = 8;      // loads issued together per thread

// Step 3: one 1024-thread workgroup per KV head.
//  * Radix select on the order-preserving bits of the (non-negative fp32)
//    scores, four 8-bit digits from the top: each pass histograms the digit
//    of the elements that match the prefix so far and keeps the digit that
//    contains the K-th largest.  Each wave counts into its own LDS
//    histogram, and since scores of one head share their top bits, a thread
//    adds runs of equal digits as one atomic.
//  * Stable compaction: wave w owns a contiguous range of positions; it
//    counts the elements above the threshold T and the copies of T, a block
//    scan turns the counts into output offsets (copies of T go to the lowest
//    positions first), and the wave writes its range in 64-element chunks
//    with a ballot prefix, so idx comes out in ascending position order.
__global__ __launch_bounds__(kTopkThreads) void radix_topk(const float* __restrict__ scores,
                                                           int vis_len, int vis_start, int topk,
                                                           int32_t* __restrict__ idx_out) {
  __shared__ unsigned whist[kTopkWaves][256];   // per-wave digit histograms
  __shared__ unsigned hist[256];
  __shared__ int wcount[2][kTopkWaves];
  __shared__ unsigned sh_prefix;
  __shared__ int sh_remaining;
  const int g = blockIdx.x;
  const unsigned* bits = reinterpret_cast<const unsigned*>(scores + (size_t)g * vis_len);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  unsigned prefix = 0, pmask = 0;
  int remaining = topk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    unsigned* wh = whist[wave];
    for (int b = lane; b < 256; b += 64) wh[b] = 0;
    __syncthreads();
    unsigned run_digit = 0, run_len = 0;
    for (int j0 = tid; j0 < vis_len; j0 += kTopkBatch * kTopkThreads) {
      // a batch of clamped loads first, so their latencies overlap
      unsigned v[kTopkBatch];
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u)
        v[u] = bits[min(j0 + u * kTopkThreads, vis_len - 1)];
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u) {
        if (j0 + u * kTopkThreads < vis_len && (v[u] & pmask) == prefix) {
          const unsigned d = (v[u] >> shift) & 255u;
          if (d != run_digit && run_len) {
            atomicAdd(&wh[run_digit], run_len);
            run_len = 0;
          }
          run_digit = d;
          ++run_len;
        }
      }
    }
    if (run_len) atomicAdd(&wh[run_digit], run_len);
    __syncthreads();
    if (tid < 256) {
      unsigned t = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) t += whist[w][tid];
      hist[tid] = t;
    }
    __syncthreads();
    if (tid < 64) {
      // the digit holding the remaining-th largest: lane l sums bins
      // 255-4l .. 252-4l, a wave suffix scan orders them from the top
      unsigned c4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) c4 += hist[255 - 4 * lane - i];
      unsigned incl = c4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
      }
      const unsigned excl = incl - c4;
      const bool here = excl < (unsigned)remaining && incl >= (unsigned)remaining;
      if (here) {
        unsigned cum = excl;
        int dgt = 255 - 4 * lane;
        for (int i = 0; i < 4; ++i) {
          const unsigned h = hist[255 - 4 * lane - i];
          if (cum + h >= (unsigned)remaining) { dgt = 255 - 4 * lane - i; break; }
          cum += h;
        }
        sh_prefix = prefix | ((unsigned)dgt << shift);
        sh_remaining = remaining - (int)cum;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const unsigned T = prefix;
  const int need_eq = remaining;  // copies of T to keep, >= 1

  // per-wave counts over contiguous ranges of whole 64-element chunks
  const int chunks = (vis_len + 63) / 64;
  const int per_wave = (chunks + kTopkWaves - 1) / kTopkWaves;
  const int c0 = wave * per_wave, c1 = min(chunks, c0 + per_wave);
  int n_gt = 0, n_eq = 0;
  for (int cb = c0; cb < c1; cb += kTopkBatch) {
    unsigned v[kTopkBatch];
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) v[u] = bits[min((cb + u) * 64 + lane, vis_len - 1)];
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) {
      const bool valid = cb + u < c1 && (cb + u) * 64 + lane < vis_len;
      n_gt += __popcll(__ballot(valid && v[u] > T));
      n_eq += __popcll(__ballot(valid && v[u] == T));
    }
  }
  if (lane == 0) {
    wcount[0][wave] = n_gt;
    wcount[1][wave] = n_eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += wcount[0][w];
    eq_before += wcount[1][w];
  }
  // copies of T taken before this wave's range, and by it
  const int eq_take_before = min(eq_before, need_eq);
  int out = gt_before + eq_take_before;
  int eq_seen = eq_before;
  const unsigned long long lower = (1ull << lane) - 1ull;
  for (int cb = c0; cb < c1; cb += kTopkBatch) {
    unsigned v[kTopkBatch];
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) v[u] = bits[min((cb + u) * 64 + lane, vis_len - 1)];
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) {
      const int j = (cb + u) * 64 + lane;
      const bool valid = cb + u < c1 && j < vis_len;
      const bool is_eq = valid && v[u] == T;
      const unsigned long long eq_mask = __ballot(is_eq);
      const int eq_rank = eq_seen + __popcll(eq_mask & lower);   // copies of T before j
      const bool take = (valid && v[u] > T) || (is_eq && eq_rank < need_eq);
      const unsigned long long take_mask = __ballot(take);
      if (take) idx_out[(size_t)g * topk + out + __popcll(take_mask & lower)] = vis_start + j;
      out += __popcll(take_mask);
      eq_seen += __popcll(eq_mask);
    }
  }
}

template <int D>
hipError_t launch_mfma_select(const SelectArgs& a, const Geo& geo, float* lse2, float* m_part,
                              double* l_part, double* col_part, float* lsep, hipStream_t st) {
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
    const int n_rb = (R + kLseRowsWg - 1) / kLseRowsWg;
    const int n_items = a.hkv * n_chunks * n_rb;
    const int grid = ((n_items + kXcds - 1) / kXcds) * kXcds;
    lse_partial_mfma<D><<<grid, kLseThreads, 0, st>>>(qt, k, geo, n_chunks, n_rb, m_part, l_part);
    const int rows = a.hq * a.n_text;
    lse_finalize<<<(rows + 255) / 256, 256, 0, st>>>(m_part, l_part, n_chunks, rows, lse2);
  }
  const int n_ct = (a.vis_len + kColsPerScoreWg - 1) / kColsPerScoreWg;
  const int R = geo.G * a.n_text;
  const int n_rt = (R + 63) / 64;
  const int n_split = col_splits(a.hkv * n_ct, n_rt);
  const int n_items = a.hkv * n_ct * n_split;
  const int grid = ((n_items + kXcds - 1) / kXcds) * kXcds;
  const int n_lsep = a.hkv * n_rt * 64;
  col_prep<<<(n_lsep + 255) / 256, 256, 0, st>>>(lse, factor, R, n_rt * 64, n_lsep, lsep);
  colscore_mfma<D><<<grid, kColThreads, 0, st>>>(qt, k, geo, lsep, n_ct, n_split, a.scores_out,
                                                 col_part);
  if (n_split > 1) {
    const int n = a.hkv * a.vis_len;
    col_finalize<<<(n + 255) / 256, 256, 0, st>>>(col_part, n_split, n,
                                                   1.0 / ((double)geo.G * (double)a.n_text),
                                                   a.scores_out);
  }
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
  size_t lse2, m_part, l_part, col_part, lsep, scores, total;
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
  L.col_part = off;
  off += align256((size_t)kColMaxSplit * hkv * vis_len * sizeof(double));
  L.lsep = off;
  off += align256((size_t)hkv * (((size_t)(hq / hkv) * n_text + 63) / 64) * 64 * sizeof(float));
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
  double* col_part = reinterpret_cast<double*>(ws + L.col_part);
  float* lsep = reinterpret_cast<float*>(ws + L.lsep);
  if (!a.scores_out) a.scores_out = reinterpret_cast<float*>(ws + L.scores);
  Geo geo{a.hq, a.hkv, a.hq / a.hkv, a.d, a.capacity, a.text_start, a.n_text,
          a.vis_start, a.vis_len, a.scale * kLog2e};
  hipError_t err;
  if (a.bf16)
    err = a.d == 128 ? launch_mfma_select<128>(a, geo, lse2, m_part, l_part, col_part, lsep, st)
                     : launch_mfma_select<64>(a, geo, lse2, m_part, l_part, col_part, lsep, st);
  else
    err = a.d == 128 ? launch_valu_select<float, 128>(a, geo, lse2, st)
                     : launch_valu_select<float, 64>(a, geo, lse2, st);
  if (err != hipSuccess) return err;
  radix_topk<<<a.hkv, kTopkThreads, 0, st>>>(a.scores_out, a.vis_len, a.vis_start, a.topk,
                                             a.idx_out);
  return hipGetLastError();
}

}  // namespace stdspec
