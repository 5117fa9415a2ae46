// Prefill attention of the text rows, with their softmax normalisers (gfx950).
//
// The selection's first step needs, for every text row, the log of its
// causal softmax denominator (technical summary, Methodology item 4: the
// top-K come from the text rows' attention to the visual tokens).  The
// prefill computes the same rows' attention anyway; this call does both at
// once: out = softmax(q K^T scale) V over keys [0, text_start + i] for text
// row i, and lse = log of that softmax's denominator, which the selection
// call accepts in place of computing it.
//
//  prefill_mfma_kernel -- one workgroup = 8 waves x 32 rows = 256 rows of
//      one KV head group (the G heads' rows stacked, as the selection
//      kernels lay them out) against one chunk of kPfChunk keys, two waves
//      per SIMD.  Each wave holds two 16-row blocks, so every K and V
//      fragment it reads from LDS feeds two MFMAs (LDS reads are half of
//      what one block per wave at four waves per SIMD needs; that form ran
//      9 % slower).  Q stays in registers; K and V tiles of 64 keys move
//      global -> LDS by direct-to-LDS copies (four buffers, three tiles in
//      flight).  Per tile: S^T = K Q^T on the matrix unit, P = 2^(s c - m)
//      against the row's lazy running max (shared by the row's four lanes;
//      it moves only when a score passes it by 2^8, found from the P sums,
//      so the per-score max is off the common path), O^T += V^T P^T on the
//      matrix unit with V^T taken by transpose reads.  The chunk's (m, l, O)
//      per row go to the workspace.
//  prefill_merge -- one wave per row: merges the chunks into O (bf16) and
//      the natural-log normaliser.

#include "common.hpp"
#include "internal.hpp"
#include "prefill.hpp"
#include "tile.hpp"

namespace stdspec {
namespace {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRB = 2;                                  // 16-row blocks per wave
constexpr int kPfRowsWg = kPfWaves * 16 * kPfRB;          // rows per workgroup
constexpr int kPfOcc = kPfWaves / 4;                      // waves per SIMD
constexpr int kPfBufs = 4;                                // tile buffers (a power of two)
constexpr int kPfXcds = 8;

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to one dword of two bf16 (round to nearest even), one
// conversion for the pair.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_t));
}

// Consecutive items (the row blocks of one KV head and key chunk) go to the
// same XCD, so the K and V tiles they share are fetched into one L2.
__device__ __forceinline__ int pf_item(int bid, int n_items) {
  const int per = (n_items + kPfXcds - 1) / kPfXcds;
  return (bid % kPfXcds) * per + bid / kPfXcds;
}

// S^T = K Q^T for one 64-key tile: s[r][kb] holds keys 16 kb + 4 grp + i
// of the tile for row col of block r.  The K fragments of two key blocks
// are read before their MFMAs.
template <int D>
__device__ __forceinline__ void pf_scores(const uint16_t* Ks, const bf16x8_t (*qb)[D / 32],
                                          int col, int grp, floatx4_t (&s)[kPfRB][4]) {
  constexpr int KST = D / 32;
#pragma unroll
  for (int kp = 0; kp < 4; kp += 2) {
    u32x4_t a[2][KST];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        a[b2][kk] = *reinterpret_cast<const u32x4_t*>(
            Ks + Tile<D>::off_k((kp + b2) * 16 + col, KST * grp + kk));
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < kPfRB; ++r) s[r][kp + b2] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int r = 0; r < kPfRB; ++r)
          s[r][kp + b2] = mfma_bf16(as_bf16x8(a[b2][kk]), qb[r][kk], s[r][kp + b2]);
  }
}

// The same scores with one key block's K fragments in registers at a time
// (fewer registers, for the rare slow path).
template <int D>
__device__ __forceinline__ void pf_scores_lean(const uint16_t* Ks, const bf16x8_t (*qb)[D / 32],
                                               int col, int grp, floatx4_t (&s)[kPfRB][4]) {
  constexpr int KST = D / 32;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int r = 0; r < kPfRB; ++r) s[r][kb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
          Ks + Tile<D>::off_k(kb * 16 + col, KST * grp + kk));
#pragma unroll
      for (int r = 0; r < kPfRB; ++r) s[r][kb] = mfma_bf16(as_bf16x8(a), qb[r][kk], s[r][kb]);
    }
    // keeps the scheduler from hoisting every block's fragment reads
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Keys at or past the chunk end, or after the row's own position, score
// -inf (selects only: the compares are per lane).
__device__ __forceinline__ void pf_mask(floatx4_t (&s)[kPfRB][4], int t0, int grp, int key1,
                                        const int (&rpos)[kPfRB]) {
#pragma unroll
  for (int r = 0; r < kPfRB; ++r)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t0 + kb * 16 + 4 * grp + i;
        const bool vis = (key < key1) & (key <= rpos[r]);
        s[r][kb][i] = vis ? s[r][kb][i] : -INFINITY;
      }
}

template <int D>
__global__ __launch_bounds__(kPfThreads, kPfOcc) void prefill_mfma_kernel(
    const uint16_t* __restrict__ qt, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int hq, int hkv, int capacity, int text_start, int n_text,
    float c, int n_chunks, int n_rb, float* __restrict__ m_part, double* __restrict__ l_part,
    float* __restrict__ o_part) {
  constexpr int KST = D / 32, DB = D / 16, CPR = D / 8;
  constexpr int TILE = 64 * D;
  // 16-byte copies per tensor and tile; with fewer copies than threads the
  // first COPIES threads (whole waves) issue one each
  constexpr int COPIES = 64 * CPR;
  constexpr int LPT = COPIES >= kPfThreads ? COPIES / kPfThreads : 1;
  static_assert(COPIES % kPfThreads == 0 || kPfThreads % COPIES == 0, "copies per thread");
  static_assert(COPIES % 64 == 0, "copying threads form whole waves");
  constexpr int NB = kPfBufs;
  __shared__ __align__(16) uint16_t smem[NB * 2 * TILE];   // [buffer][K, V]

  const int G = hq / hkv, R = G * n_text;
  const int n_items = hkv * n_chunks * n_rb;
  const int item = pf_item(blockIdx.x, n_items);
  if (item >= n_items) return;
  const int rb = item % n_rb;
  const int ch = (item / n_rb) % n_chunks;
  const int g = item / (n_rb * n_chunks);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_keys = text_start + n_text;
  const int key0 = ch * kPfChunk, key1 = min(n_keys, key0 + kPfChunk);
  const int last = key1 - 1;
  const int row0 = rb * kPfRowsWg + wave * 16 * kPfRB;     // first row of the wave

  // this lane's row (column col) of each row block and its position; rows
  // past R read row 0's query and are never stored
  int rpos[kPfRB];
  bf16x8_t qb[kPfRB][KST];
#pragma unroll
  for (int r = 0; r < kPfRB; ++r) {
    const int rho = row0 + r * 16 + col;
    const bool ok = rho < R;
    rpos[r] = text_start + (ok ? rho % n_text : 0);
    const uint16_t* qrow = qt + ((size_t)g * R + (ok ? rho : 0)) * D + (D / 4) * grp;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      qb[r][kk] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qrow + 8 * kk));
  }

  const uint16_t* kh = k + (size_t)g * capacity * D;
  const uint16_t* vh = v + (size_t)g * capacity * D;
  // Tile tt of the chunk into buffer tt % NB, K and V swizzled as in Tile<D>
  // (thread tid fills 16-byte slots kPfThreads*u + tid); rows past the
  // chunk re-read its last key.
  auto issue = [&](int tt) {
    if (COPIES < kPfThreads && tid >= COPIES) return;          // wave-uniform
    uint16_t* kb = smem + (tt & (NB - 1)) * 2 * TILE;
    uint16_t* vb = kb + TILE;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int slot = kPfThreads * u + tid;
      const int row = slot / CPR, phys = slot % CPR;
      const size_t base = (size_t)min(key0 + tt * 64 + row, last) * D;
      const uint32_t dst = (kPfThreads * u + 64 * wave) * 16;
      dma16(kh + base + (Tile<D>::slot_k(row, phys) << 3), lds_addr(kb) + dst);
      dma16(vh + base + (Tile<D>::slot_v(row, phys) << 3), lds_addr(vb) + dst);
    }
  };
  // the Q operands land before any copy is issued (the compiler does not
  // count the copies, so a wait it placed for these loads inside the loop
  // would also wait for every copy in flight)
#pragma unroll
  for (int r = 0; r < kPfRB; ++r)
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) asm volatile("" : "+v"(qb[r][kk]));

  float m[kPfRB];
  double l[kPfRB];
  floatx4_t oacc[kPfRB][DB];
#pragma unroll
  for (int r = 0; r < kPfRB; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[r][db] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Step t: wait for tile t's copies (tiles t+1, t+2 may stay in flight),
  // barrier (every wave is also done with the buffer of tile t-1), refill
  // that buffer with tile t+3, reduce tile t.  A copy is issued at every
  // step, so the count in flight is the same at every wait.
  constexpr int kInFlight = 2 * (NB - 2) * LPT;
  const int ntiles = (key1 - key0 + 63) / 64;
  const int r4 = col >> 2, rc = col & 3;
#pragma unroll
  for (int tt = 0; tt < NB - 1; ++tt) issue(tt);
  for (int t = 0; t < ntiles; ++t) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInFlight));
    __syncthreads();
    issue(t + NB - 1);
    const uint16_t* Ks = smem + (t & (NB - 1)) * 2 * TILE;
    const uint16_t* Vs = Ks + TILE;
    const int t0 = key0 + t * 64;
    // keys at or before text_start are visible to every text row (wave-uniform)
    const bool interior = t0 + 64 <= key1 && t0 + 63 <= text_start;

    // Fast path: the probabilities against the running max as it stands,
    // P = 2^(s c - m), computed in place of the scores.  While no score of
    // the tile exceeds the max by 2^8 each P is at most 2^8, so a lane sum
    // above 2^8 (or NaN / inf: the max is still unset) flags a row whose max
    // may have to move; then the whole wave (the MFMAs cover every lane)
    // recomputes the tile's scores and applies the max rule row by row.
    // Rows whose max stays get the same P either way.
    floatx4_t sp[kPfRB][4];
    pf_scores<D>(Ks, qb, col, grp, sp);
    if (!interior) pf_mask(sp, t0, grp, key1, rpos);
    float ts[kPfRB];
    bool ok = true;
#pragma unroll
    for (int r = 0; r < kPfRB; ++r) {
      ts[r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sp[r][kb][i] = fast_exp2(fmaf(sp[r][kb][i], c, -m[r]));
          ts[r] += sp[r][kb][i];
        }
      ok = ok && ts[r] <= 256.f;
    }
    if (__any(!ok)) {                     // wave-uniform; the first tile of a chunk, then rare
      pf_scores_lean<D>(Ks, qb, col, grp, sp);
      if (!interior) pf_mask(sp, t0, grp, key1, rpos);
#pragma unroll
      for (int r = 0; r < kPfRB; ++r) {
        // the row's max on the raw scores (c > 0; the row's four lanes agree)
        float tmax = sp[r][0][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sp[r][kb][i]);
        tmax = max_over_groups(tmax) * c;
        if (tmax > m[r] + 8.f) {          // also while m = -inf
          const float alpha = (m[r] == -INFINITY) ? 0.f : fast_exp2(m[r] - tmax);
          l[r] *= (double)alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[r][db] *= alpha;
          m[r] = tmax;
        }
        const float nms = (m[r] == -INFINITY) ? 0.f : -m[r];
        ts[r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sp[r][kb][i] = fast_exp2(fmaf(sp[r][kb][i], c, nms));
            ts[r] += sp[r][kb][i];
          }
      }
    }
    uint32_t pw[kPfRB][8];
#pragma unroll
    for (int r = 0; r < kPfRB; ++r) {
      l[r] += (double)ts[r];
#pragma unroll
      for (int w = 0; w < 8; ++w)
        pw[r][w] = pack2_bf16(sp[r][w >> 1][2 * (w & 1)], sp[r][w >> 1][2 * (w & 1) + 1]);
    }

    // O^T += V^T P^T in two 32-key steps.  The B operand holds the lane's
    // own probabilities (keys 32 ks + 4 grp + j, then 32 ks + 16 + 4 grp +
    // j) and the transpose reads of V follow the same key order; every V^T
    // fragment of a step is read before its MFMAs, and each serves all the
    // wave's row blocks.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int vrow = 32 * ks + 4 * grp + r4;
      uint4 va[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int chunk = 2 * db + (rc >> 1);
        const int e = 4 * (rc & 1);
        const uint2 lo = lds_read_tr16(Vs + Tile<D>::off_v(vrow, chunk) + e);
        const uint2 hi = lds_read_tr16(Vs + Tile<D>::off_v(vrow + 16, chunk) + e);
        va[db] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
#pragma unroll
      for (int r = 0; r < kPfRB; ++r) {
        const bf16x8_t pb = as_bf16x8(make_uint4(pw[r][4 * ks + 0], pw[r][4 * ks + 1],
                                                 pw[r][4 * ks + 2], pw[r][4 * ks + 3]));
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[r][db] = mfma_bf16(as_bf16x8(va[db]), pb, oacc[r][db]);
      }
    }
  }
  // no copy may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // the chunk's partial per row: m (shared), l summed over the row's lanes,
  // O^T[d][row] with d = 16 db + 4 grp + i held by lane (col, grp)
#pragma unroll
  for (int r = 0; r < kPfRB; ++r) {
    double ll = l[r];
    ll += __shfl_xor(ll, 16, kWave);
    ll += __shfl_xor(ll, 32, kWave);
    const int rho = row0 + r * 16 + col;
    if (rho >= R) continue;
    const size_t slot = (size_t)ch * hq * n_text + (size_t)g * R + rho;
    if (grp == 0) {
      m_part[slot] = m[r];
      l_part[slot] = ll;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<floatx4_t*>(o_part + slot * D + db * 16 + 4 * grp) = oacc[r][db];
  }
}

// One wave per row (row = g * R + rho of the stacked layout): out and lse
// take the head-major layout of q_text, [H_q][n_text][d] and [H_q][n_text].
template <int D>
__global__ __launch_bounds__(256) void prefill_merge(const float* __restrict__ m_part,
                                                     const double* __restrict__ l_part,
                                                     const float* __restrict__ o_part,
                                                     int n_chunks, int rows,
                                                     uint16_t* __restrict__ out,
                                                     float* __restrict__ lse) {
  constexpr int PL = D / 64;                      // output elements per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float M = -INFINITY;
  for (int cc = 0; cc < n_chunks; ++cc) M = fmaxf(M, m_part[(size_t)cc * rows + row]);
  double L = 0.0;
  float acc[PL];
#pragma unroll
  for (int u = 0; u < PL; ++u) acc[u] = 0.f;
  for (int cc = 0; cc < n_chunks; ++cc) {
    const size_t slot = (size_t)cc * rows + row;
    const float mc = m_part[slot];
    if (mc == -INFINITY) continue;                 // no key of this chunk is visible
    const float w = fast_exp2(mc - M);
    L += l_part[slot] * (double)w;
#pragma unroll
    for (int u = 0; u < PL; ++u) acc[u] = fmaf(o_part[slot * D + lane + 64 * u], w, acc[u]);
  }
  const float inv = (float)(1.0 / L);
#pragma unroll
  for (int u = 0; u < PL; ++u) Elem<uint16_t>::store(out, (size_t)row * D + lane + 64 * u, acc[u] * inv);
  // natural log of the denominator: scores were in base-2 units (x = s c)
  if (lse && lane == 0) lse[row] = (float)(((double)M + log2(L)) * 0.6931471805599453);
}

}  // namespace

size_t prefill_workspace_bytes(int hq, int d, int text_start, int n_text) {
  const size_t rows = (size_t)hq * n_text;
  const size_t n_chunks = ((size_t)text_start + n_text + kPfChunk - 1) / kPfChunk;
  return align256(n_chunks * rows * sizeof(float)) + align256(n_chunks * rows * sizeof(double)) +
         align256(n_chunks * rows * d * sizeof(float));
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const size_t rows = (size_t)a.hq * a.n_text;
  const int n_chunks = (a.text_start + a.n_text + kPfChunk - 1) / kPfChunk;
  char* ws = static_cast<char*>(a.ws);
  float* m_part = reinterpret_cast<float*>(ws);
  ws += align256((size_t)n_chunks * rows * sizeof(float));
  double* l_part = reinterpret_cast<double*>(ws);
  ws += align256((size_t)n_chunks * rows * sizeof(double));
  float* o_part = reinterpret_cast<float*>(ws);
  const int G = a.hq / a.hkv;
  const int n_rb = (G * a.n_text + kPfRowsWg - 1) / kPfRowsWg;
  const int n_items = a.hkv * n_chunks * n_rb;
  const int grid = ((n_items + kPfXcds - 1) / kPfXcds) * kPfXcds;
  const float c = a.scale * kLog2e;
  const auto* q = static_cast<const uint16_t*>(a.q_text);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  auto* out = static_cast<uint16_t*>(a.out);
  const int mgrid = (int)((rows + 3) / 4);
  if (a.d == 128) {
    prefill_mfma_kernel<128><<<grid, kPfThreads, 0, st>>>(q, k, v, a.hq, a.hkv, a.capacity,
                                                         a.text_start, a.n_text, c, n_chunks,
                                                         n_rb, m_part, l_part, o_part);
    prefill_merge<128><<<mgrid, 256, 0, st>>>(m_part, l_part, o_part, n_chunks, (int)rows, out,
                                               a.lse_out);
  } else {
    prefill_mfma_kernel<64><<<grid, kPfThreads, 0, st>>>(q, k, v, a.hq, a.hkv, a.capacity,
                                                        a.text_start, a.n_text, c, n_chunks,
                                                        n_rb, m_part, l_part, o_part);
    prefill_merge<64><<<mgrid, 256, 0, st>>>(m_part, l_part, o_part, n_chunks, (int)rows, out,
                                              a.lse_out);
  }
  return hipGetLastError();
}

}  // namespace stdspec
