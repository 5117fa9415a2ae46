// Split-K attention kernels of the StD hot path (gfx950, wave64).
//
//  * dense_mfma_kernel  -- the dense model's verify pass (technical summary,
//    Methodology items 2-3: the dense model checks the gamma drafts in one
//    pass over the full KV cache).  One workgroup streams its share of one
//    KV head's tiles ONCE for every query row of that head's GQA group (up
//    to 64 of the n_q*G rows per workgroup), so each K/V byte is read from
//    HBM once per call when n_q*G <= 64.
//  * sparse_mfma_kernel -- the sparse model's draft step (Methodology item 2:
//    top-K attention over the visual KV chosen at prefill).  One wave
//    gathers 64 entries of the head's key list (prefix + selected visual
//    positions + tail) into LDS and reduces them for the G query heads.
//  * attn_valu_kernel   -- the same two operations on the vector ALU for
//    fp32 caches (and any shape the MFMA kernels do not take).
//  * combine_kernel     -- merges the per-split (max, sum, output) partials
//    with log-sum-exp rescaling (flash-decoding style reduction pass).
//
// MFMA formulation (v_mfma_f32_16x16x32_bf16): scores are computed
// transposed, S^T = K Q^T, keys on the M side (16 per block) and query rows
// on the N side (16 per wave).  The 16x16 accumulator leaves each lane with
// four consecutive keys of one query column, which are exactly the eight
// bf16 values the lane must supply as the B operand of O^T = V^T P^T for a
// 32-key step; no shuffle is needed between the two products.  Both
// products contract over a permuted index (d, then keys) that is applied
// identically to both operands, so the sums are unchanged.  V^T for the A
// operand is read from the row-major V tile in LDS with the gfx950
// transpose read (ds_read_b64_tr_b16), so V is staged without reshuffling.
// Softmax runs in base 2 with the scale folded into one multiply.

#include "common.hpp"
#include "internal.hpp"
#include "tile.hpp"

namespace stdspec {
namespace {

// Entry e of the key list of one KV head -> cache position.
// A selected position outside the visual span is clamped into it: the
// result for such a list is unspecified, but no access leaves the cache.
struct KeyList {
  bool sparse;
  const int32_t* idx;   // this head's selected positions (sparse only)
  int vis_start, vis_end, topk;
  __device__ __forceinline__ int pos(int e) const {
    if (!sparse || e < vis_start) return e;
    const int t = e - vis_start;
    return t < topk ? min(max(idx[t], vis_start), vis_end - 1) : vis_end + (t - topk);
  }
};

// Valid cache length of a call: the host value, or (device-length calls)
// min(max(*dev + off, lo), max) read when the kernel runs, so a decode loop
// captured once in a graph sees the length the previous step committed.
// lo is the shortest length the call is defined for (dense: n_q, so every
// query row sees at least one key; sparse: the end of the visual span, or
// one past it when the key list would otherwise be empty); the host checks
// lo <= max.  ptr() never is null (a zero word stands in for a missing
// device length), so a kernel can load it as a vector load issued with its
// first memory accesses and apply resolve() where the length is first needed.
__device__ int32_t kNoDeviceLen = 0;
struct LenSrc {
  int max;
  const int32_t* dev;
  int off;
  int lo;
  __device__ __forceinline__ int get() const { return dev ? min(max_(*dev + off, lo), max) : max; }
  __device__ __forceinline__ const int32_t* ptr() const { return dev ? dev : &kNoDeviceLen; }
  __device__ __forceinline__ int resolve(int d) const {
    return dev ? min(max_(d + off, lo), max) : max;
  }
  static __device__ __forceinline__ int max_(int a, int b) { return a > b ? a : b; }
};

// One tile of 16*NKB keys (NKB = 1, 2 or 4 key blocks) for one wave's 16
// query columns.
template <int D, int NKB>
struct TileMath {
  static constexpr int KST = D / 32;   // 32-wide contraction steps over d
  static constexpr int DB = D / 16;    // 16-wide output blocks over d

  // S^T = K Q^T for the NKB key blocks: lane (col, grp) gets keys
  // kb*16 + 4*grp + i of query column col.
  static __device__ __forceinline__ void scores(const uint16_t* Ks, const bf16x8_t* qb,
                                                int col, int grp, floatx4_t* sacc) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) {
        const uint4 a = *reinterpret_cast<const uint4*>(
            Ks + Tile<D>::off_k(kb * 16 + col, KST * grp + kk));
        acc = mfma_bf16(as_bf16x8(a), qb[kk], acc);
      }
      sacc[kb] = acc;
    }
  }

  // O^T += V^T P^T over the tile's keys in 32-key steps.  The B operand
  // holds the lane's own probabilities (keys 32ks + 4grp + j and
  // 32ks + 16 + 4grp + j); the A operand (V^T, lane = d row) is read from the
  // row-major V tile with two transpose reads whose per-lane row addresses
  // follow the same key order.  With a single key block the upper 16 keys
  // of the step are absent: their operand halves are zero.
  static __device__ __forceinline__ void pv(const uint16_t* Vs, const float* p, int col,
                                            int grp, floatx4_t* oacc) {
    const int r4 = col >> 2, rc = col & 3;
    constexpr int NKS = NKB >= 2 ? NKB / 2 : 1;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 pw;
      pw.x = pack_bf16x2(p[(2 * ks) * 4 + 0], p[(2 * ks) * 4 + 1]);
      pw.y = pack_bf16x2(p[(2 * ks) * 4 + 2], p[(2 * ks) * 4 + 3]);
      if constexpr (NKB >= 2) {
        pw.z = pack_bf16x2(p[(2 * ks + 1) * 4 + 0], p[(2 * ks + 1) * 4 + 1]);
        pw.w = pack_bf16x2(p[(2 * ks + 1) * 4 + 2], p[(2 * ks + 1) * 4 + 3]);
      } else {
        pw.z = 0u;
        pw.w = 0u;
      }
      const bf16x8_t pb = as_bf16x8(pw);
      const int row0 = 32 * ks + 4 * grp + r4;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int chunk = 2 * db + (rc >> 1);
        const int e = 4 * (rc & 1);
        const uint2 lo = lds_read_tr16(Vs + Tile<D>::off_v(row0, chunk) + e);
        uint2 hi = make_uint2(0u, 0u);
        if constexpr (NKB >= 2) hi = lds_read_tr16(Vs + Tile<D>::off_v(row0 + 16, chunk) + e);
        oacc[db] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, oacc[db]);
      }
    }
  }
};

// Online softmax for one tile: x holds NJ base-2 scores (-inf when masked).
// The running max m of a column moves only when a score exceeds it by more
// than 2^8 (or m is unset); probabilities are taken relative to m, so they
// stay below 256 and the accumulator rescale (AGPR round trips) is skipped
// on almost every tile.  Exact: m is only a shift of the exponent.
constexpr float kLazyMax = 8.f;

template <int DB, int NJ>
__device__ __forceinline__ void online_update(const float* x, float* p, float& m, float& lsum,
                                              floatx4_t* oacc) {
  float tmax = x[0];
#pragma unroll
  for (int j = 1; j < NJ; ++j) tmax = fmaxf(tmax, x[j]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  if (tmax > m + kLazyMax) {            // also taken while m is still -inf
    const float alpha = fast_exp2(m - tmax);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    m = tmax;
  }
  const float msafe = (m == -INFINITY) ? 0.f : m;
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    p[j] = fast_exp2(x[j] - msafe);
    psum += p[j];
  }
  lsum += psum;
}

template <int D>
__device__ __forceinline__ void load_q_operand(const uint16_t* qrow, bool ok, int grp,
                                               bf16x8_t* qb) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (ok) u = *reinterpret_cast<const uint4*>(qrow + (D / 4) * grp + 8 * kk);
    qb[kk] = as_bf16x8(u);
  }
}

// ---------------------------------------------------------------------------
// Dense verify: grid (split, KV head, 64-row block), 512 threads = 8 waves,
// at most one workgroup per CU.
//
// The len keys form ceil(len/64) tiles of 64; split s takes tiles s,
// s + S, s + 2S, ... (S splits, a function of len and H_kv only), so at any
// moment the workgroups of a head sweep one contiguous region of the cache.
// K and V tiles move global -> LDS by direct-to-LDS copies (no staging
// registers, non-temporal: each byte is read once per call) into three
// buffers, two tiles in flight.  Wave w reduces key
// half w & 1 of every tile for the 16 query rows of block w >> 1; the two
// key halves are merged in LDS at the end.  Every K/V byte is read from HBM
// once per call when n_q * G <= 64.
constexpr int kDenseThreads = 512;
constexpr int kDenseBufs = 3;

// Copy one 64-key tile of K and V (rows past the end re-read row len - 1)
// into the swizzled LDS layout of Tile<D>.  Thread tid fills 16-byte slots
// 512u + tid of each tensor; a slot's row and physical chunk give the
// logical chunk by the (self-inverse) XOR swizzle.
template <int D, int NT>
__device__ __forceinline__ void dense_issue_tile(uint16_t* ks, uint16_t* vs, const uint16_t* kh,
                                                 const uint16_t* vh, int t0, int len, int tid,
                                                 int wave) {
  constexpr int CPR = D / 8;
  constexpr int LPT = 64 * CPR / NT;
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int slot = NT * u + tid;
    const int row = slot / CPR, phys = slot % CPR;
    const size_t base = (size_t)min(t0 + row, len - 1) * D;
    const uint32_t dst = (NT * u + 64 * wave) * 16;
    dma16_stream(kh + base + (Tile<D>::slot_k(row, phys) << 3), lds_addr(ks) + dst);
    dma16_stream(vh + base + (Tile<D>::slot_v(row, phys) << 3), lds_addr(vs) + dst);
  }
}

// One wave's share of a 64-key tile: the 32 keys of key half kh (key
// blocks 2kh, 2kh+1) against the wave's 16 query rows.
template <int D>
__device__ __forceinline__ void dense_step(const uint16_t* Ks, const uint16_t* Vs,
                                           const bf16x8_t* qb, int kh, int t0, int len,
                                           int safe_end, int qpos, float c, int col, int grp,
                                           bool rok, float& m, float& lsum, floatx4_t* oacc) {
  constexpr int KST = D / 32;
  constexpr int DB = D / 16;
  floatx4_t sacc[2];
#pragma unroll
  for (int kbi = 0; kbi < 2; ++kbi) {
    const int row = (2 * kh + kbi) * 16 + col;
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      const uint4 a = *reinterpret_cast<const uint4*>(Ks + Tile<D>::off_k(row, KST * grp + kk));
      acc = mfma_bf16(as_bf16x8(a), qb[kk], acc);
    }
    sacc[kbi] = acc;
  }
  float x[8];
  const bool interior = t0 + 64 <= safe_end;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float sv = sacc[j >> 2][j & 3] * c;
    if (interior) {
      x[j] = sv;
    } else {
      const int key = t0 + (2 * kh + (j >> 2)) * 16 + 4 * grp + (j & 3);
      x[j] = (key < len && key <= qpos) ? sv : -INFINITY;
    }
  }
  float tmax = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, x[j]);
  tmax = max_over_groups(tmax);
  if (tmax > m + kLazyMax) {              // rare: see online_update
    const float alpha = fast_exp2(m - tmax);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    m = tmax;
  }
  const float msafe = (m == -INFINITY) ? 0.f : m;
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = fast_exp2(x[j] - msafe);
  lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  // padding rows (never stored) feed zeros to the matrix unit: an MFMA on
  // zero operands draws less power, and this kernel runs at the power limit
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = rok ? p[j] : 0.f;
  // O^T += V^T P^T over the 32 keys (one MFMA step per 16 output columns)
  uint4 pw;
  pw.x = pack_bf16x2(p[0], p[1]);
  pw.y = pack_bf16x2(p[2], p[3]);
  pw.z = pack_bf16x2(p[4], p[5]);
  pw.w = pack_bf16x2(p[6], p[7]);
  const bf16x8_t pb = as_bf16x8(pw);
  const int r4 = col >> 2, rc = col & 3;
  const int row0 = 32 * kh + 4 * grp + r4;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 2 * db + (rc >> 1);
    const int e = 4 * (rc & 1);
    const uint2 lo = lds_read_tr16(Vs + Tile<D>::off_v(row0, chunk) + e);
    const uint2 hi = lds_read_tr16(Vs + Tile<D>::off_v(row0 + 16, chunk) + e);
    oacc[db] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, oacc[db]);
  }
}

// W = 1: 512 threads, 64 query rows per workgroup; W = 2 (head_dim 128 with
// more than 64 rows in a group, e.g. gamma + 1 >= 10 queries of a 7-head
// group): 1,024 threads and 128 rows, so each K/V tile is still read once
// for all of them (at head_dim 64 such groups keep 64-row blocks).
template <int D, int W>
__global__ __launch_bounds__(kDenseThreads * W, 1) void dense_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int hq, int hkv, int capacity, LenSrc lsrc, int n_q, float c,
    int splits, float2* __restrict__ ml, float* __restrict__ o, int rows_total) {
  constexpr int DB = D / 16;
  constexpr int CPR = D / 8;
  constexpr int TILE = 64 * D;                       // elements of one K or V tile
  constexpr int NT = kDenseThreads * W;              // threads per workgroup
  constexpr int ROWS = 64 * W;                       // query rows per workgroup
  constexpr int LPT = 64 * CPR / NT;                 // copies per thread per tensor per tile
  constexpr int LQ = ROWS * CPR / NT;                // query-row copies per thread
  static_assert(LPT >= 1 && LPT * NT == 64 * CPR && LQ * NT == ROWS * CPR,
                "every thread issues the same whole number of copies");
  __shared__ __align__(16) uint16_t smem[kDenseBufs * 2 * TILE + ROWS * D];   // [buffer][K, V], Q

  const int G = hq / hkv;
  const int Rg = n_q * G;
  // grid z = (sequence, ROWS-row block); sequence b of a batch has its own
  // queries, cache and length (one sequence: b = 0)
  const int n_rb = (Rg + ROWS - 1) / ROWS;
  const int s = blockIdx.x, g = blockIdx.y, rb = blockIdx.z % n_rb, b = blockIdx.z / n_rb;
  q += (size_t)b * n_q * hq * D;
  k += (size_t)b * hkv * capacity * D;
  v += (size_t)b * hkv * capacity * D;
  if (lsrc.dev) lsrc.dev += b;
  const int len = lsrc.get();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kh = wave & 1, nbw = wave >> 1;
  const int col = lane & 15, grp = lane >> 4;
  const int r0 = rb * ROWS + nbw * 16;               // first query row of this wave
  const bool active = r0 < Rg;                       // wave-uniform
  const int rho = r0 + col;
  const bool rok = rho < Rg;
  const int qi = rok ? rho / G : 0;
  const int hh = g * G + (rok ? rho % G : 0);
  // The row block's query rows go to LDS by direct-to-LDS copies ahead of
  // the first K/V tiles, so their latency overlaps the tiles' (rows past
  // Rg re-read row Rg - 1; their results are never stored).
  uint16_t* qs = smem + kDenseBufs * 2 * TILE;
#pragma unroll
  for (int u = 0; u < LQ; ++u) {
    const int slot = NT * u + tid;
    const int row = slot / CPR, phys = slot % CPR;
    const int rr = min(rb * ROWS + row, Rg - 1);
    const uint16_t* src = q + ((size_t)(rr / G) * hq + g * G + rr % G) * D +
                          (Tile<D>::slot_k(row, phys) << 3);
    dma16(src, lds_addr(qs) + (NT * u + 64 * wave) * 16);
  }

  // (the device length, loaded at entry, is first needed here)
  const int qpos = len - n_q + qi;
  const int ntiles_all = (len + 63) / 64;
  // tiles of this split (none when a device length leaves it past the end)
  const int ntiles = s < ntiles_all ? (ntiles_all - s + splits - 1) / splits : 0;
  const int safe_end = len - n_q + 1;    // keys < safe_end: visible to every row
  const uint16_t* khd = k + (size_t)g * capacity * D;
  const uint16_t* vhd = v + (size_t)g * capacity * D;
  auto tile_key = [&](int i) { return (s + i * splits) * 64; };
  auto kbuf = [&](int b) { return smem + b * 2 * TILE; };
  auto vbuf = [&](int b) { return smem + b * 2 * TILE + TILE; };

  float m = -INFINITY, lsum = 0.f;
  floatx4_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // Step i (B = kDenseBufs buffers): wait until tile i has landed (tiles
  // i+1 .. i+B-2 may still be in flight), barrier, refill the buffer read
  // in step i-1 with tile i+B-1, reduce tile i.  Copies past the last tile
  // re-read valid rows, so the count in flight is the same at every step.
  // Unrolled by B so every buffer index is static.
  constexpr int kInFlight = 2 * (kDenseBufs - 2) * LPT;   // copies of B-2 tiles
#pragma unroll
  for (int b = 0; b < kDenseBufs - 1; ++b)
    dense_issue_tile<D, NT>(kbuf(b), vbuf(b), khd, vhd, tile_key(b), len, tid, wave);
  // the query rows have landed (the prologue's tile copies may still be in
  // flight); each wave takes its 16 rows' operand
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (kDenseBufs - 1) * LPT));
  __syncthreads();
  // (padding rows take a zero operand: see dense_step)
  bf16x8_t qb[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    uint4 u = *reinterpret_cast<const uint4*>(qs + Tile<D>::off_k(nbw * 16 + col, (D / 32) * grp + kk));
    if (!rok) u = make_uint4(0u, 0u, 0u, 0u);
    qb[kk] = as_bf16x8(u);
  }
  for (int i = 0; i < ntiles; i += kDenseBufs) {
#pragma unroll
    for (int b = 0; b < kDenseBufs; ++b) {
      if (i + b < ntiles) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInFlight));
        __syncthreads();
        const int nb = (b + kDenseBufs - 1) % kDenseBufs;
        dense_issue_tile<D, NT>(kbuf(nb), vbuf(nb), khd, vhd, tile_key(i + b + kDenseBufs - 1), len,
                            tid, wave);
        if (active)
          dense_step<D>(kbuf(b), vbuf(b), qb, kh, tile_key(i + b), len, safe_end, qpos, c, col,
                        grp, rok, m, lsum, oacc);
      }
    }
  }
  // every copy has landed before the buffers are reused for the merge
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // merge the two key halves: odd waves hand (m, l, O) to their even partner
  constexpr int XS = 2 + 4 * DB;                     // floats per lane
  static_assert(4 * W * 64 * XS * 4 <= kDenseBufs * 2 * TILE * 2, "the merge fits the tile buffers");
  float* xch = reinterpret_cast<float*>(smem);
  if (kh == 1 && active) {
    float* dst = xch + (size_t)(nbw * 64 + lane) * XS;
    dst[0] = m;
    dst[1] = lsum;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[2 + 4 * db + i] = oacc[db][i];
  }
  __syncthreads();
  if (kh == 1 || !active) return;
  const float* src = xch + (size_t)(nbw * 64 + lane) * XS;
  const float m1 = src[0];
  const float l1 = src[1];
  const float M = fmaxf(m, m1);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  const float a0 = fast_exp2(m - Ms), a1 = fast_exp2(m1 - Ms);
  const float L = sum_over_groups(lsum * a0 + l1 * a1);
  if (!rok) return;
  const size_t slot = (size_t)s * rows_total + ((size_t)b * n_q + qi) * hq + hh;
  if (grp == 0) ml[slot] = make_float2(M, L);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    floatx4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = oacc[db][i] * a0 + src[2 + 4 * db + i] * a1;
    *reinterpret_cast<floatx4_t*>(o + slot * D + db * 16 + 4 * grp) = r;
  }
}

// ---------------------------------------------------------------------------
// Sparse draft step: grid (split of P * kSparseChunk key-list entries, KV
// head, sequence), kSparseWaves waves of kSparseEntriesPerWave entries per
// pass; P = 1, or 2 for a batch whose grid would exceed one round of
// resident workgroups (two per CU).
//
// Each wave gathers its entries of the head's key list (prefix + selected
// visual positions + tail) into its own LDS region -- one contiguous
// 256-byte row per 16 lanes, all loads issued before any is used -- and
// reduces them for the G <= 16 query heads of the group (one MFMA column
// block).  The waves merge in LDS and the workgroup writes one
// (max, sum, output) partial for the combine pass.  Splits are small so the
// grid covers the chip: the step moves only a few MB and is bound by the
// latency of the index load -> row gather -> reduce chain, which every
// workgroup runs once.
constexpr int kSparseWaves = kSparseChunk / kSparseEntriesPerWave;

template <int D, int P>
__global__ __launch_bounds__(64 * kSparseWaves, 2) void sparse_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int hq, int hkv, int capacity, float c,
    const int32_t* __restrict__ idx, int vis_start, int vis_end, int topk, LenSrc lsrc,
    const int32_t* __restrict__ gamma_dev, int step, int splits, int rows_total,
    float2* __restrict__ ml, float* __restrict__ o) {
  constexpr int EW = kSparseEntriesPerWave;
  constexpr int NKB = EW / 16;
  using TM = TileMath<D, NKB>;
  constexpr int DB = TM::DB;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int NL = EW * CPR / 64;   // loads per lane per tensor
  constexpr int REGION = EW * D;      // elements of one wave's K (or V) tile
  constexpr int XS = 2 + 4 * DB;      // floats per lane in the merge
  constexpr int STAGE = kSparseWaves * 2 * REGION * 2;
  constexpr int XCH = kSparseWaves * 64 * XS * 4;
  __shared__ __align__(16) uint8_t smem_raw[STAGE > XCH ? STAGE : XCH];
  __shared__ int pos_s[kSparseChunk * P];
  uint16_t* smem = reinterpret_cast<uint16_t*>(smem_raw);

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;   // split, KV head, sequence
  // a sequence whose own draft length ends before this step drafts nothing
  // (the whole workgroup leaves; the combine skips its rows likewise)
  if (gamma_dev && gamma_dev[b] <= step) return;
  // sequence b of a batch: its query rows, cache, index list and length
  q += (size_t)b * hq * D;
  k += (size_t)b * hkv * capacity * D;
  v += (size_t)b * hkv * capacity * D;
  idx += (size_t)b * hkv * topk;
  if (lsrc.dev) lsrc.dev += b;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = hq / hkv;
  const int col = lane & 15, grp = lane >> 4;
  const bool row_ok = col < G;
  const int h = g * G + (row_ok ? col : 0);
  uint16_t* Ks = smem + wave * 2 * REGION;
  uint16_t* Vs = Ks + REGION;
  int* pw = pos_s + wave * EW * P;

  // Positions come from the list at the host bound (entries past it re-read
  // its last row), so the index reads and the row gathers do not wait for
  // the device length; entries past the actual list are masked below.
  KeyList kl{true, idx + (size_t)g * topk, vis_start, vis_end, topk};
  const int n_bound = vis_start + topk + max(0, lsrc.max - vis_end);
  // A workgroup takes P consecutive chunks of kSparseChunk entries; in pass
  // p wave w reduces entries e0 + p * kSparseChunk + [0, EW).
  const int e0 = s * (kSparseChunk * P) + wave * EW;   // this wave's first entry
  // lane 63 fetches the device length beside the index reads.  An opaque
  // zero lane offset makes it a vector load: a scalar load would be waited
  // for together with the argument loads (scalar loads complete out of
  // order), i.e. before anything else is issued.
  int zero_v;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero_v));
  int len_raw = 0;
  if (lane == 63) len_raw = lsrc.ptr()[zero_v];
  if (lane < EW * P)
    pw[lane] = kl.pos(min(e0 + (lane / EW) * kSparseChunk + lane % EW, n_bound - 1));
  // The query operand: padding columns (G < 16) read a valid row (head g*G)
  // unconditionally, so the loads need no merge and stay in flight beside
  // the index reads; their results are never stored.
  bf16x8_t qb[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qb[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(q + (size_t)h * D + (D / 4) * grp + 8 * kk));
  // pw is written and read by this wave only
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();

  const uint16_t* kh = k + (size_t)g * capacity * D;
  const uint16_t* vh = v + (size_t)g * capacity * D;
  // gathered rows load in their natural chunk order (short address path
  // after the index read); the swizzle is applied to the LDS stores.  The
  // rows of every pass are loaded before any is used, so P passes wait
  // about one memory latency.  The loads are non-temporal: a call reads each
  // row once, and at 28 layers a draft step's rows do not stay cached until
  // the next step anyway.
  u32x4_t kreg[P][NL], vreg[P][NL];
#pragma unroll
  for (int ps = 0; ps < P; ++ps)
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int cl = lane + 64 * u;
      const int row = cl / CPR, chunk = cl % CPR;
      const size_t base = (size_t)pw[ps * EW + row] * D + (chunk << 3);
      kreg[ps][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kh + base));
      vreg[ps][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vh + base));
    }
  // Entries past the actual list read rows the cache need not hold finite
  // values in: their scores are masked by selects below, and their V rows
  // are stored as zeros so that 0 * V stays 0 in the PV product.
  const int len = lsrc.resolve(__builtin_amdgcn_readlane(len_raw, 63));
  const int n_entries = vis_start + topk + max(0, len - vis_end);

  float m = -INFINITY, lsum = 0.f;
  floatx4_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ps = 0; ps < P; ++ps) {
    const int ep = e0 + ps * kSparseChunk;     // this pass's first entry (wave-uniform)
    // the previous pass's LDS reads have returned before its rows are overwritten
    if (ps > 0) {
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int cl = lane + 64 * u;
      const int row = cl / CPR, chunk = cl % CPR;
      const u32x4_t zero = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(Ks + Tile<D>::off_k(row, chunk)) = kreg[ps][u];
      *reinterpret_cast<u32x4_t*>(Vs + Tile<D>::off_v(row, chunk)) =
          ep + row < n_entries ? vreg[ps][u] : zero;
    }
    // the wave reads back only its own region: no workgroup barrier needed
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own LDS stores done
    __builtin_amdgcn_wave_barrier();
    if (ep < n_entries) {
      floatx4_t sacc[NKB];
      TM::scores(Ks, qb, col, grp, sacc);
      float x[4 * NKB], p[4 * NKB];
#pragma unroll
      for (int j = 0; j < 4 * NKB; ++j)
        x[j] = ep + (j >> 2) * 16 + 4 * grp + (j & 3) < n_entries ? sacc[j >> 2][j & 3] * c
                                                                  : -INFINITY;
      online_update<DB, 4 * NKB>(x, p, m, lsum, oacc);
      TM::pv(Vs, p, col, grp, oacc);
    }
  }
  lsum = sum_over_groups(lsum);

  // merge the waves: each lane's (m, l, 4*DB outputs) through LDS
  float* xch = reinterpret_cast<float*>(smem_raw);
  __syncthreads();                     // every wave is done with its tile
  if (wave > 0) {
    float* dst = xch + (size_t)(wave * 64 + lane) * XS;
    dst[0] = m;
    dst[1] = lsum;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[2 + 4 * db + i] = oacc[db][i];
  }
  __syncthreads();
  if (wave == 0) {
    float mw[kSparseWaves];
    mw[0] = m;
    float M = m;
#pragma unroll
    for (int w = 1; w < kSparseWaves; ++w) {
      mw[w] = xch[(size_t)(w * 64 + lane) * XS];
      M = fmaxf(M, mw[w]);
    }
    const float Ms = (M == -INFINITY) ? 0.f : M;
    const float a0 = fast_exp2(mw[0] - Ms);
    float L = lsum * a0;
    floatx4_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = oacc[db] * a0;
#pragma unroll
    for (int w = 1; w < kSparseWaves; ++w) {
      const float* src = xch + (size_t)(w * 64 + lane) * XS;
      const float a = fast_exp2(mw[w] - Ms);
      L = fmaf(src[1], a, L);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[db][i] = fmaf(src[2 + 4 * db + i], a, acc[db][i]);
    }
    if (row_ok) {
      const size_t slot = (size_t)s * rows_total + (size_t)b * hq + h;
      if (grp == 0) ml[slot] = make_float2(M, L);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<floatx4_t*>(o + slot * D + db * 16 + 4 * grp) = acc[db];
    }
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU split-K attention, one wave per (query row, KV head, chunk).
// Used for fp32 caches; straightforward rather than fast.
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int hq, int hkv,
    int capacity, LenSrc lsrc, int n_q, float c, KeyList kl, int sparse_chunk,
    float2* __restrict__ ml, float* __restrict__ o, int rows_total) {
  const int len = lsrc.get();
  const int n_entries = kl.sparse ? kl.vis_start + kl.topk + max(0, len - kl.vis_end) : len;
  const int chunk = kl.sparse ? sparse_chunk : (n_entries + gridDim.z - 1) / gridDim.z;
  constexpr int DPL = D / 64;  // output elements per lane
  __shared__ float qs[D];
  __shared__ float ps[64];
  __shared__ int poss[64];
  const int rho = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = hq / hkv;
  const int qi = rho / G;
  const int h = g * G + rho % G;
  const int qpos = len - n_q + qi;
  if (kl.sparse) kl.idx += (size_t)g * kl.topk;
  for (int d = lane; d < D; d += 64) qs[d] = Elem<T>::load(q, ((size_t)qi * hq + h) * D + d);
  __syncthreads();

  const T* kh = k + (size_t)g * capacity * D;
  const T* vh = v + (size_t)g * capacity * D;
  const int e0 = s * chunk, e1 = min(n_entries, e0 + chunk);
  float m = -INFINITY, lsum = 0.f;
  float oa[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) oa[u] = 0.f;

  for (int t0 = e0; t0 < e1; t0 += 64) {
    const int e = t0 + lane;
    bool valid = e < e1;
    const int pos = valid ? kl.pos(e) : 0;
    if (!kl.sparse && pos > qpos) valid = false;
    float x = -INFINITY;
    if (valid) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], Elem<T>::load(kh, (size_t)pos * D + d), acc);
      x = acc * c;
    }
    const float mnew = fmaxf(m, wave_max(x));
    const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(m - msafe);
    const float p = valid ? fast_exp2(x - msafe) : 0.f;
    lsum = lsum * alpha + wave_sum(p);
    ps[lane] = p;
    poss[lane] = valid ? pos : -1;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < DPL; ++u) oa[u] *= alpha;
    for (int j = 0; j < 64; ++j) {
      const int pj = poss[j];
      if (pj < 0) continue;
      const float w = ps[j];
#pragma unroll
      for (int u = 0; u < DPL; ++u)
        oa[u] = fmaf(w, Elem<T>::load(vh, (size_t)pj * D + lane + 64 * u), oa[u]);
    }
    __syncthreads();
    m = mnew;
  }
  const size_t slot = (size_t)s * rows_total + (size_t)qi * hq + h;
  if (lane == 0) ml[slot] = make_float2(m, lsum);
#pragma unroll
  for (int u = 0; u < DPL; ++u) o[slot * D + lane + 64 * u] = oa[u];
}

// ---------------------------------------------------------------------------
// Split combine: out[r] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// M = max_s m_s.  One 256-thread workgroup per query row.  Thread (sg, dq)
// merges splits sg, sg + NSG, ... online (running max, rescale on a new
// max); the loads of kCombineBatch of its splits are issued together
// before any is merged, so a call waits about one memory latency per batch.
// The NSG groups are then merged in LDS in a fixed order, so the result
// does not depend on timing.
constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float2* __restrict__ ml, const float* __restrict__ o, int splits, int rows,
    T* __restrict__ out, const int32_t* __restrict__ gamma_dev, int step, int rows_per_seq) {
  constexpr int DQ = D / 4;                      // float4 columns
  constexpr int NSG = kCombineThreads / DQ;      // split groups
  __shared__ float4 part[NSG][DQ];
  __shared__ float2 stat[NSG][DQ];
  const int r = blockIdx.x, tid = threadIdx.x;
  // rows of a sequence that drafts nothing in this step keep their output
  if (gamma_dev && gamma_dev[r / rows_per_seq] <= step) return;
  const int dq = tid % DQ, sg = tid / DQ;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = sg; s0 < splits; s0 += NSG * kCombineBatch) {
    float2 st[kCombineBatch];
    float4 x[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int s = s0 + u * NSG;
      st[u] = make_float2(-INFINITY, 0.f);
      x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < splits) {
        st[u] = ml[(size_t)s * rows + r];
        x[u] = *reinterpret_cast<const float4*>(o + ((size_t)s * rows + r) * D + 4 * dq);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const float Mn = fmaxf(M, st[u].x);
      const float Ms = (Mn == -INFINITY) ? 0.f : Mn;
      const float a = fast_exp2(M - Ms), b = fast_exp2(st[u].x - Ms);
      L = L * a + st[u].y * b;
      acc.x = acc.x * a + x[u].x * b;
      acc.y = acc.y * a + x[u].y * b;
      acc.z = acc.z * a + x[u].z * b;
      acc.w = acc.w * a + x[u].w * b;
      M = Mn;
    }
  }
  part[sg][dq] = acc;
  stat[sg][dq] = make_float2(M, L);
  __syncthreads();
  if (tid < DQ) {
    float Mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < NSG; ++g) Mt = fmaxf(Mt, stat[g][tid].x);
    const float Ms = (Mt == -INFINITY) ? 0.f : Mt;
    float Lt = 0.f;
    float4 a4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int g = 0; g < NSG; ++g) {
      const float w = fast_exp2(stat[g][tid].x - Ms);
      Lt = fmaf(stat[g][tid].y, w, Lt);
      const float4 b = part[g][tid];
      a4.x = fmaf(b.x, w, a4.x);
      a4.y = fmaf(b.y, w, a4.y);
      a4.z = fmaf(b.z, w, a4.z);
      a4.w = fmaf(b.w, w, a4.w);
    }
    const float inv = 1.f / Lt;
    const size_t base = (size_t)r * D + 4 * tid;
    Elem<T>::store(out, base + 0, a4.x * inv);
    Elem<T>::store(out, base + 1, a4.y * inv);
    Elem<T>::store(out, base + 2, a4.z * inv);
    Elem<T>::store(out, base + 3, a4.w * inv);
  }
}

template <typename T>
hipError_t launch_combine(const AttnArgs& a, hipStream_t st) {
  const int rows = (a.batch > 1 ? a.batch : 1) * a.n_q * a.hq;
  const auto* mlp = reinterpret_cast<const float2*>(a.ml);
  T* out = static_cast<T*>(a.out);
  const int rps = a.n_q * a.hq;                  // rows of one sequence
  if (a.d == 128)
    combine_kernel<T, 128><<<rows, kCombineThreads, 0, st>>>(mlp, a.o, a.splits, rows, out,
                                                             a.gamma_dev, a.step, rps);
  else
    combine_kernel<T, 64><<<rows, kCombineThreads, 0, st>>>(mlp, a.o, a.splits, rows, out,
                                                            a.gamma_dev, a.step, rps);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu(const AttnArgs& a, const KeyList& kl, hipStream_t st) {
  const int rows_group = a.n_q * (a.hq / a.hkv);
  dim3 grid(rows_group, a.hkv, a.splits);
  attn_valu_kernel<T, D><<<grid, 64, 0, st>>>(
      static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
      a.hq, a.hkv, a.capacity, LenSrc{a.len, a.len_dev, a.len_off, a.len_lo}, a.n_q,
      a.scale * kLog2e, kl,
      a.chunk, reinterpret_cast<float2*>(a.ml), a.o, a.n_q * a.hq);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t st) {
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const float c = a.scale * kLog2e;
  const LenSrc lsrc{a.len, a.len_dev, a.len_off, a.len_lo};
  if (a.sparse) {
    const int batch = a.batch > 1 ? a.batch : 1;
    const dim3 grid(a.splits, a.hkv, batch);
    if (a.passes == 2)
      sparse_mfma_kernel<D, 2><<<grid, 64 * kSparseWaves, 0, st>>>(
          q, k, v, a.hq, a.hkv, a.capacity, c, a.idx, a.vis_start, a.vis_start + a.vis_len,
          a.topk, lsrc, a.gamma_dev, a.step, a.splits, batch * a.hq,
          reinterpret_cast<float2*>(a.ml), a.o);
    else
      sparse_mfma_kernel<D, 1><<<grid, 64 * kSparseWaves, 0, st>>>(
          q, k, v, a.hq, a.hkv, a.capacity, c, a.idx, a.vis_start, a.vis_start + a.vis_len,
          a.topk, lsrc, a.gamma_dev, a.step, a.splits, batch * a.hq,
          reinterpret_cast<float2*>(a.ml), a.o);
  } else {
    const int batch = a.batch > 1 ? a.batch : 1;
    const int rows_group = a.n_q * (a.hq / a.hkv);
    if constexpr (D == 128) {
      if (rows_group > 64) {
        dim3 grid(a.splits, a.hkv, batch * ((rows_group + 127) / 128));
        dense_mfma_kernel<D, 2><<<grid, kDenseThreads * 2, 0, st>>>(
            q, k, v, a.hq, a.hkv, a.capacity, lsrc, a.n_q, c, a.splits,
            reinterpret_cast<float2*>(a.ml), a.o, batch * a.n_q * a.hq);
        return hipGetLastError();
      }
    }
    dim3 grid(a.splits, a.hkv, batch * ((rows_group + 63) / 64));
    dense_mfma_kernel<D, 1><<<grid, kDenseThreads, 0, st>>>(
        q, k, v, a.hq, a.hkv, a.capacity, lsrc, a.n_q, c, a.splits,
        reinterpret_cast<float2*>(a.ml), a.o, batch * a.n_q * a.hq);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  const int G = a.hq / a.hkv;
  hipError_t err;
  const bool mfma = a.bf16 && (!a.sparse || G <= 16);
  if (mfma) {
    err = a.d == 128 ? launch_mfma<128>(a, st) : launch_mfma<64>(a, st);
  } else {
    KeyList kl{a.sparse, a.idx, a.vis_start, a.vis_start + a.vis_len, a.topk};
    if (a.bf16)
      err = a.d == 128 ? launch_valu<uint16_t, 128>(a, kl, st)
                       : launch_valu<uint16_t, 64>(a, kl, st);
    else
      err = a.d == 128 ? launch_valu<float, 128>(a, kl, st)
                       : launch_valu<float, 64>(a, kl, st);
  }
  if (err != hipSuccess) return err;
  return a.bf16 ? launch_combine<uint16_t>(a, st) : launch_combine<float>(a, st);
}

}  // namespace stdspec
