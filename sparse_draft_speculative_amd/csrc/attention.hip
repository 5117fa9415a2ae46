// Split-K attention kernels of the StD hot path (gfx950, wave64).
//
//  * dense_mfma_kernel  -- the dense model's verify pass (technical summary,
//    Methodology items 2-3: the dense model checks the gamma drafts in one
//    pass over the full KV cache).  One workgroup streams one key chunk of
//    one KV head ONCE for every query row of that head's GQA group (n_q*G
//    rows, 16 per wave), so each K/V byte is read from HBM once per call.
//  * sparse_mfma_kernel -- the sparse model's draft step (Methodology item 2:
//    top-K attention over the visual KV chosen at prefill).  One wave
//    gathers 64 entries of the head's key list (prefix + selected visual
//    positions + tail) into LDS and reduces them for the G query heads.
//  * attn_valu_kernel   -- the same two operations on the vector ALU for
//    fp32 caches (and any shape the MFMA kernels do not take).
//  * combine_kernel     -- merges the per-chunk (max, sum, output) partials
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
// operand is produced by transposing V while staging it into LDS.
// Softmax runs in base 2 with the scale folded into one multiply.

#include "common.hpp"
#include "internal.hpp"

namespace stdspec {
namespace {

// Entry e of the key list of one KV head -> cache position.
struct KeyList {
  bool sparse;
  const int32_t* idx;   // this head's selected positions (sparse only)
  int vis_start, vis_end, topk;
  __device__ __forceinline__ int pos(int e) const {
    if (!sparse || e < vis_start) return e;
    const int t = e - vis_start;
    return t < topk ? idx[t] : vis_end + (t - topk);
  }
};

__device__ __forceinline__ uint32_t half16(const uint4& r, int j) {
  const uint32_t w = (j < 2) ? r.x : (j < 4) ? r.y : (j < 6) ? r.z : r.w;
  return (j & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ floatx4_t mfma_bf16(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 64-key tile of the online softmax for one wave's 16 query columns.
//   Ks: [64][KP] keys (row-major), Vt: [D][VP] transposed values.
//   x[kb*4+i] receives the scaled scores of keys kb*16 + 4*grp + i (already
//   masked by the caller through ``valid``).
template <int D>
struct TileMath {
  static constexpr int KST = D / 32;   // 32-wide contraction steps over d
  static constexpr int DB = D / 16;    // 16-wide output blocks over d
  static constexpr int KP = D + 8;     // LDS pitch of a K row (elements)
  static constexpr int VP = 64 + 8;    // LDS pitch of a V^T row (elements)

  static __device__ __forceinline__ void scores(const uint16_t* Ks, const bf16x8_t* qb,
                                                int col, int grp, floatx4_t* sacc) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) {
        const uint4 a = *reinterpret_cast<const uint4*>(
            Ks + (kb * 16 + col) * KP + (D / 4) * grp + 8 * kk);
        acc = mfma_bf16(as_bf16x8(a), qb[kk], acc);
      }
      sacc[kb] = acc;
    }
  }

  // p holds 16 probabilities in (kb, i) order; accumulate O^T += V^T P^T.
  static __device__ __forceinline__ void pv(const uint16_t* Vt, const float* p, int col,
                                            int grp, floatx4_t* oacc) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 pw;
      pw.x = pack_bf16x2(p[(2 * ks) * 4 + 0], p[(2 * ks) * 4 + 1]);
      pw.y = pack_bf16x2(p[(2 * ks) * 4 + 2], p[(2 * ks) * 4 + 3]);
      pw.z = pack_bf16x2(p[(2 * ks + 1) * 4 + 0], p[(2 * ks + 1) * 4 + 1]);
      pw.w = pack_bf16x2(p[(2 * ks + 1) * 4 + 2], p[(2 * ks + 1) * 4 + 3]);
      const bf16x8_t pb = as_bf16x8(pw);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vr = Vt + (db * 16 + col) * VP + 32 * ks + 4 * grp;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        oacc[db] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, oacc[db]);
      }
    }
  }
};

// Online-softmax state update for one tile.  x: 16 scaled scores (-inf when
// masked).  Returns probabilities in p; updates m (column max, identical in
// the four lanes of a column), lsum (this lane's partial sum) and oacc.
template <int DB>
__device__ __forceinline__ void online_update(const float* x, float* p, float& m, float& lsum,
                                              floatx4_t* oacc) {
  float tmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, x[j]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  const float mnew = fmaxf(m, tmax);
  const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
  const float alpha = fast_exp2(m - msafe);
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    p[j] = fast_exp2(x[j] - msafe);
    psum += p[j];
  }
  lsum = lsum * alpha + psum;
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
  m = mnew;
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
// Dense verify: grid (key chunk, KV head, 64-row block), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void dense_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int hq, int hkv, int capacity, int len, int n_q, float c,
    int chunk, float2* __restrict__ ml, float* __restrict__ o, int rows_total) {
  using TM = TileMath<D>;
  constexpr int KP = TM::KP, VP = TM::VP, DB = TM::DB;
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int KPT = D / 32;    // K chunks per thread == V keys per thread
  __shared__ __align__(16) uint16_t Ks[64 * KP];
  __shared__ __align__(16) uint16_t Vt[D * VP];

  const int s = blockIdx.x, g = blockIdx.y, rb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = hq / hkv;
  const int Rg = n_q * G;
  const int col = lane & 15, grp = lane >> 4;
  const int rho = rb * 64 + wave * 16 + col;
  const bool row_ok = rho < Rg;
  const int qi = row_ok ? rho / G : 0;
  const int h = g * G + (row_ok ? rho % G : 0);
  const int qpos = len - n_q + qi;
  const bool wave_active = rb * 64 + wave * 16 < Rg;

  bf16x8_t qb[D / 32];
  load_q_operand<D>(q + ((size_t)qi * hq + h) * D, row_ok, grp, qb);

  const int key0 = s * chunk;
  const int key1 = min(len, key0 + chunk);
  const uint16_t* kh = k + (size_t)g * capacity * D;
  const uint16_t* vh = v + (size_t)g * capacity * D;
  const int cv = tid % CPR, kg = tid / CPR;

  // Two register staging buffers: while tile t is reduced from LDS, tiles
  // t+1 and t+2 are in flight from HBM.
  uint4 kA[KPT], vA[KPT], kB[KPT], vB[KPT];
  auto load_tile = [&](uint4* kr, uint4* vr, int t0) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int cl = tid + 256 * u;
      const int key = t0 + cl / CPR;
      kr[u] = key < key1 ? *reinterpret_cast<const uint4*>(kh + (size_t)key * D + (cl % CPR) * 8)
                         : make_uint4(0, 0, 0, 0);
      const int vkey = t0 + KPT * kg + u;
      vr[u] = vkey < key1 ? *reinterpret_cast<const uint4*>(vh + (size_t)vkey * D + cv * 8)
                          : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](const uint4* kr, const uint4* vr) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int cl = tid + 256 * u;
      *reinterpret_cast<uint4*>(Ks + (cl / CPR) * KP + (cl % CPR) * 8) = kr[u];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint16_t* dst = Vt + (cv * 8 + j) * VP + KPT * kg;
      if constexpr (KPT == 4) {
        uint2 w;
        w.x = half16(vr[0], j) | (half16(vr[1], j) << 16);
        w.y = half16(vr[2], j) | (half16(vr[3], j) << 16);
        *reinterpret_cast<uint2*>(dst) = w;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = half16(vr[0], j) | (half16(vr[1], j) << 16);
      }
    }
  };

  float m = -INFINITY, lsum = 0.f;
  floatx4_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (key1 - key0 + 63) / 64;
  auto step = [&](uint4* kr, uint4* vr, int t) {
    const int t0 = key0 + t * 64;
    __syncthreads();
    store_tile(kr, vr);
    __syncthreads();
    if (t + 2 < ntiles) load_tile(kr, vr, t0 + 128);
    if (!wave_active) return;
    floatx4_t sacc[4];
    TM::scores(Ks, qb, col, grp, sacc);
    float x[16], p[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t0 + kb * 16 + 4 * grp + i;
        const bool ok = key < key1 && key <= qpos;
        x[kb * 4 + i] = ok ? sacc[kb][i] * c : -INFINITY;
      }
    }
    online_update<DB>(x, p, m, lsum, oacc);
    TM::pv(Vt, p, col, grp, oacc);
  };
  load_tile(kA, vA, key0);
  if (ntiles > 1) load_tile(kB, vB, key0 + 64);
  for (int t = 0; t < ntiles; t += 2) {
    step(kA, vA, t);
    if (t + 1 < ntiles) step(kB, vB, t + 1);
  }

  if (!wave_active) return;
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (!row_ok) return;
  const size_t slot = (size_t)s * rows_total + (size_t)qi * hq + h;
  if (grp == 0) ml[slot] = make_float2(m, lsum);
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *reinterpret_cast<floatx4_t*>(o + slot * D + db * 16 + 4 * grp) = oacc[db];
}

// ---------------------------------------------------------------------------
// Sparse draft step: grid (64-entry chunk of the key list, KV head), 1 wave.
// The wave gathers its 64 K and V rows (16-byte loads, 16 lanes per row, so
// each row is one contiguous 256-byte read) into LDS, all loads issued
// before any is consumed.
template <int D>
__global__ __launch_bounds__(64) void sparse_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int hq, int hkv, int capacity, float c,
    const int32_t* __restrict__ idx, int vis_start, int vis_end, int topk, int n_entries,
    float2* __restrict__ ml, float* __restrict__ o) {
  using TM = TileMath<D>;
  constexpr int KP = TM::KP, VP = TM::VP, DB = TM::DB;
  constexpr int CPR = D / 8;          // chunks per row; also loads per lane
  constexpr int KPV = 64 / (64 / CPR);  // V keys per lane (== CPR)
  __shared__ __align__(16) uint16_t Ks[64 * KP];
  __shared__ __align__(16) uint16_t Vt[D * VP];
  __shared__ int pos_s[64];

  const int s = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x;
  const int G = hq / hkv;
  const int col = lane & 15, grp = lane >> 4;
  const bool row_ok = col < G;
  const int h = g * G + (row_ok ? col : 0);

  KeyList kl{true, idx + (size_t)g * topk, vis_start, vis_end, topk};
  const int e = s * 64 + lane;
  pos_s[lane] = e < n_entries ? kl.pos(e) : -1;
  __syncthreads();

  const uint16_t* kh = k + (size_t)g * capacity * D;
  const uint16_t* vh = v + (size_t)g * capacity * D;
  const int cv = lane % CPR, kg = lane / CPR;
  uint4 kreg[CPR], vreg[KPV];
#pragma unroll
  for (int u = 0; u < CPR; ++u) {
    const int cl = lane + 64 * u;
    const int pk = pos_s[cl / CPR];
    kreg[u] = pk >= 0 ? *reinterpret_cast<const uint4*>(kh + (size_t)pk * D + (cl % CPR) * 8)
                      : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < KPV; ++u) {
    const int pv = pos_s[KPV * kg + u];
    vreg[u] = pv >= 0 ? *reinterpret_cast<const uint4*>(vh + (size_t)pv * D + cv * 8)
                      : make_uint4(0, 0, 0, 0);
  }
  bf16x8_t qb[D / 32];
  load_q_operand<D>(q + (size_t)h * D, row_ok, grp, qb);

#pragma unroll
  for (int u = 0; u < CPR; ++u) {
    const int cl = lane + 64 * u;
    *reinterpret_cast<uint4*>(Ks + (cl / CPR) * KP + (cl % CPR) * 8) = kreg[u];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int w4 = 0; w4 < KPV / 4; ++w4) {
      uint2 w;
      w.x = half16(vreg[4 * w4 + 0], j) | (half16(vreg[4 * w4 + 1], j) << 16);
      w.y = half16(vreg[4 * w4 + 2], j) | (half16(vreg[4 * w4 + 3], j) << 16);
      *reinterpret_cast<uint2*>(Vt + (cv * 8 + j) * VP + KPV * kg + 4 * w4) = w;
    }
  }
  __syncthreads();

  floatx4_t sacc[4];
  TM::scores(Ks, qb, col, grp, sacc);
  float x[16], p[16];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[kb * 4 + i] = pos_s[kb * 16 + 4 * grp + i] >= 0 ? sacc[kb][i] * c : -INFINITY;
  float m = -INFINITY, lsum = 0.f;
  floatx4_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  online_update<DB>(x, p, m, lsum, oacc);
  TM::pv(Vt, p, col, grp, oacc);
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (!row_ok) return;
  const size_t slot = (size_t)s * hq + h;
  if (grp == 0) ml[slot] = make_float2(m, lsum);
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *reinterpret_cast<floatx4_t*>(o + slot * D + db * 16 + 4 * grp) = oacc[db];
}

// ---------------------------------------------------------------------------
// Vector-ALU split-K attention, one wave per (query row, KV head, chunk).
// Used for fp32 caches; straightforward rather than fast.
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int hq, int hkv,
    int capacity, int len, int n_q, float c, KeyList kl, int n_entries, int chunk,
    float2* __restrict__ ml, float* __restrict__ o, int rows_total) {
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
// M = max_s m_s.  One 256-thread workgroup per query row; the splits are
// spread over the threads (weights staged in LDS), each thread then sums a
// float4 column over a strided subset of splits and the subsets are added
// in a fixed order, so the result does not depend on timing.
constexpr int kCombineThreads = 256;
constexpr int kCombineMaxSplits = 4096;   // LDS weights; larger S loops in chunks

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float2* __restrict__ ml, const float* __restrict__ o, int splits, int rows,
    T* __restrict__ out) {
  constexpr int DQ = D / 4;                      // float4 columns
  constexpr int NSG = kCombineThreads / DQ;      // split groups
  __shared__ float wsh[kCombineMaxSplits];
  __shared__ float red[kCombineThreads / kWave];
  __shared__ float4 part[NSG][DQ];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  float M = -INFINITY;
  for (int s = tid; s < splits; s += kCombineThreads) M = fmaxf(M, ml[(size_t)s * rows + r].x);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / kWave; ++w) M = fmaxf(M, red[w]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  __syncthreads();

  const int dq = tid % DQ, sg = tid / DQ;
  float Lloc = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += kCombineMaxSplits) {
    const int s1 = min(splits, s0 + kCombineMaxSplits);
    for (int s = s0 + tid; s < s1; s += kCombineThreads) {
      const float2 st = ml[(size_t)s * rows + r];
      const float w = fast_exp2(st.x - Ms);
      wsh[s - s0] = w;
      Lloc = fmaf(st.y, w, Lloc);
    }
    __syncthreads();
#pragma unroll 4
    for (int s = s0 + sg; s < s1; s += NSG) {
      const float w = wsh[s - s0];
      const float4 x = *reinterpret_cast<const float4*>(o + ((size_t)s * rows + r) * D + 4 * dq);
      acc.x = fmaf(w, x.x, acc.x);
      acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z);
      acc.w = fmaf(w, x.w, acc.w);
    }
    __syncthreads();
  }
  Lloc = wave_sum(Lloc);
  if (lane == 0) red[wave] = Lloc;
  part[sg][dq] = acc;
  __syncthreads();
  if (tid < DQ) {
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kCombineThreads / kWave; ++w) L += red[w];
    float4 a = part[0][tid];
#pragma unroll
    for (int g = 1; g < NSG; ++g) {
      const float4 b = part[g][tid];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    const float inv = 1.f / L;
    const size_t base = (size_t)r * D + 4 * tid;
    Elem<T>::store(out, base + 0, a.x * inv);
    Elem<T>::store(out, base + 1, a.y * inv);
    Elem<T>::store(out, base + 2, a.z * inv);
    Elem<T>::store(out, base + 3, a.w * inv);
  }
}

template <typename T>
hipError_t launch_combine(const AttnArgs& a, hipStream_t st) {
  const int rows = a.n_q * a.hq;
  const auto* mlp = reinterpret_cast<const float2*>(a.ml);
  T* out = static_cast<T*>(a.out);
  if (a.d == 128)
    combine_kernel<T, 128><<<rows, kCombineThreads, 0, st>>>(mlp, a.o, a.splits, rows, out);
  else
    combine_kernel<T, 64><<<rows, kCombineThreads, 0, st>>>(mlp, a.o, a.splits, rows, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu(const AttnArgs& a, const KeyList& kl, int n_entries, hipStream_t st) {
  const int rows_group = a.n_q * (a.hq / a.hkv);
  dim3 grid(rows_group, a.hkv, a.splits);
  attn_valu_kernel<T, D><<<grid, 64, 0, st>>>(
      static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
      a.hq, a.hkv, a.capacity, a.len, a.n_q, a.scale * kLog2e, kl, n_entries, a.chunk,
      reinterpret_cast<float2*>(a.ml), a.o, a.n_q * a.hq);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t st) {
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const float c = a.scale * kLog2e;
  if (a.sparse) {
    const int n_entries = sparse_list_len(a.len, a.vis_start, a.vis_len, a.topk);
    sparse_mfma_kernel<D><<<dim3(a.splits, a.hkv), 64, 0, st>>>(
        q, k, v, a.hq, a.hkv, a.capacity, c, a.idx, a.vis_start, a.vis_start + a.vis_len,
        a.topk, n_entries, reinterpret_cast<float2*>(a.ml), a.o);
  } else {
    const int rows_group = a.n_q * (a.hq / a.hkv);
    dim3 grid(a.splits, a.hkv, (rows_group + 63) / 64);
    dense_mfma_kernel<D><<<grid, 256, 0, st>>>(q, k, v, a.hq, a.hkv, a.capacity, a.len, a.n_q,
                                               c, a.chunk, reinterpret_cast<float2*>(a.ml), a.o,
                                               a.n_q * a.hq);
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
    const int n_entries =
        a.sparse ? sparse_list_len(a.len, a.vis_start, a.vis_len, a.topk) : a.len;
    if (a.bf16)
      err = a.d == 128 ? launch_valu<uint16_t, 128>(a, kl, n_entries, st)
                       : launch_valu<uint16_t, 64>(a, kl, n_entries, st);
    else
      err = a.d == 128 ? launch_valu<float, 128>(a, kl, n_entries, st)
                       : launch_valu<float, 64>(a, kl, n_entries, st);
  }
  if (err != hipSuccess) return err;
  return a.bf16 ? launch_combine<uint16_t>(a, st) : launch_combine<float>(a, st);
}

}  // namespace stdspec
