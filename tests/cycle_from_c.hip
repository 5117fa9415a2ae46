// A whole StD cycle driven through the C ABI alone (no Python, no torch):
// selection, the device-length draft steps, the dense verify pass and the
// acceptance, on seeded host-made bf16 data.  Checks what holds without an
// oracle: the selected lists are valid (std_check_idx), the draft over all
// visual positions equals the dense single-query pass, every output is
// finite, and the acceptance emits the planted prefix plus the bonus and
// advances the device length by n + 1.  Exit status 0 when every check holds.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "stdspec.h"

static int failures = 0;
#define EXPECT(cond, ...)                   \
  do {                                      \
    if (!(cond)) {                          \
      std::printf("FAIL: " __VA_ARGS__);    \
      std::printf("\n");                    \
      ++failures;                           \
    }                                       \
  } while (0)
#define HIP_OK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); return 2; } } while (0)
#define STD_OK_(x) do { std_status_t s_ = (x); if (s_ != STD_OK) { \
    std::printf("%s: %s (%s)\n", #x, std_status_str(s_), std_last_error()); return 3; } } while (0)

// xorshift64*; a sum of four uniforms, centred and scaled to unit variance
static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni() {
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
static float gauss() { return (float)((uni() + uni() + uni() + uni() - 2.0) * std::sqrt(3.0)); }
static uint16_t to_bf16(float f) {     // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

template <typename T>
static T* dev_copy(const std::vector<T>& h) {
  T* d = nullptr;
  if (hipMalloc(&d, h.size() * sizeof(T) + 256) != hipSuccess) return nullptr;
  if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return d;
}

int main() {
  const int hq = 8, hkv = 2, d = 128, vis = 2000, n_text = 64, topk = 256, gamma = 4;
  const int ctx = vis + n_text, cap = ctx + gamma + 1, vocab = 1000;
  std_attn_shape_t shape = {hq, hkv, d, 1.0f / std::sqrt((float)d)};

  std::vector<uint16_t> k((size_t)hkv * cap * d), v(k.size()), qt((size_t)hq * n_text * d),
      qd((size_t)gamma * hq * d), qv((size_t)(gamma + 1) * hq * d);
  for (auto& x : k) x = to_bf16(gauss());
  for (auto& x : v) x = to_bf16(gauss());
  for (auto& x : qt) x = to_bf16(gauss());
  for (auto& x : qd) x = to_bf16(gauss());
  for (auto& x : qv) x = to_bf16(gauss());
  uint16_t *dk = dev_copy(k), *dv = dev_copy(v), *dqt = dev_copy(qt), *dqd = dev_copy(qd),
           *dqv = dev_copy(qv);
  if (!dk || !dv || !dqt || !dqd || !dqv) { std::printf("allocation failed\n"); return 2; }
  std_kv_t kv = {dk, dv, cap, ctx, STD_DTYPE_BF16};
  std_vis_t vs = {0, vis};
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  // (a) selection
  int32_t *idx = nullptr, *bad = nullptr;
  HIP_OK(hipMalloc(&idx, sizeof(int32_t) * hkv * topk));
  HIP_OK(hipMalloc(&bad, sizeof(int32_t)));
  size_t ws_sel = std_select_topk_workspace(&shape, n_text, vs, topk, &kv);
  void* ws = nullptr;
  std_kv_t kv_cap = {dk, dv, cap, cap, STD_DTYPE_BF16};
  size_t ws_dense = std_dense_verify_workspace(&shape, gamma + 1, &kv_cap);
  std_vis_t all = {0, vis};
  size_t ws_sp = std_sparse_decode_workspace(&shape, &kv_cap, all, vis);
  size_t ws_bytes = ws_sel > ws_dense ? ws_sel : ws_dense;
  if (ws_sp > ws_bytes) ws_bytes = ws_sp;
  EXPECT(ws_sel && ws_dense && ws_sp, "a workspace query returned 0: %s", std_last_error());
  HIP_OK(hipMalloc(&ws, ws_bytes));
  STD_OK_(std_select_topk(&shape, dqt, vis, n_text, &kv, vs, topk, nullptr, idx, nullptr, ws,
                          ws_bytes, st));
  STD_OK_(std_check_idx(idx, hkv, topk, vs, bad, st));
  int32_t h_bad = -1;
  HIP_OK(hipMemcpyAsync(&h_bad, bad, 4, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  EXPECT(h_bad == 0, "selection returned %d invalid list entries", h_bad);

  // (b) the draft over every visual position is the dense model's
  std::vector<int32_t> full((size_t)hkv * vis);
  for (int g = 0; g < hkv; ++g)
    for (int j = 0; j < vis; ++j) full[(size_t)g * vis + j] = j;
  int32_t* dfull = dev_copy(full);
  uint16_t *o_sp = nullptr, *o_dn = nullptr;
  HIP_OK(hipMalloc(&o_sp, 2 * (gamma + 1) * hq * d));
  HIP_OK(hipMalloc(&o_dn, 2 * (gamma + 1) * hq * d));
  std_kv_t kv1 = {dk, dv, cap, ctx + 1, STD_DTYPE_BF16};
  STD_OK_(std_sparse_decode_attn(&shape, dqd, &kv1, all, dfull, vis, o_sp, ws, ws_bytes, st));
  HIP_OK(hipStreamSynchronize(st));
  STD_OK_(std_dense_verify_attn(&shape, dqd, 1, &kv1, o_dn, ws, ws_bytes, st));
  std::vector<uint16_t> a(hq * d), b(hq * d);
  HIP_OK(hipMemcpyAsync(a.data(), o_sp, 2 * hq * d, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(b.data(), o_dn, 2 * hq * d, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  double worst = 0;
  for (int i = 0; i < hq * d; ++i) worst = std::fmax(worst, std::fabs(from_bf16(a[i]) - from_bf16(b[i])));
  EXPECT(worst <= 2e-2, "sparse over every visual position differs from dense by %.3e", worst);
  std::printf("sparse(K = vis_len) vs dense, one query: max |diff| %.3e\n", worst);

  // (c) one device-length cycle: gamma draft steps, a verify pass, acceptance
  int32_t* seq = nullptr;
  int32_t h_seq = ctx;
  HIP_OK(hipMalloc(&seq, 4));
  HIP_OK(hipMemcpy(seq, &h_seq, 4, hipMemcpyHostToDevice));
  for (int j = 0; j < gamma; ++j)
    STD_OK_(std_sparse_decode_attn_dlen(&shape, dqd + (size_t)j * hq * d, &kv_cap, seq, 1 + j,
                                        vs, idx, topk, o_sp + (size_t)j * hq * d, ws, ws_bytes, st));
  STD_OK_(std_dense_verify_attn_dlen(&shape, dqv, gamma + 1, &kv_cap, seq, gamma + 1, o_dn, ws,
                                     ws_bytes, st));
  // logits: row i's winner is 10 + i; the drafts agree on rows 0 and 1 only
  std::vector<float> logits((size_t)(gamma + 1) * vocab);
  for (auto& x : logits) x = (float)uni();
  for (int i = 0; i <= gamma; ++i) logits[(size_t)i * vocab + 10 + i] = 5.0f;
  std::vector<int32_t> draft = {10, 11, 99, 13};
  float* dlog = dev_copy(logits);
  int32_t *ddraft = dev_copy(draft), *toks = nullptr, *n_out = nullptr;
  HIP_OK(hipMalloc(&toks, 4 * (gamma + 1)));
  HIP_OK(hipMalloc(&n_out, 4));
  STD_OK_(std_accept(ddraft, gamma, dlog, vocab, STD_DTYPE_F32, toks, n_out, nullptr, seq, st));
  std::vector<int32_t> h_toks(gamma + 1);
  int32_t h_n = 0;
  std::vector<uint16_t> h_sp((size_t)gamma * hq * d), h_dn((size_t)(gamma + 1) * hq * d);
  HIP_OK(hipMemcpyAsync(h_toks.data(), toks, 4 * (gamma + 1), hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(&h_n, n_out, 4, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(&h_seq, seq, 4, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(h_sp.data(), o_sp, h_sp.size() * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(h_dn.data(), o_dn, h_dn.size() * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  bool finite = true;
  for (auto x : h_sp) finite = finite && std::isfinite(from_bf16(x));
  for (auto x : h_dn) finite = finite && std::isfinite(from_bf16(x));
  EXPECT(finite, "a draft or verify output is not finite");
  EXPECT(h_n == 3, "n_out %d, want 3 (two drafts accepted, then the bonus)", h_n);
  EXPECT(h_toks[0] == 10 && h_toks[1] == 11 && h_toks[2] == 12 && h_toks[3] == -1 &&
             h_toks[4] == -1,
         "tokens %d %d %d %d %d", h_toks[0], h_toks[1], h_toks[2], h_toks[3], h_toks[4]);
  EXPECT(h_seq == ctx + 3, "device length %d, want %d", h_seq, ctx + 3);
  std::printf("cycle: n_out %d, tokens %d %d %d, device length %d -> %d\n", h_n, h_toks[0],
              h_toks[1], h_toks[2], ctx, h_seq);
  std::printf("%d failure(s)\n", failures);
  return failures ? 1 : 0;
}
