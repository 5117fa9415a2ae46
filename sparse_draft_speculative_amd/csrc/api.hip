// C ABI of libstdspec: host-side argument checks, workspace sizing and
// dispatch to the gfx950 kernels.  Declarations and their contracts are in
// include/stdspec.h.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/stdspec.h"
#include "internal.hpp"
#include "prefill.hpp"

using namespace stdspec;

namespace {

thread_local char g_err[256] = "";

std_status_t fail(std_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
std_status_t fail(std_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

std_status_t ok() {
  g_err[0] = '\0';
  return STD_OK;
}

std_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(STD_ERR_HIP, "HIP error %d: %s", (int)e, hipGetErrorString(e));
}

#define CHECK(cond, st, ...) \
  do {                       \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

std_status_t check_shape(const std_attn_shape_t* s) {
  CHECK(s, STD_ERR_INVALID_ARGUMENT, "shape is null");
  CHECK(s->n_q_heads >= 1 && s->n_kv_heads >= 1, STD_ERR_INVALID_ARGUMENT,
        "head counts must be >= 1 (got %d, %d)", s->n_q_heads, s->n_kv_heads);
  CHECK(s->n_q_heads % s->n_kv_heads == 0, STD_ERR_INVALID_ARGUMENT,
        "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", s->n_q_heads, s->n_kv_heads);
  CHECK(s->head_dim > 0, STD_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  CHECK(s->head_dim == 64 || s->head_dim == 128, STD_ERR_UNSUPPORTED,
        "head_dim %d unsupported (64 or 128)", s->head_dim);
  CHECK(isfinite(s->scale) && s->scale > 0.f, STD_ERR_INVALID_ARGUMENT,
        "scale must be finite and > 0");
  return ok();
}

std_status_t check_kv(const std_kv_t* kv, bool need_ptrs) {
  CHECK(kv, STD_ERR_INVALID_ARGUMENT, "kv is null");
  CHECK(kv->dtype == STD_DTYPE_F32 || kv->dtype == STD_DTYPE_BF16, STD_ERR_INVALID_ARGUMENT,
        "unknown kv dtype %d", (int)kv->dtype);
  CHECK(kv->capacity >= 1 && kv->len >= 1 && kv->len <= kv->capacity, STD_ERR_INVALID_ARGUMENT,
        "need 1 <= len (%d) <= capacity (%d)", kv->len, kv->capacity);
  if (need_ptrs) CHECK(kv->k && kv->v, STD_ERR_INVALID_ARGUMENT, "kv->k / kv->v is null");
  return ok();
}

// Cache extent in elements must stay addressable with 32-bit row indices
// multiplied out in 64-bit; reject absurd sizes early.
std_status_t check_extent(const std_attn_shape_t* s, const std_kv_t* kv) {
  const double elems = (double)s->n_kv_heads * kv->capacity * s->head_dim;
  CHECK(elems < 9.0e15, STD_ERR_INVALID_ARGUMENT, "cache too large");
  return ok();
}

#define TRY(expr)                            \
  do {                                       \
    std_status_t _st = (expr);               \
    if (_st != STD_OK) return _st;           \
  } while (0)

std_status_t check_sparse(const std_attn_shape_t* s, const std_kv_t* kv, std_vis_t vis,
                          int32_t topk) {
  CHECK(vis.vis_start >= 0 && vis.vis_len >= 1, STD_ERR_INVALID_ARGUMENT,
        "need vis_start >= 0 and vis_len >= 1");
  CHECK((long long)vis.vis_start + vis.vis_len <= kv->len, STD_ERR_INVALID_ARGUMENT,
        "visual span [%d, %lld) exceeds len %d", vis.vis_start,
        (long long)vis.vis_start + vis.vis_len, kv->len);
  CHECK(topk >= 0 && topk <= vis.vis_len, STD_ERR_INVALID_ARGUMENT,
        "need 0 <= topk (%d) <= vis_len (%d)", topk, vis.vis_len);
  CHECK(sparse_list_len(kv->len, vis.vis_start, vis.vis_len, topk) >= 1, STD_ERR_INVALID_ARGUMENT,
        "the sparse key set is empty");
  (void)s;
  return ok();
}

// Entry passes per draft workgroup: one kSparseChunk-entry chunk, or two
// when a batch's grid would otherwise need more than one round of the
// machine's resident workgroups (two per CU).  Two passes load both
// chunks' rows before using either, so a workgroup still waits about one
// memory latency while the grid halves (bf16 MFMA path only; the vector
// ALU path takes one chunk per split).
int sparse_passes(const std_attn_shape_t* s, const std_kv_t* kv, std_vis_t vis, int topk,
                  int batch) {
  if (batch <= 1 || kv->dtype != STD_DTYPE_BF16 || s->n_q_heads / s->n_kv_heads > 16) return 1;
  const long long L = sparse_list_len(kv->len, vis.vis_start, vis.vis_len, topk);
  const long long wg = (long long)batch * s->n_kv_heads * ((L + kSparseChunk - 1) / kSparseChunk);
  return wg > 2 * 256 ? 2 : 1;
}

int sparse_splits(const std_kv_t* kv, std_vis_t vis, int topk, int passes = 1) {
  const int L = sparse_list_len(kv->len, vis.vis_start, vis.vis_len, topk);
  const int per = kSparseChunk * passes;
  return (L + per - 1) / per;
}

// One sequence: dense_split_count.  A batch of several sequences runs in
// rounds of 256 workgroups (one per CU).  Measured at 140k keys, 2 to 16
// sequences: whole rounds and long workgroups read fastest (6.1-6.5 TB/s,
// against 5.2-5.6 with the split count of one sequence rounded up to
// whole rounds), so the split count fills one round, or two when every
// workgroup then still streams at least 128 tiles of 64 keys.
int dense_splits(const std_attn_shape_t* s, const std_kv_t* kv, int n_q, int* chunk,
                 int batch = 1) {
  *chunk = 64;                                   // tile size; splits interleave tiles
  if (batch <= 1) return dense_split_count(kv->len, s->n_kv_heads);
  const long long tiles = (kv->len + 63) / 64;
  // workgroups take 64 query rows, or 128 when a group has more than 64 at
  // head_dim 128
  const long long rows = (long long)n_q * (s->n_q_heads / s->n_kv_heads);
  const long long per_block = rows > 64 && s->head_dim == 128 ? 128 : 64;
  const long long row_blocks = (rows + per_block - 1) / per_block;
  const long long wg = (long long)batch * s->n_kv_heads * row_blocks;   // per split
  const long long rounds = tiles * wg >= 128LL * 512 ? 2 : 1;
  long long S = 256 * rounds / wg;
  if (S < 1) S = 1;
  if (S > tiles) S = tiles;
  return (int)S;
}

std_status_t check_ws(void* ws, size_t have, size_t need) {
  CHECK(have >= need, STD_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", have,
        need);
  CHECK(need == 0 || ws, STD_ERR_INVALID_ARGUMENT, "workspace is null");
  CHECK(((uintptr_t)ws & 255) == 0, STD_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Checks of the dense verify call that need no device pointer (its
// workspace queries apply them too).
std_status_t check_dense(const std_attn_shape_t* s, const std_kv_t* kv, int32_t n_q,
                         int32_t batch) {
  TRY(check_shape(s));
  TRY(check_kv(kv, false));
  TRY(check_extent(s, kv));
  CHECK(n_q >= 1 && n_q <= kv->len, STD_ERR_INVALID_ARGUMENT, "need 1 <= n_q (%d) <= len (%d)",
        n_q, kv->len);
  CHECK(batch >= 1 && (long long)batch * n_q * s->n_q_heads <= (1 << 24),
        STD_ERR_INVALID_ARGUMENT, "need batch (%d) >= 1 and batch * n_q * n_q_heads <= 2^24",
        batch);
  if (batch > 1) {
    const long long n_rb = ((long long)n_q * (s->n_q_heads / s->n_kv_heads) + 63) / 64;
    CHECK(kv->dtype == STD_DTYPE_BF16, STD_ERR_UNSUPPORTED, "batched dense verify needs bf16 KV");
    CHECK(batch * n_rb <= 65535, STD_ERR_INVALID_ARGUMENT,
          "batch * row blocks (%lld) exceeds the grid", batch * n_rb);
  }
  return ok();
}

// The same for the sparse draft call.
std_status_t check_sparse_call(const std_attn_shape_t* s, const std_kv_t* kv, std_vis_t vis,
                               int32_t topk, int32_t batch) {
  TRY(check_shape(s));
  TRY(check_kv(kv, false));
  TRY(check_extent(s, kv));
  TRY(check_sparse(s, kv, vis, topk));
  CHECK(batch >= 1 && batch <= 65535 && (long long)batch * s->n_q_heads <= (1 << 24),
        STD_ERR_INVALID_ARGUMENT, "need 1 <= batch (%d) <= 65535 and batch * n_q_heads <= 2^24",
        batch);
  if (batch > 1) {
    CHECK(kv->dtype == STD_DTYPE_BF16 && s->n_q_heads / s->n_kv_heads <= 16,
          STD_ERR_UNSUPPORTED, "batched sparse decode needs bf16 KV and G <= 16");
  }
  return ok();
}

}  // namespace

namespace stdspec {
// Streaming-read probe (probe.hip): STD_PROBE_SINK_WORDS / 256 workgroups.
hipError_t launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                 hipStream_t stream);
// Index-list check (check.hip): one workgroup.
hipError_t launch_check_idx(const int32_t* idx, int n_kv_heads, int topk, int vis_start,
                            int vis_len, int32_t* bad_out, hipStream_t stream);
}  // namespace stdspec

extern "C" {

int32_t std_abi_version(void) { return STD_ABI_VERSION; }

const char* std_status_str(std_status_t st) {
  switch (st) {
    case STD_OK: return "STD_OK";
    case STD_ERR_INVALID_ARGUMENT: return "STD_ERR_INVALID_ARGUMENT";
    case STD_ERR_UNSUPPORTED: return "STD_ERR_UNSUPPORTED";
    case STD_ERR_WORKSPACE_TOO_SMALL: return "STD_ERR_WORKSPACE_TOO_SMALL";
    case STD_ERR_HIP: return "STD_ERR_HIP";
  }
  return "STD_ERR_UNKNOWN";
}

const char* std_last_error(void) { return g_err; }

// ---------------------------------------------------------------- dense verify
size_t std_dense_verify_workspace(const std_attn_shape_t* s, int32_t n_q, const std_kv_t* kv) {
  if (check_dense(s, kv, n_q, 1) != STD_OK) return 0;
  int chunk;
  const int splits = dense_splits(s, kv, n_q, &chunk);
  return split_workspace(splits, n_q * s->n_q_heads, s->head_dim).bytes();
}

}  // extern "C"

namespace {

std_status_t dense_verify(const std_attn_shape_t* s, const void* q, int32_t n_q, int32_t batch,
                          const std_kv_t* kv, const int32_t* len_dev, int32_t len_off,
                          void* out, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dense(s, kv, n_q, batch));
  TRY(check_kv(kv, true));
  CHECK(q && out, STD_ERR_INVALID_ARGUMENT, "q / out is null");
  CHECK(aligned16(q) && aligned16(kv->k) && aligned16(kv->v) && aligned16(out),
        STD_ERR_INVALID_ARGUMENT, "q, k, v, out must be 16-byte aligned");
  int chunk;
  const int splits = dense_splits(s, kv, n_q, &chunk, batch);
  const SplitWorkspace w = split_workspace(splits, batch * n_q * s->n_q_heads, s->head_dim);
  TRY(check_ws(ws, ws_bytes, w.bytes()));
  AttnArgs a{};
  a.q = q; a.k = kv->k; a.v = kv->v; a.out = out;
  a.hq = s->n_q_heads; a.hkv = s->n_kv_heads; a.d = s->head_dim; a.scale = s->scale;
  a.capacity = kv->capacity; a.len = kv->len; a.n_q = n_q; a.batch = batch;
  a.len_dev = len_dev; a.len_off = len_off;
  a.len_lo = n_q;                         // every query row sees a key
  a.bf16 = kv->dtype == STD_DTYPE_BF16;
  a.sparse = false;
  a.ml = static_cast<float*>(ws);
  a.o = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(w.ml_bytes));
  a.splits = splits; a.chunk = chunk;
  return hip_status(launch_attention(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

std_status_t std_dense_verify_attn(const std_attn_shape_t* s, const void* q, int32_t n_q,
                                   const std_kv_t* kv, void* out, void* ws, size_t ws_bytes,
                                   void* stream) {
  return dense_verify(s, q, n_q, 1, kv, nullptr, 0, out, ws, ws_bytes, stream);
}

std_status_t std_dense_verify_attn_dlen(const std_attn_shape_t* s, const void* q, int32_t n_q,
                                        const std_kv_t* kv, const int32_t* len_dev,
                                        int32_t len_offset, void* out, void* ws,
                                        size_t ws_bytes, void* stream) {
  CHECK(len_dev, STD_ERR_INVALID_ARGUMENT, "len_dev is null");
  return dense_verify(s, q, n_q, 1, kv, len_dev, len_offset, out, ws, ws_bytes, stream);
}

size_t std_dense_verify_batch_workspace(const std_attn_shape_t* s, int32_t n_q, int32_t batch,
                                        const std_kv_t* kv) {
  if (check_dense(s, kv, n_q, batch) != STD_OK) return 0;
  int chunk;
  const int splits = dense_splits(s, kv, n_q, &chunk, batch);
  return split_workspace(splits, batch * n_q * s->n_q_heads, s->head_dim).bytes();
}

std_status_t std_dense_verify_attn_batch(const std_attn_shape_t* s, const void* q, int32_t n_q,
                                         int32_t batch, const std_kv_t* kv,
                                         const int32_t* len_dev, int32_t len_offset, void* out,
                                         void* ws, size_t ws_bytes, void* stream) {
  return dense_verify(s, q, n_q, batch, kv, len_dev, len_offset, out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- sparse draft
size_t std_sparse_decode_workspace(const std_attn_shape_t* s, const std_kv_t* kv, std_vis_t vis,
                                   int32_t topk) {
  if (check_sparse_call(s, kv, vis, topk, 1) != STD_OK) return 0;
  return split_workspace(sparse_splits(kv, vis, topk), s->n_q_heads, s->head_dim).bytes();
}

}  // extern "C"

namespace {

// Every host check of a sparse draft call except the workspace's.
std_status_t check_sparse_args(const std_attn_shape_t* s, const void* q, int32_t batch,
                               const std_kv_t* kv, std_vis_t vis, const int32_t* idx,
                               int32_t topk, const int32_t* gamma_dev, int32_t step,
                               const void* out) {
  TRY(check_sparse_call(s, kv, vis, topk, batch));
  CHECK(!gamma_dev || step >= 0, STD_ERR_INVALID_ARGUMENT, "need step (%d) >= 0", step);
  TRY(check_kv(kv, true));
  CHECK(q && out, STD_ERR_INVALID_ARGUMENT, "q / out is null");
  CHECK(topk == 0 || idx, STD_ERR_INVALID_ARGUMENT, "idx is null");
  CHECK(aligned16(q) && aligned16(kv->k) && aligned16(kv->v) && aligned16(out),
        STD_ERR_INVALID_ARGUMENT, "q, k, v, out must be 16-byte aligned");
  return ok();
}

std_status_t sparse_decode(const std_attn_shape_t* s, const void* q, int32_t batch,
                           const std_kv_t* kv, const int32_t* len_dev, int32_t len_off,
                           std_vis_t vis, const int32_t* idx, int32_t topk,
                           const int32_t* gamma_dev, int32_t step, void* out, void* ws,
                           size_t ws_bytes, void* stream) {
  TRY(check_sparse_args(s, q, batch, kv, vis, idx, topk, gamma_dev, step, out));
  const int passes = sparse_passes(s, kv, vis, topk, batch);
  const int splits = sparse_splits(kv, vis, topk, passes);
  const SplitWorkspace w = split_workspace(splits, batch * s->n_q_heads, s->head_dim);
  TRY(check_ws(ws, ws_bytes, w.bytes()));
  AttnArgs a{};
  a.q = q; a.k = kv->k; a.v = kv->v; a.out = out;
  a.hq = s->n_q_heads; a.hkv = s->n_kv_heads; a.d = s->head_dim; a.scale = s->scale;
  a.capacity = kv->capacity; a.len = kv->len; a.n_q = 1; a.batch = batch;
  a.len_dev = len_dev; a.len_off = len_off;
  // the query sits after the visual span; with neither a prefix nor a
  // selected position the key list needs one position past it
  a.len_lo = vis.vis_start + vis.vis_len + (vis.vis_start + topk == 0 ? 1 : 0);
  a.gamma_dev = gamma_dev; a.step = step;
  a.bf16 = kv->dtype == STD_DTYPE_BF16;
  a.sparse = true; a.idx = idx;
  a.vis_start = vis.vis_start; a.vis_len = vis.vis_len; a.topk = topk;
  a.ml = static_cast<float*>(ws);
  a.o = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(w.ml_bytes));
  a.splits = splits; a.chunk = kSparseChunk; a.passes = passes;
  return hip_status(launch_attention(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

std_status_t std_sparse_decode_attn(const std_attn_shape_t* s, const void* q, const std_kv_t* kv,
                                    std_vis_t vis, const int32_t* idx, int32_t topk, void* out,
                                    void* ws, size_t ws_bytes, void* stream) {
  return sparse_decode(s, q, 1, kv, nullptr, 0, vis, idx, topk, nullptr, 0, out, ws, ws_bytes,
                       stream);
}

std_status_t std_sparse_decode_attn_dlen(const std_attn_shape_t* s, const void* q,
                                         const std_kv_t* kv, const int32_t* len_dev,
                                         int32_t len_offset, std_vis_t vis, const int32_t* idx,
                                         int32_t topk, void* out, void* ws, size_t ws_bytes,
                                         void* stream) {
  CHECK(len_dev, STD_ERR_INVALID_ARGUMENT, "len_dev is null");
  return sparse_decode(s, q, 1, kv, len_dev, len_offset, vis, idx, topk, nullptr, 0, out, ws,
                       ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------- library-owned scratch
// For std_sparse_decode_attn_noalloc (callers that cannot allocate).  Each
// GPU the library runs on holds its own copy of this array until the process
// ends.  On the host its name is only a stand-in, never a device address:
// host code uses the address hipGetSymbolAddress returns, looked up once per
// device with that device current and kept in g_scratch_ptr.
namespace {

__device__ __align__(256) uint8_t scratch[STD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch of the device the call's kernels run on: the current device,
// which a non-null stream must belong to (the address of another device's
// copy would be used on the wrong GPU).
std_status_t scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e);
    CHECK(sdev == dev, STD_ERR_INVALID_ARGUMENT,
          "the stream belongs to device %d but device %d is current", (int)sdev, dev);
  }
  CHECK(dev >= 0 && dev < kMaxDevices, STD_ERR_UNSUPPORTED,
        "device %d is past the library's scratch table (%d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    CHECK(p && ((uintptr_t)p & 255) == 0, STD_ERR_HIP, "scratch address not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" {

std_status_t std_sparse_decode_attn_noalloc(const std_attn_shape_t* s, const void* q,
                                            const std_kv_t* kv, const int32_t* len_dev_or_null,
                                            int32_t len_offset, std_vis_t vis,
                                            const int32_t* idx, int32_t topk, void* out,
                                            void* stream) {
  // every argument check (the scratch size included) before the first HIP call
  TRY(check_sparse_args(s, q, 1, kv, vis, idx, topk, nullptr, 0, out));
  const size_t need =
      split_workspace(sparse_splits(kv, vis, topk), s->n_q_heads, s->head_dim).bytes();
  CHECK(need <= STD_NOALLOC_SCRATCH_BYTES, STD_ERR_WORKSPACE_TOO_SMALL,
        "this call needs %zu bytes of scratch; the library holds %zu", need,
        (size_t)STD_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  TRY(scratch_for_current_device(static_cast<hipStream_t>(stream), &ws));
  return sparse_decode(s, q, 1, kv, len_dev_or_null, len_offset, vis, idx, topk, nullptr, 0, out,
                       ws, STD_NOALLOC_SCRATCH_BYTES, stream);
}

size_t std_sparse_decode_batch_workspace(const std_attn_shape_t* s, int32_t batch,
                                         const std_kv_t* kv, std_vis_t vis, int32_t topk) {
  if (check_sparse_call(s, kv, vis, topk, batch) != STD_OK) return 0;
  return split_workspace(sparse_splits(kv, vis, topk, sparse_passes(s, kv, vis, topk, batch)),
                         batch * s->n_q_heads, s->head_dim)
      .bytes();
}

std_status_t std_sparse_decode_attn_batch(const std_attn_shape_t* s, const void* q,
                                          int32_t batch, const std_kv_t* kv,
                                          const int32_t* len_dev, int32_t len_offset,
                                          std_vis_t vis, const int32_t* idx, int32_t topk,
                                          const int32_t* gamma_dev_or_null, int32_t step,
                                          void* out, void* ws, size_t ws_bytes, void* stream) {
  return sparse_decode(s, q, batch, kv, len_dev, len_offset, vis, idx, topk, gamma_dev_or_null,
                       step, out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- selection
static std_status_t check_select(const std_attn_shape_t* s, int32_t text_start, int32_t n_text,
                                 const std_kv_t* kv, std_vis_t vis, int32_t topk) {
  TRY(check_shape(s));
  TRY(check_kv(kv, false));
  CHECK(n_text >= 1, STD_ERR_INVALID_ARGUMENT, "n_text must be >= 1");
  CHECK(vis.vis_start >= 0 && vis.vis_len >= 1, STD_ERR_INVALID_ARGUMENT,
        "need vis_start >= 0 and vis_len >= 1");
  CHECK((long long)vis.vis_start + vis.vis_len <= text_start, STD_ERR_INVALID_ARGUMENT,
        "text rows must follow the visual span (text_start %d < vis_end %lld)", text_start,
        (long long)vis.vis_start + vis.vis_len);
  CHECK((long long)text_start + n_text <= kv->len, STD_ERR_INVALID_ARGUMENT,
        "text rows [%d, %lld) exceed len %d", text_start, (long long)text_start + n_text,
        kv->len);
  CHECK(topk >= 1 && topk <= vis.vis_len, STD_ERR_INVALID_ARGUMENT,
        "need 1 <= topk (%d) <= vis_len (%d)", topk, vis.vis_len);
  CHECK((long long)s->n_q_heads * n_text <= (1 << 26), STD_ERR_INVALID_ARGUMENT,
        "too many text rows");
  return ok();
}

size_t std_select_topk_workspace(const std_attn_shape_t* s, int32_t n_text, std_vis_t vis,
                                 int32_t topk, const std_kv_t* kv) {
  if (!kv) {
    fail(STD_ERR_INVALID_ARGUMENT, "kv is null");
    return 0;
  }
  if (check_shape(s) != STD_OK) return 0;
  const int text_start = vis.vis_start + vis.vis_len;  // earliest legal start
  const int ts = kv->len - n_text > text_start ? kv->len - n_text : text_start;
  if (check_select(s, ts, n_text, kv, vis, topk) != STD_OK) return 0;
  // size for the largest text_start the cache allows, so the value covers
  // any call with this (shape, n_text, vis, topk, kv)
  return select_workspace_bytes(s->n_q_heads, s->n_kv_heads, s->head_dim, n_text, vis.vis_len,
                                kv->len - n_text, true);
}

std_status_t std_select_topk(const std_attn_shape_t* s, const void* q_text, int32_t text_start,
                             int32_t n_text, const std_kv_t* kv, std_vis_t vis, int32_t topk,
                             const float* lse_or_null, int32_t* idx_out, float* scores_or_null,
                             void* ws, size_t ws_bytes, void* stream) {
  TRY(check_select(s, text_start, n_text, kv, vis, topk));
  TRY(check_extent(s, kv));
  CHECK(kv->k, STD_ERR_INVALID_ARGUMENT, "kv->k is null");
  CHECK(q_text && idx_out, STD_ERR_INVALID_ARGUMENT, "q_text / idx_out is null");
  CHECK(aligned16(q_text) && aligned16(kv->k), STD_ERR_INVALID_ARGUMENT,
        "q_text, k must be 16-byte aligned");
  const size_t need = select_workspace_bytes(s->n_q_heads, s->n_kv_heads, s->head_dim, n_text,
                                             vis.vis_len, text_start, scores_or_null == nullptr);
  TRY(check_ws(ws, ws_bytes, need));
  SelectArgs a{};
  a.q_text = q_text; a.k = kv->k;
  a.hq = s->n_q_heads; a.hkv = s->n_kv_heads; a.d = s->head_dim; a.scale = s->scale;
  a.capacity = kv->capacity; a.text_start = text_start; a.n_text = n_text;
  a.vis_start = vis.vis_start; a.vis_len = vis.vis_len; a.topk = topk;
  a.bf16 = kv->dtype == STD_DTYPE_BF16;
  a.lse_in = lse_or_null; a.idx_out = idx_out; a.scores_out = scores_or_null; a.ws = ws;
  return hip_status(launch_select(a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- acceptance
std_status_t std_accept(const int32_t* draft, int32_t gamma, const void* logits, int32_t vocab,
                        std_dtype_t logits_dtype, int32_t* out_tokens, int32_t* n_out,
                        float* margins_or_null, int32_t* seq_len_inout_or_null, void* stream) {
  return std_accept_batch(draft, gamma, 1, nullptr, logits, vocab, logits_dtype, out_tokens,
                          n_out, margins_or_null, seq_len_inout_or_null, stream);
}

std_status_t std_accept_batch(const int32_t* draft, int32_t gamma, int32_t batch,
                              const int32_t* gamma_dev_or_null, const void* logits, int32_t vocab,
                              std_dtype_t logits_dtype, int32_t* out_tokens, int32_t* n_out,
                              float* margins_or_null, int32_t* seq_len_inout_or_null,
                              void* stream) {
  CHECK(gamma >= 0 && gamma < (1 << 20), STD_ERR_INVALID_ARGUMENT, "gamma %d out of range",
        gamma);
  CHECK(batch >= 1 && (long long)batch * (gamma + 1) <= 0x7fffffffLL, STD_ERR_INVALID_ARGUMENT,
        "need batch (%d) >= 1 and batch * (gamma + 1) rows to fit the grid", batch);
  CHECK(vocab >= 1, STD_ERR_INVALID_ARGUMENT, "vocab must be >= 1");
  CHECK(gamma == 0 || draft, STD_ERR_INVALID_ARGUMENT, "draft is null");
  CHECK(logits && out_tokens && n_out, STD_ERR_INVALID_ARGUMENT,
        "logits / out_tokens / n_out is null");
  CHECK(logits_dtype == STD_DTYPE_F32 || logits_dtype == STD_DTYPE_BF16,
        STD_ERR_INVALID_ARGUMENT, "unknown logits dtype %d", (int)logits_dtype);
  return hip_status(launch_accept(draft, gamma, batch, gamma_dev_or_null, logits, vocab,
                                  logits_dtype == STD_DTYPE_BF16, out_tokens, n_out,
                                  margins_or_null, seq_len_inout_or_null,
                                  static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------ prefill text attention

size_t std_prefill_text_attn_workspace(const std_attn_shape_t* s, int32_t text_start,
                                       int32_t n_text) {
  if (check_shape(s) != STD_OK) return 0;
  if (text_start < 0 || n_text < 1) {
    fail(STD_ERR_INVALID_ARGUMENT, "need text_start (%d) >= 0 and n_text (%d) >= 1", text_start,
         n_text);
    return 0;
  }
  return prefill_workspace_bytes(s->n_q_heads, s->head_dim, text_start, n_text);
}

std_status_t std_prefill_text_attn(const std_attn_shape_t* s, const void* q_text,
                                   int32_t text_start, int32_t n_text, const std_kv_t* kv,
                                   void* out, float* lse_out_or_null, void* ws, size_t ws_bytes,
                                   void* stream) {
  TRY(check_shape(s));
  TRY(check_kv(kv, true));
  TRY(check_extent(s, kv));
  CHECK(kv->dtype == STD_DTYPE_BF16, STD_ERR_UNSUPPORTED,
        "the prefill text attention takes a bf16 cache");
  CHECK(text_start >= 0 && n_text >= 1, STD_ERR_INVALID_ARGUMENT,
        "need text_start (%d) >= 0 and n_text (%d) >= 1", text_start, n_text);
  CHECK((long long)text_start + n_text <= kv->len, STD_ERR_INVALID_ARGUMENT,
        "text rows end at %lld, past len %d", (long long)text_start + n_text, kv->len);
  CHECK((long long)s->n_q_heads * n_text <= (1LL << 30), STD_ERR_INVALID_ARGUMENT,
        "too many text rows");
  CHECK(q_text && out, STD_ERR_INVALID_ARGUMENT, "q_text / out is null");
  CHECK(aligned16(q_text) && aligned16(kv->k) && aligned16(kv->v) && aligned16(out) &&
            ((uintptr_t)lse_out_or_null & 3) == 0,
        STD_ERR_INVALID_ARGUMENT, "q_text, k, v, out must be 16-byte aligned, lse 4-byte");
  TRY(check_ws(ws, ws_bytes,
               prefill_workspace_bytes(s->n_q_heads, s->head_dim, text_start, n_text)));
  PrefillArgs a{};
  a.q_text = q_text; a.k = kv->k; a.v = kv->v; a.out = out; a.lse_out = lse_out_or_null;
  a.hq = s->n_q_heads; a.hkv = s->n_kv_heads; a.d = s->head_dim; a.capacity = kv->capacity;
  a.text_start = text_start; a.n_text = n_text; a.scale = s->scale; a.ws = ws;
  return hip_status(launch_prefill(a, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------ index check

std_status_t std_check_idx(const int32_t* idx, int32_t n_kv_heads, int32_t topk, std_vis_t vis,
                           int32_t* bad_out, void* stream) {
  CHECK(bad_out, STD_ERR_INVALID_ARGUMENT, "bad_out is null");
  CHECK(n_kv_heads >= 1, STD_ERR_INVALID_ARGUMENT, "n_kv_heads must be >= 1");
  CHECK(vis.vis_start >= 0 && vis.vis_len >= 1 &&
            (long long)vis.vis_start + vis.vis_len <= 0x7fffffffLL,
        STD_ERR_INVALID_ARGUMENT, "bad visual span [%d, +%d)", vis.vis_start, vis.vis_len);
  CHECK(topk >= 0 && topk <= vis.vis_len, STD_ERR_INVALID_ARGUMENT,
        "need 0 <= topk (%d) <= vis_len (%d)", topk, vis.vis_len);
  CHECK(topk == 0 || idx, STD_ERR_INVALID_ARGUMENT, "idx is null");
  return hip_status(launch_check_idx(idx, n_kv_heads, topk, vis.vis_start, vis.vis_len, bad_out,
                                     static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------ streaming comparator

std_status_t std_static_window_idx(int32_t n_kv_heads, std_vis_t vis, int32_t sink, int32_t topk,
                                   int32_t* idx_out, void* stream) {
  CHECK(n_kv_heads >= 1, STD_ERR_INVALID_ARGUMENT, "n_kv_heads must be >= 1");
  CHECK(vis.vis_start >= 0 && vis.vis_len >= 1 &&
            (long long)vis.vis_start + vis.vis_len <= 0x7fffffffLL,
        STD_ERR_INVALID_ARGUMENT, "bad visual span [%d, +%d)", vis.vis_start, vis.vis_len);
  CHECK(topk >= 0 && topk <= vis.vis_len, STD_ERR_INVALID_ARGUMENT,
        "need 0 <= topk (%d) <= vis_len (%d)", topk, vis.vis_len);
  CHECK(sink >= 0, STD_ERR_INVALID_ARGUMENT, "need sink (%d) >= 0", sink);
  CHECK((long long)n_kv_heads * topk <= 0x7fffffffLL, STD_ERR_INVALID_ARGUMENT,
        "n_kv_heads * topk too large");
  CHECK(topk == 0 || idx_out, STD_ERR_INVALID_ARGUMENT, "idx_out is null");
  return hip_status(launch_static_window_idx(n_kv_heads, vis.vis_start, vis.vis_len, sink, topk,
                                             idx_out, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------ read probe

std_status_t std_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  CHECK(buf && sink, STD_ERR_INVALID_ARGUMENT, "buf / sink is null");
  CHECK(bytes >= 16 && bytes % 16 == 0, STD_ERR_INVALID_ARGUMENT,
        "bytes (%zu) must be a positive multiple of 16", bytes);
  CHECK(aligned16(buf) && ((uintptr_t)sink & 3) == 0, STD_ERR_INVALID_ARGUMENT,
        "buf must be 16-byte aligned and sink 4-byte aligned");
  return hip_status(launch_hbm_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
