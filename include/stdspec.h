/*
 * stdspec.h -- C ABI of the MI355X (gfx950) Sparse-to-Dense decoding hot path.
 *
 * Source: "Sparse-to-Dense: A Free Lunch for Lossless Acceleration of Video
 * Understanding in LLMs".  The pages describe StD as two modes of one model:
 * a sparse model M_s that drafts gamma tokens with top-K attention over the
 * visual KV chosen at prefill, and the dense model M that verifies them in
 * one pass over the full KV cache, accepting the longest agreeing prefix and
 * one bonus token (technical summary, Methodology items 2-4).
 *
 * Four calls make the hot path, all per layer (except accept), all
 * asynchronous on the caller's HIP stream:
 *   std_select_topk        prefill-time top-K visual KV selection
 *   std_sparse_decode_attn draft-step attention over the selected KV
 *   std_dense_verify_attn  verify attention of gamma+1 queries, full KV
 *   std_accept             greedy longest-prefix acceptance + bonus token
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named q, k, v, out, logits, idx, ... are DEVICE pointers; the
 *   shape structs are HOST pointers read during the call only.  The caller
 *   owns every buffer.  The library allocates and frees nothing and keeps no
 *   state between calls, so calls on different streams do not interfere
 *   (except through buffers the caller shares between them).  The one
 *   exception is std_sparse_decode_attn_noalloc, whose partials live in a
 *   static device array the library holds per GPU (see there).
 * - KV cache of one layer: separate K and V, each [n_kv_heads][capacity]
 *   [head_dim], row-major, dtype bf16 or fp32; positions [0, len) are valid.
 * - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 * - Queries take the KV dtype; outputs are written in the KV dtype; all
 *   accumulation is fp32 (selection scores accumulate across tiles in fp64).
 * - scale multiplies q.k before the softmax (usually 1/sqrt(head_dim)).
 * - head_dim must be 64 or 128.
 * - Argument checks run on the host before any launch; a failed check returns
 *   a status and launches nothing.  STD_ERR_HIP reports a launch failure.
 *   Device-side contents (idx inside the visual span, ascending, distinct)
 *   are preconditions and are not checked; an idx entry outside the span is
 *   clamped into it (the output is then unspecified, but every access stays
 *   inside the cache).  Nothing prints or aborts.
 * - stream is a hipStream_t passed as void*; NULL means the default stream.
 * - Workspace: each call that needs scratch takes a caller-allocated device
 *   buffer of at least the size its *_workspace query returns (256-byte
 *   aligned).  A query returns 0 when its arguments fail a check that its
 *   call makes on them (std_last_error() then names it).  The buffer's
 *   contents need no initialisation and are garbage after the call.  A
 *   workspace serves one call at a time: two calls in flight at once (on
 *   different streams) need two workspaces.
 */
#ifndef STDSPEC_H
#define STDSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STD_ABI_VERSION 2

typedef enum {
  STD_OK = 0,
  STD_ERR_INVALID_ARGUMENT = 1,   /* a null pointer, a size out of range ...  */
  STD_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. d=96)    */
  STD_ERR_WORKSPACE_TOO_SMALL = 3,
  STD_ERR_HIP = 4                 /* a HIP launch or runtime call failed      */
} std_status_t;

typedef enum { STD_DTYPE_F32 = 0, STD_DTYPE_BF16 = 1 } std_dtype_t;

/* Attention shape of one layer. */
typedef struct {
  int32_t n_q_heads;   /* H_q >= 1                                    */
  int32_t n_kv_heads;  /* H_kv >= 1, divides H_q                      */
  int32_t head_dim;    /* d, 64 or 128                                */
  float scale;         /* > 0, finite                                 */
} std_attn_shape_t;

/* One layer's KV cache (device pointers). */
typedef struct {
  const void* k;       /* [n_kv_heads][capacity][head_dim]            */
  const void* v;       /* [n_kv_heads][capacity][head_dim]            */
  int32_t capacity;    /* allocated positions per head                */
  int32_t len;         /* valid positions, 1 <= len <= capacity       */
  std_dtype_t dtype;
} std_kv_t;

/* The visual span [vis_start, vis_start + vis_len) of the cache. */
typedef struct {
  int32_t vis_start;
  int32_t vis_len;
} std_vis_t;

/* ABI version the library was built with (STD_ABI_VERSION). */
int32_t std_abi_version(void);

/* Static string naming a status. */
const char* std_status_str(std_status_t status);

/* Human-readable reason for the last non-OK status returned on the calling
 * thread (thread-local; "" if none).  Valid until the next call on it. */
const char* std_last_error(void);

/* ------------------------------------------------------------------------
 * (a) Prefill-time top-K visual KV selection.
 *
 * Technical summary, Methodology item 4 ("KV cache selection"): the top-K
 * visual KV are chosen once, during prefill, from the average attention
 * score directed from text tokens to visual tokens; the choice differs per
 * layer and per attention head.  Item 2 names the basis: attention weights
 * from text tokens to visual tokens.
 *
 * For each KV head g and visual position j:
 *   score[g][j] = 1/(G*n_text) * sum_{h in group g} sum_{i < n_text}
 *                 softmax_h,i(j)
 * where softmax_h,i is the causal attention row of text query i of query
 * head h, at position text_start + i, over every key it sees (positions
 * [0, text_start + i]).  idx_out[g] receives the K positions with the
 * largest scores, ties to the lower position, in ascending order.
 *
 * q_text   [n_q_heads][n_text][head_dim], KV dtype, the prefill's text
 *          queries (already rotated if the model rotates them).
 * kv       cache holding at least positions [0, text_start + n_text);
 *          kv->len >= text_start + n_text.
 * vis      visual span; vis_start + vis_len <= text_start (text follows the
 *          visual span), vis_len >= 1.
 * topk     1 <= topk <= vis_len.
 * lse_or_null  optional [n_q_heads][n_text] fp32 natural-log log-sum-exp of
 *          each text row (scale applied), e.g. from the caller's prefill
 *          attention; when given the library skips computing it.
 * idx_out  [n_kv_heads][topk] int32, absolute cache positions, ascending.
 * scores_or_null  optional [n_kv_heads][vis_len] fp32 mean probabilities.
 * ------------------------------------------------------------------------ */
size_t std_select_topk_workspace(const std_attn_shape_t* shape, int32_t n_text,
                                 std_vis_t vis, int32_t topk, const std_kv_t* kv);
std_status_t std_select_topk(const std_attn_shape_t* shape, const void* q_text,
                             int32_t text_start, int32_t n_text, const std_kv_t* kv,
                             std_vis_t vis, int32_t topk, const float* lse_or_null,
                             int32_t* idx_out, float* scores_or_null,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * (b) Sparse draft attention, one query token.
 *
 * Technical summary, Methodology item 2: the sparse model M_s uses top-K
 * attention over the visual KV chosen at prefill, cutting draft-phase I/O;
 * item 3: it drafts gamma tokens autoregressively, one at a time.
 *
 * The query sits at position kv->len - 1.  Query head h (KV head g) attends
 * with softmax over the positions
 *   [0, vis_start)  +  idx[g][0..topk)  +  [vis_start + vis_len, kv->len)
 * i.e. every non-visual position and the selected visual ones.
 *
 * q    [n_q_heads][head_dim], KV dtype.
 * idx  [n_kv_heads][topk] int32 absolute positions inside the visual span,
 *      distinct (as std_select_topk returns them); 0 <= topk <= vis_len.
 * vis  the visual span lies inside the valid cache:
 *      vis_start + vis_len <= kv->len; the key set must be non-empty.
 * out  [n_q_heads][head_dim], KV dtype.
 * ------------------------------------------------------------------------ */
size_t std_sparse_decode_workspace(const std_attn_shape_t* shape, const std_kv_t* kv,
                                   std_vis_t vis, int32_t topk);
std_status_t std_sparse_decode_attn(const std_attn_shape_t* shape, const void* q,
                                    const std_kv_t* kv, std_vis_t vis, const int32_t* idx,
                                    int32_t topk, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * (c) Dense verify attention: n_q queries, one pass over the full KV.
 *
 * Technical summary, Methodology item 2: the dense model M uses the full KV
 * cache (standard attention); item 3: it verifies the gamma drafted tokens
 * in parallel with a single I/O pass over the full KV cache.
 *
 * Query i (0 <= i < n_q) sits at position kv->len - n_q + i and attends
 * causally to positions [0, kv->len - n_q + i].  With n_q = 1 this is plain
 * dense decoding.  Each KV head is streamed from HBM once for all n_q*G of
 * its query rows.  The split of the keys across workgroups depends only on
 * kv->len, never on n_q.
 *
 * q    [n_q][n_q_heads][head_dim], KV dtype.   1 <= n_q <= kv->len.
 * out  [n_q][n_q_heads][head_dim], KV dtype.
 * ------------------------------------------------------------------------ */
size_t std_dense_verify_workspace(const std_attn_shape_t* shape, int32_t n_q,
                                  const std_kv_t* kv);
std_status_t std_dense_verify_attn(const std_attn_shape_t* shape, const void* q,
                                   int32_t n_q, const std_kv_t* kv, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Device-resident length variants of (b) and (c).
 *
 * A draft-verify cycle changes the valid length after every acceptance
 * (Methodology item 3: accepted tokens are appended); keeping that length in
 * device memory lets a caller capture a whole cycle once (for example in a
 * HIP graph) and replay it with no host round trip.  These calls read the
 * valid length when their kernels run:
 *     len = min(max(*len_dev + len_offset, lo), kv->len)
 * where lo is the shortest length the call is defined for: n_q (dense: every
 * query row sees at least one key); vis_start + vis_len (sparse: the query
 * follows the visual span), plus one when vis_start + topk == 0 (so the key
 * list is never empty).  A device value below lo is raised to it, so the
 * result is always a defined attention output.  kv->len is the upper bound:
 * it sizes the launch and the workspace (query the *_workspace functions
 * with it), and every other argument, check and result is that of the
 * host-length call with this len.  len_dev is an int32 device pointer, e.g.
 * the seq_len std_accept advances.
 * ------------------------------------------------------------------------ */
std_status_t std_sparse_decode_attn_dlen(const std_attn_shape_t* shape, const void* q,
                                         const std_kv_t* kv, const int32_t* len_dev,
                                         int32_t len_offset, std_vis_t vis, const int32_t* idx,
                                         int32_t topk, void* out, void* workspace,
                                         size_t workspace_bytes, void* stream);
std_status_t std_dense_verify_attn_dlen(const std_attn_shape_t* shape, const void* q,
                                        int32_t n_q, const std_kv_t* kv, const int32_t* len_dev,
                                        int32_t len_offset, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * (b) without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the sparse draft call with its split-K partials in scratch
 * memory the library owns, a static device array of
 * STD_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends.  The call allocates and frees nothing.
 *
 * Arguments and result are those of std_sparse_decode_attn_dlen with
 * len_dev_or_null given, else of std_sparse_decode_attn (length kv->len);
 * the kernels and the split are the same, so the output equals theirs bit
 * for bit.  The scratch needs no initialisation.
 * Errors: every check of those calls; STD_ERR_WORKSPACE_TOO_SMALL when the
 * partials would exceed the scratch (about 4 * n_q_heads * (head_dim + 2)
 * bytes per 128 key-list entries; the 140k-context Qwen2-VL shape with
 * K = 4,096 needs 0.7 MB), before any HIP call.
 * The call runs on the current device; a non-null stream must belong to it
 * (STD_ERR_INVALID_ARGUMENT otherwise).
 * Concurrency: every call on one GPU shares that GPU's scratch, so calls
 * that overlap on one GPU (different streams, or host threads) race; order
 * them on one stream.
 * ------------------------------------------------------------------------ */
#define STD_NOALLOC_SCRATCH_BYTES (8u << 20)
std_status_t std_sparse_decode_attn_noalloc(const std_attn_shape_t* shape, const void* q,
                                            const std_kv_t* kv, const int32_t* len_dev_or_null,
                                            int32_t len_offset, std_vis_t vis, const int32_t* idx,
                                            int32_t topk, void* out, void* stream);

/* ------------------------------------------------------------------------
 * (b, batched) Sparse draft attention for `batch` independent sequences in
 * one launch: the draft step of (b) applied to each sequence, data-parallel
 * over requests (the pages fix no batch size; this serves batch > 1).
 *
 * Layout: q and out [batch][n_q_heads][head_dim]; the caches lie back to
 * back, K and V [batch][n_kv_heads][kv->capacity][head_dim] (kv->k, kv->v
 * point at sequence 0); idx [batch][n_kv_heads][topk], each list as in (b).
 * kv->len bounds every sequence's length and sizes the launch; sequence b
 * uses min(max(len_dev[b] + len_offset, lo), kv->len) (lo as for the
 * device-length calls) when len_dev (batch int32 in device memory) is
 * given, else kv->len.  All sequences share vis and topk.  bf16 KV with
 * n_q_heads / n_kv_heads <= 16 only (STD_ERR_UNSUPPORTED otherwise);
 * 1 <= batch <= 65535.  With batch == 1 the result equals
 * std_sparse_decode_attn(_dlen) bit for bit.
 *
 * Per-sequence draft lengths (Methodology item 3 defines the cycle per
 * sequence: each drafts its own gamma tokens): gamma_dev_or_null is NULL
 * (every sequence drafts in this step) or [batch] int32 device, and the
 * call is draft step `step` (0-based) of a cycle: sequence b takes part only
 * while step < gamma_dev[b]; for the others nothing is read and out[b] is
 * left as it was.  step >= 0 when gamma_dev_or_null is given.
 * ------------------------------------------------------------------------ */
size_t std_sparse_decode_batch_workspace(const std_attn_shape_t* shape, int32_t batch,
                                         const std_kv_t* kv, std_vis_t vis, int32_t topk);
std_status_t std_sparse_decode_attn_batch(const std_attn_shape_t* shape, const void* q,
                                          int32_t batch, const std_kv_t* kv,
                                          const int32_t* len_dev, int32_t len_offset,
                                          std_vis_t vis, const int32_t* idx, int32_t topk,
                                          const int32_t* gamma_dev_or_null, int32_t step,
                                          void* out, void* workspace, size_t workspace_bytes,
                                          void* stream);

/* ------------------------------------------------------------------------
 * (c, batched) Dense verify attention for `batch` independent sequences in
 * one launch, each as std_dense_verify_attn (Technical summary, Methodology
 * items 2-3: one pass of the dense model over each sequence's full cache
 * verifies its gamma drafts).
 *
 * q    [batch][n_q][n_q_heads][head_dim]; out the same layout.
 * kv   kv->k, kv->v point at [batch][n_kv_heads][capacity][head_dim];
 *      kv->len is the bound every sequence's length is clamped to.
 * len_dev  NULL (every sequence has length kv->len) or [batch] int32
 *      device: sequence b uses min(max(len_dev[b] + len_offset, n_q),
 *      kv->len).
 * A batch whose sequences draft different numbers of tokens verifies with
 * n_q = 1 + the largest gamma: sequence b's rows 0..gamma_b are its verify
 * rows (row i sees only keys up to its own position, so the rows after
 * them change nothing in them) and std_accept_batch reads only those.
 * bf16 only for batch > 1 (fp32: STD_ERR_UNSUPPORTED); batch = 1 is
 * std_dense_verify_attn(_dlen) bit for bit.  With batch > 1 the key split
 * count is chosen so the grid fills one whole round of the machine (two
 * when each workgroup still streams at least 128 tiles of 64 keys), which
 * changes the summation order (results stay within the same tolerance).
 * ------------------------------------------------------------------------ */
size_t std_dense_verify_batch_workspace(const std_attn_shape_t* shape, int32_t n_q,
                                        int32_t batch, const std_kv_t* kv);
std_status_t std_dense_verify_attn_batch(const std_attn_shape_t* shape, const void* q,
                                         int32_t n_q, int32_t batch, const std_kv_t* kv,
                                         const int32_t* len_dev, int32_t len_offset, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * (d) Greedy acceptance plus the bonus token.
 *
 * Technical summary, Methodology item 3: verification finds the longest
 * prefix of drafted tokens matching the dense model's predictions (n
 * tokens) and accepts one extra bonus token; the accepted tokens are
 * appended to the context.
 *
 * pred[i] = argmax_v logits[i][v] (ties to the lowest id); row i is the
 * dense prediction after the i-th verify input (x_t, d_1, ..., d_gamma).
 * n = the largest n <= gamma with draft[j] == pred[j] for all j < n.
 *
 * draft        [gamma] int32 device; gamma >= 0 (gamma = 0: plain greedy).
 * logits       [gamma+1][vocab] device, fp32 or bf16; vocab >= 1.
 * out_tokens   [gamma+1] int32 device: pred[0..n] (= d_1..d_n, then the
 *              bonus), -1 in the remaining slots.
 * n_out        int32 device scalar: n + 1, in [1, gamma + 1].
 * margins_or_null  [gamma+1] fp32 device: top1 - top2 of each row (0 on a
 *              tie at the top).
 * Logits are expected finite: a row holding a NaN gets an unspecified
 * prediction and margin (no error is raised).
 * seq_len_inout_or_null  int32 device scalar; if given, n + 1 is added.
 * ------------------------------------------------------------------------ */
std_status_t std_accept(const int32_t* draft, int32_t gamma, const void* logits,
                        int32_t vocab, std_dtype_t logits_dtype, int32_t* out_tokens,
                        int32_t* n_out, float* margins_or_null,
                        int32_t* seq_len_inout_or_null, void* stream);

/* (d, batched) Acceptance for `batch` sequences, each as std_accept (the
 * cycle of Methodology item 3 runs per sequence): draft [batch][gamma],
 * logits [batch][gamma+1][vocab], out_tokens [batch][gamma+1], n_out
 * [batch], margins [batch][gamma+1] or NULL, seq_len [batch] or NULL
 * (sequence b's length advances by its own n + 1).
 * gamma_dev_or_null: NULL (every sequence drafted gamma tokens) or [batch]
 * int32 device holding each sequence's own draft length gamma_b, clamped
 * into [0, gamma]; gamma is then the row stride of draft, logits and
 * out_tokens.  Sequence b reads draft[b][0..gamma_b) and logit rows
 * [b][0..gamma_b] only; n_b <= gamma_b; out_tokens[b][0..n_b] = its
 * predictions, -1 in the remaining slots up to gamma; margins of rows past
 * gamma_b are NaN.  batch = 1 with NULL is std_accept. */
std_status_t std_accept_batch(const int32_t* draft, int32_t gamma, int32_t batch,
                              const int32_t* gamma_dev_or_null, const void* logits, int32_t vocab,
                              std_dtype_t logits_dtype, int32_t* out_tokens, int32_t* n_out,
                              float* margins_or_null, int32_t* seq_len_inout_or_null,
                              void* stream);

/* ------------------------------------------------------------------------
 * Prefill attention of the text rows, returning their normalisers.
 *
 * The selection (a) starts from each text row's causal softmax normaliser
 * (Technical summary, Methodology item 4: the top-K come from the average
 * attention of the text tokens to the visual tokens, taken at prefill).
 * The prefill computes those rows' attention anyway, so this call does it
 * and returns the normaliser beside the output; passed as lse_or_null to
 * std_select_topk, it spares the selection its first pass.
 *
 * Text row i (position text_start + i) of query head h (KV head
 * h / (n_q_heads / n_kv_heads)) attends with softmax over keys
 * [0, text_start + i]:
 *   out[h][i]  = sum_j softmax_j(scale * q_text[h][i] . k[g][j]) v[g][j]
 *   lse[h][i]  = log sum_j exp(scale * q_text[h][i] . k[g][j])   (natural log)
 *
 * q_text      [n_q_heads][n_text][head_dim] bf16 device, 16-byte aligned.
 * kv          bf16 cache (fp32: STD_ERR_UNSUPPORTED);
 *             text_start + n_text <= kv->len.
 * out         [n_q_heads][n_text][head_dim] bf16 device (q_text's layout).
 * lse_out_or_null  [n_q_heads][n_text] fp32 device, or NULL.
 * workspace   std_prefill_text_attn_workspace() bytes (per-chunk partials:
 *             about n_q_heads * n_text * (4 * head_dim + 12) bytes per
 *             16,384 keys).
 * Errors: STD_ERR_INVALID_ARGUMENT before any launch for null pointers,
 * misalignment, text_start < 0, n_text < 1 or rows past kv->len.
 * ------------------------------------------------------------------------ */
size_t std_prefill_text_attn_workspace(const std_attn_shape_t* shape, int32_t text_start,
                                       int32_t n_text);
std_status_t std_prefill_text_attn(const std_attn_shape_t* shape, const void* q_text,
                                   int32_t text_start, int32_t n_text, const std_kv_t* kv,
                                   void* out, float* lse_out_or_null, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Index-list check (debug aid for (b)).
 *
 * The sparse draft calls take, per KV head, selected visual positions
 * (Technical summary, Methodology item 4: top-K over the visual KV) inside
 * the span, ascending, without repeats, and do not verify this on the
 * device (they clamp each position into the span).  This call counts the
 * entries of idx [n_kv_heads][topk] (int32 device) that lie outside
 * [vis_start, vis_start + vis_len) or are not larger than the previous
 * entry of the same head, and writes the count to bad_out (int32 device
 * scalar; 0 = the list meets every precondition).  topk = 0 writes 0.
 * Errors: STD_ERR_INVALID_ARGUMENT before any launch for a null pointer,
 * n_kv_heads < 1, a bad span or topk outside [0, vis_len].
 * ------------------------------------------------------------------------ */
std_status_t std_check_idx(const int32_t* idx, int32_t n_kv_heads, int32_t topk, std_vis_t vis,
                           int32_t* bad_out, void* stream);

/* ------------------------------------------------------------------------
 * Index lists of the streaming-attention comparator.
 *
 * The pages compare StD with a streaming-attention draft that accepts fewer
 * drafts (technical summary, Experimental results).  Such a policy keeps a
 * few initial "sink" positions and a window of the most recent ones instead
 * of ranking positions by attention.  Applied to the visual span only (the
 * text KV stays whole, as in the StD draft), it is a fixed index list for
 * the sparse draft calls; this call writes it:
 *   idx_out[g] = vis_start + 0 .. vis_start + s - 1,
 *                vis_start + vis_len - (topk - s) .. vis_start + vis_len - 1
 * with s = min(sink, topk), the same for every KV head g, ascending and
 * distinct (topk <= vis_len), i.e. a valid list for std_sparse_decode_attn.
 * The pages give no sink or window size; the caller chooses them.
 *
 * idx_out  [n_kv_heads][topk] int32 device.  topk = 0 writes nothing.
 * Errors: STD_ERR_INVALID_ARGUMENT before any launch for n_kv_heads < 1, a
 * bad span, topk outside [0, vis_len], sink < 0 or a null idx_out.
 * ------------------------------------------------------------------------ */
std_status_t std_static_window_idx(int32_t n_kv_heads, std_vis_t vis, int32_t sink, int32_t topk,
                                   int32_t* idx_out, void* stream);

/* ------------------------------------------------------------------------
 * Streaming-read probe (measurement harness; no step of the method).
 *
 * The sparse draft and dense verify calls are bound by HBM bandwidth
 * (Technical summary, Methodology item 2: the sparse mode cuts draft-phase
 * I/O; the verify pass reads the full cache once).  This call reads
 * [buf, buf + bytes) once with a fixed grid of 256 workgroups x 256 lanes
 * in 16 KB tiles (tile t to workgroup t mod 256), with non-temporal 16-byte
 * loads, and does nothing else, so
 * timing it on a buffer larger than the 256 MB last-level cache gives the
 * read bandwidth this part attains, the yardstick beside the nominal peak.
 *
 * buf    device, 16-byte aligned; bytes a positive multiple of 16.
 * sink   [STD_PROBE_SINK_WORDS] uint32 device, 4-byte aligned: lane l of
 *        workgroup w writes word 256 w + l, the XOR of every 32-bit word
 *        it loaded (16-byte element e belongs to tile e / 1024, load
 *        (e mod 1024) / 256, lane e mod 256).  The digest only keeps the
 *        loads alive; tests use it to check that every byte was read once.
 * Errors: STD_ERR_INVALID_ARGUMENT for a null pointer, misalignment or a
 * bad size, before any launch.
 * ------------------------------------------------------------------------ */
#define STD_PROBE_SINK_WORDS 65536
std_status_t std_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STDSPEC_H */
