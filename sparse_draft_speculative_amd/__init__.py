"""Sparse-to-Dense (StD) speculative decoding hot path for MI355X (gfx950).

The four calls of the hot path are hand-written HIP kernels behind the C ABI
of libstdspec.so (include/stdspec.h); this package is the thin Python
binding over it (torch supplies device memory and the HIP stream):

  std_select_topk         prefill-time top-K visual KV selection
  std_sparse_decode_attn  sparse draft attention (one query token)
  std_dense_verify_attn   dense verify attention (gamma+1 queries, full KV)
  std_accept              greedy longest-prefix acceptance + bonus token

std_prefill_text_attn computes the prefill attention of the text rows and
returns their softmax normalisers, which std_select_topk accepts in place of
its own first pass.

std_sparse_decode_attn_dlen / std_dense_verify_attn_dlen read the valid
cache length from device memory, so a whole draft-verify cycle can be
captured once and replayed; std_sparse_decode_attn_batch,
std_dense_verify_attn_batch and std_accept_batch run the three decode steps
for several independent sequences, one launch each (each sequence with its
own valid length and, optionally, its own draft length).
std_sparse_decode_attn_noalloc is the draft call for callers that cannot
allocate: its partials live in scratch memory the library owns.
std_static_window_idx writes the index lists of the streaming-attention
comparator (attention sink + recent window over the visual span) for the
same draft calls.  std_check_idx counts index-list entries that break the
draft call's preconditions (a debug aid).  std_hbm_read_probe
is measurement harness: a plain streaming read that gives the attainable
HBM bandwidth the HBM-bound kernels are compared with.

Importing this package does not load the library; the first call does, and
fails loudly if it has not been built.
"""

from ._lib import (  # noqa: F401
    StdError, load, attn_shape, kv_desc,
    std_select_topk, std_select_topk_workspace,
    std_sparse_decode_attn, std_sparse_decode_workspace, std_sparse_decode_attn_dlen,
    std_sparse_decode_attn_batch, std_sparse_decode_batch_workspace,
    std_sparse_decode_attn_noalloc,
    std_dense_verify_attn, std_dense_verify_workspace, std_dense_verify_attn_dlen,
    std_accept, std_accept_batch, std_dense_verify_attn_batch, std_dense_verify_batch_workspace,
    std_check_idx, std_hbm_read_probe, std_static_window_idx,
    std_prefill_text_attn, std_prefill_text_attn_workspace,
    PreparedCall, prepare_dense_verify, prepare_sparse_decode, prepare_select_topk,
    prepare_accept, prepare_dense_verify_dlen, prepare_sparse_decode_dlen,
    prepare_prefill_text_attn, prepare_sparse_decode_batch, prepare_dense_verify_batch,
    prepare_accept_batch,
)
