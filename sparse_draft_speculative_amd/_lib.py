"""ctypes binding of libstdspec (the gfx950 HIP library); marshalling only.

Each function has the name of the C entry point it wraps (include/stdspec.h),
takes torch tensors that live on the GPU, passes their device pointers and
torch's current HIP stream, and raises StdError on a non-OK status.  Every
step of the computation runs in the HIP kernels; there is no fallback: if
the library is missing, loading fails with an error.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstdspec.so")

STD_OK = 0
STD_ERR_INVALID_ARGUMENT = 1
STD_ERR_UNSUPPORTED = 2
STD_ERR_WORKSPACE_TOO_SMALL = 3
STD_ERR_HIP = 4
STD_DTYPE_F32 = 0
STD_DTYPE_BF16 = 1


class StdError(RuntimeError):
    def __init__(self, status, name, detail):
        super().__init__(f"{name}: {detail}")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float)]


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("capacity", ctypes.c_int32), ("len", ctypes.c_int32),
                ("dtype", ctypes.c_int)]


class Vis(ctypes.Structure):
    _fields_ = [("vis_start", ctypes.c_int32), ("vis_len", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_SIGS = {
    "std_abi_version": (_I, []),
    "std_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "std_last_error": (ctypes.c_char_p, []),
    "std_dense_verify_workspace": (_SZ, [ctypes.POINTER(AttnShape), _I, ctypes.POINTER(KV)]),
    "std_dense_verify_attn": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P, _I,
                                             ctypes.POINTER(KV), _P, _P, _SZ, _P]),
    "std_dense_verify_attn_dlen": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P, _I,
                                                  ctypes.POINTER(KV), _P, _I, _P, _P, _SZ, _P]),
    "std_sparse_decode_workspace": (_SZ, [ctypes.POINTER(AttnShape), ctypes.POINTER(KV), Vis, _I]),
    "std_sparse_decode_attn_dlen": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P,
                                                   ctypes.POINTER(KV), _P, _I, Vis, _P, _I, _P,
                                                   _P, _SZ, _P]),
    "std_sparse_decode_attn": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P, ctypes.POINTER(KV),
                                              Vis, _P, _I, _P, _P, _SZ, _P]),
    "std_sparse_decode_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P,
                                                      ctypes.POINTER(KV), _P, _I, Vis, _P, _I,
                                                      _P, _P]),
    "std_sparse_decode_batch_workspace": (_SZ, [ctypes.POINTER(AttnShape), _I,
                                                ctypes.POINTER(KV), Vis, _I]),
    "std_sparse_decode_attn_batch": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P, _I,
                                                    ctypes.POINTER(KV), _P, _I, Vis, _P, _I, _P,
                                                    _I, _P, _P, _SZ, _P]),
    "std_select_topk_workspace": (_SZ, [ctypes.POINTER(AttnShape), _I, Vis, _I,
                                        ctypes.POINTER(KV)]),
    "std_select_topk": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P, _I, _I,
                                       ctypes.POINTER(KV), Vis, _I, _P, _P, _P, _P, _SZ, _P]),
    "std_accept": (ctypes.c_int, [_P, _I, _P, _I, ctypes.c_int, _P, _P, _P, _P, _P]),
    "std_hbm_read_probe": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "std_dense_verify_batch_workspace": (_SZ, [ctypes.POINTER(AttnShape), _I, _I,
                                               ctypes.POINTER(KV)]),
    "std_dense_verify_attn_batch": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P, _I, _I,
                                                   ctypes.POINTER(KV), _P, _I, _P, _P, _SZ, _P]),
    "std_accept_batch": (ctypes.c_int, [_P, _I, _I, _P, _P, _I, ctypes.c_int, _P, _P, _P, _P,
                                        _P]),
    "std_static_window_idx": (ctypes.c_int, [_I, Vis, _I, _I, _P, _P]),
    "std_check_idx": (ctypes.c_int, [_P, _I, _I, Vis, _P, _P]),
    "std_prefill_text_attn_workspace": (_SZ, [ctypes.POINTER(AttnShape), _I, _I]),
    "std_prefill_text_attn": (ctypes.c_int, [ctypes.POINTER(AttnShape), _P, _I, _I,
                                             ctypes.POINTER(KV), _P, _P, _P, _SZ, _P]),
}

PROBE_SINK_WORDS = 65536

_lib = None


def load():
    """Load libstdspec.so (built by sparse_draft_speculative_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_draft_speculative_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status, name):
    if status != STD_OK:
        lib = load()
        raise StdError(status, lib.std_status_str(status).decode(),
                       f"{name}: {lib.std_last_error().decode()}")


def _dtype_code(t):
    if t.dtype == torch.float32:
        return STD_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return STD_DTYPE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _tensor(t, name, dtype=None, shape=None, min_numel=None):
    """A contiguous tensor with the given dtype / exact shape / size.

    Every wrapper and prepare_* helper validates its tensors here before a
    pointer reaches the library (the C calls read and write exactly the
    sizes implied by the shapes they are given); the device is checked
    afterwards (_gpu), so a caller sees the specific mismatch first."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError(f"{name} must be {' or '.join(str(a) for a in allowed)}, "
                             f"got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, "
                         f"got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")
    return t


def _gpu(**tensors):
    """Every given (non-None) tensor lives on the GPU."""
    for name, t in tensors.items():
        if t is not None:
            _dev(t, name)


_KV_DTYPES = (torch.float32, torch.bfloat16)


def _check_cache(k, v, dims, name="k"):
    """k (and v, same shape and dtype): a [..][H_kv][capacity][d] cache of
    ``dims`` dimensions in fp32 or bf16 with d 64 or 128 (the library
    reports other head sizes as unsupported)."""
    _tensor(k, name, _KV_DTYPES)
    if k.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {k.dim()}")
    if v is not None:
        _tensor(v, "v", k.dtype, k.shape)
    return k.shape[-1]


def _check_queries(q, k, dims, d, name="q"):
    _tensor(q, name, k.dtype)
    if q.dim() != dims or q.shape[-1] != d:
        raise ValueError(f"{name} must have {dims} dimensions ending in head_dim {d}, "
                         f"got {tuple(q.shape)}")
    return q


def _check_out(out, like, name="out"):
    return _tensor(out, name, like.dtype, like.shape)


def _check_len_dev(len_dev, n):
    if len_dev is not None:
        _tensor(len_dev, "len_dev", torch.int32, min_numel=n)
        if n > 1 and len_dev.numel() != n:
            raise ValueError(f"len_dev must hold {n} int32 lengths")
        _gpu(len_dev=len_dev)


def _check_gamma_dev(gamma_dev, n):
    if gamma_dev is not None:
        _tensor(gamma_dev, "gamma_dev", torch.int32, (n,))
        _gpu(gamma_dev=gamma_dev)


def _check_accept_io(draft, logits, gamma_rows, lead, out_tokens, n_out, margins, seq_len):
    """draft [*lead][gamma]; logits [*lead][gamma+1][vocab]; outputs sized
    for every sequence of the batch."""
    _tensor(draft, "draft", torch.int32, (*lead, gamma_rows - 1))
    _tensor(logits, "logits", _KV_DTYPES)
    if logits.dim() != len(lead) + 2 or tuple(logits.shape[:-1]) != (*lead, gamma_rows):
        raise ValueError(f"logits must be {(*lead, gamma_rows)} x vocab, got "
                         f"{tuple(logits.shape)}")
    nb = 1
    for x in lead:
        nb *= int(x)
    if out_tokens is not None:
        _tensor(out_tokens, "out_tokens", torch.int32, (*lead, gamma_rows))
    if n_out is not None:
        _tensor(n_out, "n_out", torch.int32, min_numel=nb)
    if margins is not None:
        _tensor(margins, "margins", torch.float32, (*lead, gamma_rows))
    if seq_len is not None:
        _tensor(seq_len, "seq_len", torch.int32, min_numel=nb)
    _gpu(draft=draft, logits=logits, out_tokens=out_tokens, n_out=n_out, margins=margins,
         seq_len=seq_len)


def _nbytes(t):
    return t.numel() * t.element_size()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def attn_shape(n_q_heads, n_kv_heads, head_dim, scale=None):
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return AttnShape(n_q_heads, n_kv_heads, head_dim, scale)


def kv_desc(k, v, length):
    return KV(k.data_ptr() if k is not None else 0, v.data_ptr() if v is not None else 0,
              k.shape[1], int(length), _dtype_code(k))


def _workspace(nbytes, device, workspace):
    # the library needs no initialised workspace; zero-filled for tidiness
    if workspace is None:
        return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace")
    return workspace


def _ws_bytes(ws):
    return _nbytes(ws)


# ----------------------------------------------------------------------------
# Validated argument sets, shared by the wrappers and the prepare_* helpers.

def _dense_args(q, k, v, out, batched=False):
    """q [B?][n_q][H_q][d]; k, v [B?][H_kv][capacity][d]; out like q."""
    lead = 1 if batched else 0
    d = _check_cache(k, v, 3 + lead)
    _check_queries(q, k, 3 + lead, d)
    if batched and q.shape[0] != k.shape[0]:
        raise ValueError(f"q and k must hold the same batch ({q.shape[0]} vs {k.shape[0]})")
    if out is not None:
        _check_out(out, q)
    _gpu(q=q, k=k, v=v, out=out)
    return d


def _sparse_args(q, k, v, idx, out, batched=False):
    """q [B?][H_q][d]; k, v [B?][H_kv][capacity][d]; idx [B?][H_kv][K] int32."""
    lead = 1 if batched else 0
    d = _check_cache(k, v, 3 + lead)
    _check_queries(q, k, 2 + lead, d)
    hkv = k.shape[lead]
    _tensor(idx, "idx", torch.int32)
    if idx.dim() != 2 + lead or idx.shape[lead] != hkv or (batched and idx.shape[0] != q.shape[0]):
        want = "[B][H_kv][K]" if batched else "[H_kv][K]"
        raise ValueError(f"idx must be {want} with H_kv = {hkv}, got {tuple(idx.shape)}")
    if batched and k.shape[0] != q.shape[0]:
        raise ValueError(f"q and k must hold the same batch ({q.shape[0]} vs {k.shape[0]})")
    if out is not None:
        _check_out(out, q)
    _gpu(q=q, k=k, v=v, idx=idx, out=out)
    return d


def _select_args(q_text, k, idx_out, scores_out, lse, vis_len, topk):
    d = _check_cache(k, None, 3)
    _check_queries(q_text, k, 3, d, "q_text")
    hq, n_text = q_text.shape[0], q_text.shape[1]
    hkv = k.shape[0]
    if idx_out is not None:
        _tensor(idx_out, "idx_out", torch.int32, (hkv, topk))
    if scores_out is not None:
        _tensor(scores_out, "scores_out", torch.float32, (hkv, vis_len))
    if lse is not None:
        _tensor(lse, "lse", torch.float32)
        if lse.numel() != hq * n_text:
            raise ValueError(f"lse must hold H_q * n_text = {hq * n_text} float32 values")
    _gpu(q_text=q_text, k=k, idx_out=idx_out, scores_out=scores_out, lse=lse)
    return d


def _prefill_args(q_text, k, v, out, lse_out):
    d = _check_cache(k, v, 3)
    _check_queries(q_text, k, 3, d, "q_text")
    if out is not None:
        _check_out(out, q_text)
    if lse_out is not None:
        _tensor(lse_out, "lse_out", torch.float32)
        if lse_out.numel() != q_text.shape[0] * q_text.shape[1]:
            raise ValueError("lse_out must be [H_q][n_text] float32")
    _gpu(q_text=q_text, k=k, v=v, out=out, lse_out=lse_out)
    return d


# ----------------------------------------------------------------------------
def std_dense_verify_workspace(shape, n_q, k, length):
    return load().std_dense_verify_workspace(ctypes.byref(shape), int(n_q),
                                             ctypes.byref(kv_desc(k, None, length)))


def std_dense_verify_attn(q, k, v, length, out=None, scale=None, workspace=None, stream=None):
    """Dense verify attention.  q [n_q][H_q][d]; k, v [H_kv][capacity][d]."""
    lib = load()
    _dense_args(q, k, v, out)
    n_q, hq, d = q.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, length)
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(lib.std_dense_verify_workspace(ctypes.byref(shape), n_q, ctypes.byref(kv)),
                    q.device, workspace)
    _check(lib.std_dense_verify_attn(ctypes.byref(shape), _ptr(q), n_q, ctypes.byref(kv),
                                     _ptr(out), _ptr(ws), _ws_bytes(ws), _stream(stream)),
           "std_dense_verify_attn")
    return out


def std_dense_verify_batch_workspace(shape, n_q, batch, k, length):
    """Workspace bytes of std_dense_verify_attn_batch; k [B][H_kv][capacity][d]."""
    kv = KV(k.data_ptr(), 0, k.shape[2], int(length), _dtype_code(k))
    return load().std_dense_verify_batch_workspace(ctypes.byref(shape), int(n_q), int(batch),
                                                   ctypes.byref(kv))


def std_dense_verify_attn_batch(q, k, v, max_len, len_dev=None, len_offset=0, out=None,
                                scale=None, workspace=None, stream=None):
    """Dense verify for B sequences in one launch.  q [B][n_q][H_q][d];
    k, v [B][H_kv][capacity][d]; len_dev None (every sequence has length
    max_len) or [B] int32 device lengths: min(max(len_dev[b] + len_offset, n_q),
    max_len)."""
    lib = load()
    _check_len_dev(len_dev, q.shape[0])
    _dense_args(q, k, v, out, batched=True)
    B, n_q, hq, d = q.shape
    shape = attn_shape(hq, k.shape[1], d, scale)
    kv = KV(k.data_ptr(), v.data_ptr(), k.shape[2], int(max_len), _dtype_code(k))
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(std_dense_verify_batch_workspace(shape, n_q, B, k, max_len), q.device,
                    workspace)
    _check(lib.std_dense_verify_attn_batch(ctypes.byref(shape), _ptr(q), n_q, B, ctypes.byref(kv),
                                           _ptr(len_dev), int(len_offset), _ptr(out), _ptr(ws),
                                           _ws_bytes(ws), _stream(stream)),
           "std_dense_verify_attn_batch")
    return out


def std_dense_verify_attn_dlen(q, k, v, max_len, len_dev, len_offset, out=None, scale=None,
                               workspace=None, stream=None):
    """Dense verify with the valid length read on the device:
    min(max(len_dev[0] + len_offset, n_q), max_len)."""
    lib = load()
    _check_len_dev(len_dev, 1)
    _dense_args(q, k, v, out)
    n_q, hq, d = q.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, max_len)
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(lib.std_dense_verify_workspace(ctypes.byref(shape), n_q, ctypes.byref(kv)),
                    q.device, workspace)
    _check(lib.std_dense_verify_attn_dlen(ctypes.byref(shape), _ptr(q), n_q, ctypes.byref(kv),
                                          _ptr(len_dev), int(len_offset), _ptr(out), _ptr(ws),
                                          _ws_bytes(ws), _stream(stream)),
           "std_dense_verify_attn_dlen")
    return out


def std_sparse_decode_workspace(shape, k, length, vis_start, vis_len, topk):
    return load().std_sparse_decode_workspace(ctypes.byref(shape),
                                              ctypes.byref(kv_desc(k, None, length)),
                                              Vis(vis_start, vis_len), int(topk))


def std_sparse_decode_attn(q, k, v, length, vis_start, vis_len, idx, out=None, scale=None,
                           workspace=None, stream=None):
    """Sparse draft attention.  q [H_q][d]; idx [H_kv][K] int32 (K may be 0)."""
    lib = load()
    _sparse_args(q, k, v, idx, out)
    hq, d = q.shape
    hkv = k.shape[0]
    topk = idx.shape[1]
    shape = attn_shape(hq, hkv, d, scale)
    kv = kv_desc(k, v, length)
    vis = Vis(vis_start, vis_len)
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(lib.std_sparse_decode_workspace(ctypes.byref(shape), ctypes.byref(kv), vis,
                                                    topk), q.device, workspace)
    _check(lib.std_sparse_decode_attn(ctypes.byref(shape), _ptr(q), ctypes.byref(kv), vis,
                                      _ptr(idx), topk, _ptr(out), _ptr(ws), _ws_bytes(ws),
                                      _stream(stream)),
           "std_sparse_decode_attn")
    return out


def std_sparse_decode_attn_dlen(q, k, v, max_len, len_dev, len_offset, vis_start, vis_len, idx,
                                out=None, scale=None, workspace=None, stream=None):
    """Sparse draft attention with the valid length read on the device:
    min(max(len_dev[0] + len_offset, lo), max_len), lo = vis_start + vis_len
    (+1 with neither a prefix nor a selected position)."""
    lib = load()
    _check_len_dev(len_dev, 1)
    _sparse_args(q, k, v, idx, out)
    hq, d = q.shape
    hkv = k.shape[0]
    topk = idx.shape[1]
    shape = attn_shape(hq, hkv, d, scale)
    kv = kv_desc(k, v, max_len)
    vis = Vis(vis_start, vis_len)
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(lib.std_sparse_decode_workspace(ctypes.byref(shape), ctypes.byref(kv), vis,
                                                    topk), q.device, workspace)
    _check(lib.std_sparse_decode_attn_dlen(ctypes.byref(shape), _ptr(q), ctypes.byref(kv),
                                           _ptr(len_dev), int(len_offset), vis, _ptr(idx), topk,
                                           _ptr(out), _ptr(ws), _ws_bytes(ws), _stream(stream)),
           "std_sparse_decode_attn_dlen")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20


def std_sparse_decode_attn_noalloc(q, k, v, length, vis_start, vis_len, idx, len_dev=None,
                                   len_offset=0, out=None, scale=None, stream=None):
    """Sparse draft attention with its partials in the library's own scratch
    (no workspace; for callers that cannot allocate).  len_dev None: length
    ``length``; else min(max(len_dev[0] + len_offset, lo), length) as in
    std_sparse_decode_attn_dlen.  Calls overlapping on one GPU race."""
    lib = load()
    _check_len_dev(len_dev, 1)
    _sparse_args(q, k, v, idx, out)
    hq, d = q.shape
    hkv = k.shape[0]
    topk = idx.shape[1]
    shape = attn_shape(hq, hkv, d, scale)
    kv = kv_desc(k, v, length)
    if out is None:
        out = torch.empty_like(q)
    _check(lib.std_sparse_decode_attn_noalloc(ctypes.byref(shape), _ptr(q), ctypes.byref(kv),
                                              _ptr(len_dev), int(len_offset),
                                              Vis(vis_start, vis_len), _ptr(idx), topk,
                                              _ptr(out), _stream(stream)),
           "std_sparse_decode_attn_noalloc")
    return out


def std_sparse_decode_batch_workspace(shape, batch, k, length, vis_start, vis_len, topk):
    """Workspace bytes of std_sparse_decode_attn_batch; k [B][H_kv][capacity][d]."""
    kv = KV(k.data_ptr(), 0, k.shape[2], int(length), _dtype_code(k))
    return load().std_sparse_decode_batch_workspace(ctypes.byref(shape), int(batch),
                                                    ctypes.byref(kv), Vis(vis_start, vis_len),
                                                    int(topk))


def std_sparse_decode_attn_batch(q, k, v, max_len, vis_start, vis_len, idx, len_dev=None,
                                 len_offset=0, gamma_dev=None, step=0, out=None, scale=None,
                                 workspace=None, stream=None):
    """Sparse draft attention for B sequences in one launch.

    q [B][H_q][d]; k, v [B][H_kv][capacity][d]; idx [B][H_kv][K] int32;
    len_dev None (every sequence has length max_len) or [B] int32 device
    lengths, sequence b using min(max(len_dev[b] + len_offset, lo), max_len).
    gamma_dev None or [B] int32 device draft lengths: the call is draft step
    ``step`` and sequence b takes part only while step < gamma_dev[b] (the
    others' rows of ``out`` are left as they were).
    """
    lib = load()
    B = q.shape[0]
    _check_len_dev(len_dev, B)
    _check_gamma_dev(gamma_dev, B)
    _sparse_args(q, k, v, idx, out, batched=True)
    B, hq, d = q.shape
    hkv, cap = k.shape[1], k.shape[2]
    topk = idx.shape[2]
    shape = attn_shape(hq, hkv, d, scale)
    kv = KV(k.data_ptr(), v.data_ptr(), cap, int(max_len), _dtype_code(k))
    vis = Vis(vis_start, vis_len)
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(lib.std_sparse_decode_batch_workspace(ctypes.byref(shape), B,
                                                          ctypes.byref(kv), vis, topk),
                    q.device, workspace)
    _check(lib.std_sparse_decode_attn_batch(ctypes.byref(shape), _ptr(q), B, ctypes.byref(kv),
                                            _ptr(len_dev), int(len_offset), vis, _ptr(idx), topk,
                                            _ptr(gamma_dev), int(step), _ptr(out), _ptr(ws),
                                            _ws_bytes(ws), _stream(stream)),
           "std_sparse_decode_attn_batch")
    return out


def std_select_topk_workspace(shape, n_text, vis_start, vis_len, topk, k, length):
    return load().std_select_topk_workspace(ctypes.byref(shape), int(n_text),
                                            Vis(vis_start, vis_len), int(topk),
                                            ctypes.byref(kv_desc(k, None, length)))


def std_select_topk(q_text, k, length, text_start, vis_start, vis_len, topk, lse=None,
                    idx_out=None, scores_out=None, scale=None, workspace=None, stream=None,
                    want_scores=False):
    """Top-K visual KV selection.  q_text [H_q][n_text][d]; k [H_kv][capacity][d].

    Returns idx [H_kv][topk] int32 (and the fp32 scores if want_scores).
    """
    lib = load()
    _select_args(q_text, k, idx_out, scores_out, lse, vis_len, topk)
    hq, n_text, d = q_text.shape
    hkv = k.shape[0]
    shape = attn_shape(hq, hkv, d, scale)
    kv = kv_desc(k, k, length)
    vis = Vis(vis_start, vis_len)
    if idx_out is None:
        idx_out = torch.empty(hkv, topk, dtype=torch.int32, device=k.device)
    if scores_out is None and want_scores:
        scores_out = torch.empty(hkv, vis_len, dtype=torch.float32, device=k.device)
    ws = _workspace(lib.std_select_topk_workspace(ctypes.byref(shape), n_text, vis, topk,
                                                  ctypes.byref(kv)), k.device, workspace)
    _check(lib.std_select_topk(ctypes.byref(shape), _ptr(q_text), text_start, n_text,
                               ctypes.byref(kv), vis, topk, _ptr(lse), _ptr(idx_out),
                               _ptr(scores_out), _ptr(ws), _ws_bytes(ws), _stream(stream)),
           "std_select_topk")
    return (idx_out, scores_out) if want_scores else idx_out


def std_accept(draft, logits, out_tokens=None, n_out=None, margins=None, seq_len=None,
               stream=None):
    """Greedy acceptance.  draft [gamma] int32; logits [gamma+1][vocab].

    Returns (out_tokens [gamma+1] int32, n_out [1] int32) on the device.
    """
    lib = load()
    _tensor(draft, "draft", torch.int32)
    if draft.dim() != 1:
        raise ValueError("draft must be [gamma] int32")
    gamma = draft.numel()
    _check_accept_io(draft, logits, gamma + 1, (), out_tokens, n_out, margins, seq_len)
    vocab = logits.shape[1]
    dev = logits.device
    if out_tokens is None:
        out_tokens = torch.empty(gamma + 1, dtype=torch.int32, device=dev)
    if n_out is None:
        n_out = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.std_accept(_ptr(draft), gamma, _ptr(logits), vocab, _dtype_code(logits),
                          _ptr(out_tokens), _ptr(n_out), _ptr(margins), _ptr(seq_len),
                          _stream(stream)),
           "std_accept")
    return out_tokens, n_out


def std_accept_batch(draft, logits, out_tokens=None, n_out=None, margins=None, seq_len=None,
                     gamma_dev=None, stream=None):
    """Greedy acceptance for B sequences.  draft [B][gamma] int32; logits
    [B][gamma+1][vocab].  gamma_dev None or [B] int32 device draft lengths
    (each clamped into [0, gamma]; gamma is then the row stride).  Returns
    (out_tokens [B][gamma+1], n_out [B])."""
    lib = load()
    _tensor(draft, "draft", torch.int32)
    if draft.dim() != 2:
        raise ValueError("draft must be [B][gamma] int32")
    B, gamma = draft.shape
    _check_gamma_dev(gamma_dev, B)
    _check_accept_io(draft, logits, gamma + 1, (B,), out_tokens, n_out, margins, seq_len)
    vocab = logits.shape[2]
    dev = logits.device
    if out_tokens is None:
        out_tokens = torch.empty(B, gamma + 1, dtype=torch.int32, device=dev)
    if n_out is None:
        n_out = torch.empty(B, dtype=torch.int32, device=dev)
    _check(lib.std_accept_batch(_ptr(draft), gamma, B, _ptr(gamma_dev), _ptr(logits), vocab,
                                _dtype_code(logits), _ptr(out_tokens), _ptr(n_out),
                                _ptr(margins), _ptr(seq_len), _stream(stream)),
           "std_accept_batch")
    return out_tokens, n_out


def std_prefill_text_attn_workspace(shape, text_start, n_text):
    return load().std_prefill_text_attn_workspace(ctypes.byref(shape), int(text_start),
                                                  int(n_text))


def std_prefill_text_attn(q_text, k, v, length, text_start, out=None, lse_out=None,
                          want_lse=True, scale=None, workspace=None, stream=None):
    """Prefill attention of the text rows: q_text [H_q][n_text][d] bf16 (text
    row i at position text_start + i) over the causal keys of the cache
    k, v [H_kv][capacity][d] (valid length ``length``).  Returns
    (out [H_q][n_text][d] bf16, lse [H_q][n_text] fp32 natural log or None)."""
    lib = load()
    _prefill_args(q_text, k, v, out, lse_out)
    hq, n_text, d = q_text.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, length)
    if out is None:
        out = torch.empty_like(q_text)
    if lse_out is None and want_lse:
        lse_out = torch.empty(hq, n_text, dtype=torch.float32, device=q_text.device)
    ws = _workspace(lib.std_prefill_text_attn_workspace(ctypes.byref(shape), text_start, n_text),
                    q_text.device, workspace)
    _check(lib.std_prefill_text_attn(ctypes.byref(shape), _ptr(q_text), int(text_start),
                                     int(n_text), ctypes.byref(kv), _ptr(out), _ptr(lse_out),
                                     _ptr(ws), _ws_bytes(ws), _stream(stream)),
           "std_prefill_text_attn")
    return out, lse_out


def std_static_window_idx(n_kv_heads, vis_start, vis_len, sink, topk, idx_out=None,
                          device="cuda", stream=None):
    """Index lists of the streaming-attention comparator: for each of the
    n_kv_heads heads the first min(sink, topk) visual positions and the last
    topk - min(sink, topk), ascending.  Returns idx [H_kv][topk] int32."""
    lib = load()
    if idx_out is None:
        idx_out = torch.empty(int(n_kv_heads), int(topk), dtype=torch.int32, device=device)
    _tensor(idx_out, "idx_out", torch.int32, (n_kv_heads, topk))
    _gpu(idx_out=idx_out)
    _check(lib.std_static_window_idx(int(n_kv_heads), Vis(vis_start, vis_len), int(sink),
                                     int(topk), _ptr(idx_out), _stream(stream)),
           "std_static_window_idx")
    return idx_out


def std_check_idx(idx, vis_start, vis_len, bad_out=None, stream=None):
    """Count the entries of idx [H_kv][K] int32 (device) outside the visual
    span or not above the previous entry of their head.  Returns the count
    as a [1] int32 device tensor (0: the list meets every precondition)."""
    lib = load()
    _tensor(idx, "idx", torch.int32)
    if idx.dim() != 2:
        raise ValueError("idx must be [H_kv][K] int32")
    if bad_out is None:
        bad_out = torch.empty(1, dtype=torch.int32, device=idx.device)
    _tensor(bad_out, "bad_out", torch.int32, min_numel=1)
    _gpu(idx=idx, bad_out=bad_out)
    _check(lib.std_check_idx(_ptr(idx), idx.shape[0], idx.shape[1], Vis(vis_start, vis_len),
                             _ptr(bad_out), _stream(stream)),
           "std_check_idx")
    return bad_out


def std_hbm_read_probe(buf, sink=None, stream=None):
    """Streaming-read probe: read every byte of the device tensor ``buf``
    once (size a multiple of 16 bytes).  Returns the [65536] int32 digest
    (the bit patterns of the C call's uint32 words)."""
    lib = load()
    _dev(buf, "buf")
    if sink is None:
        sink = torch.empty(PROBE_SINK_WORDS, dtype=torch.int32, device=buf.device)
    _dev(sink, "sink")
    if _nbytes(sink) < 4 * PROBE_SINK_WORDS:
        raise ValueError(f"sink must hold {PROBE_SINK_WORDS} 32-bit words")
    _check(lib.std_hbm_read_probe(_ptr(buf), _nbytes(buf), _ptr(sink), _stream(stream)),
           "std_hbm_read_probe")
    return sink


# ----------------------------------------------------------------------------
# Prepared calls: the argument tuple is built once, so a repeated call (the
# decode loop issues a few hundred per cycle) costs one ctypes call.  Only
# the valid cache length changes between calls; it lives in the KV struct.

class PreparedCall:
    def __init__(self, name, args, kv=None, keep=()):
        self.name = name
        self.fn = getattr(load(), name)
        self.args = args
        self.kv = kv
        self._keep = keep           # keep ctypes structs and tensors alive

    def __call__(self, length=None):
        if length is not None:
            self.kv.len = int(length)
        st = self.fn(*self.args)
        if st != STD_OK:
            _check(st, self.name)


def prepare_dense_verify(q, k, v, out, workspace, stream=None, scale=None):
    _dense_args(q, k, v, out)
    _dev(workspace, "workspace")
    n_q, hq, d = q.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, k.shape[1])
    args = (ctypes.byref(shape), _ptr(q), n_q, ctypes.byref(kv), _ptr(out), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    return PreparedCall("std_dense_verify_attn", args, kv, (shape, kv, q, k, v, out, workspace))


def prepare_sparse_decode(q, k, v, vis_start, vis_len, idx, out, workspace, stream=None,
                          scale=None):
    _sparse_args(q, k, v, idx, out)
    _dev(workspace, "workspace")
    hq, d = q.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, k.shape[1])
    args = (ctypes.byref(shape), _ptr(q), ctypes.byref(kv), Vis(vis_start, vis_len), _ptr(idx),
            idx.shape[1], _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return PreparedCall("std_sparse_decode_attn", args, kv,
                        (shape, kv, q, k, v, idx, out, workspace))


def prepare_dense_verify_dlen(q, k, v, out, workspace, len_dev, len_offset, max_len=None,
                              stream=None, scale=None):
    """Prepared dense verify reading its length from len_dev (see
    std_dense_verify_attn_dlen); max_len defaults to the cache capacity."""
    _dense_args(q, k, v, out)
    _dev(workspace, "workspace")
    _check_len_dev(len_dev, 1)
    n_q, hq, d = q.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, k.shape[1] if max_len is None else max_len)
    args = (ctypes.byref(shape), _ptr(q), n_q, ctypes.byref(kv), _ptr(len_dev), int(len_offset),
            _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return PreparedCall("std_dense_verify_attn_dlen", args, kv,
                        (shape, kv, q, k, v, out, workspace, len_dev))


def prepare_sparse_decode_dlen(q, k, v, vis_start, vis_len, idx, out, workspace, len_dev,
                               len_offset, max_len=None, stream=None, scale=None):
    """Prepared sparse draft attention reading its length from len_dev."""
    _sparse_args(q, k, v, idx, out)
    _dev(workspace, "workspace")
    _check_len_dev(len_dev, 1)
    hq, d = q.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, k.shape[1] if max_len is None else max_len)
    args = (ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(len_dev), int(len_offset),
            Vis(vis_start, vis_len), _ptr(idx), idx.shape[1], _ptr(out), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    return PreparedCall("std_sparse_decode_attn_dlen", args, kv,
                        (shape, kv, q, k, v, idx, out, workspace, len_dev))


def prepare_sparse_decode_batch(q, k, v, max_len, vis_start, vis_len, idx, out, workspace,
                                len_dev=None, len_offset=0, gamma_dev=None, step=0, stream=None,
                                scale=None):
    """Prepared batched sparse draft attention (see std_sparse_decode_attn_batch)."""
    B = q.shape[0]
    _check_len_dev(len_dev, B)
    _check_gamma_dev(gamma_dev, B)
    _sparse_args(q, k, v, idx, out, batched=True)
    _dev(workspace, "workspace")
    B, hq, d = q.shape
    shape = attn_shape(hq, k.shape[1], d, scale)
    kv = KV(k.data_ptr(), v.data_ptr(), k.shape[2], int(max_len), _dtype_code(k))
    args = (ctypes.byref(shape), _ptr(q), B, ctypes.byref(kv), _ptr(len_dev), int(len_offset),
            Vis(vis_start, vis_len), _ptr(idx), idx.shape[2], _ptr(gamma_dev), int(step),
            _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return PreparedCall("std_sparse_decode_attn_batch", args, kv,
                        (shape, kv, q, k, v, idx, out, workspace, len_dev, gamma_dev))


def prepare_dense_verify_batch(q, k, v, max_len, out, workspace, len_dev=None, len_offset=0,
                               stream=None, scale=None):
    """Prepared batched dense verify (see std_dense_verify_attn_batch)."""
    _check_len_dev(len_dev, q.shape[0])
    _dense_args(q, k, v, out, batched=True)
    _dev(workspace, "workspace")
    B, n_q, hq, d = q.shape
    shape = attn_shape(hq, k.shape[1], d, scale)
    kv = KV(k.data_ptr(), v.data_ptr(), k.shape[2], int(max_len), _dtype_code(k))
    args = (ctypes.byref(shape), _ptr(q), n_q, B, ctypes.byref(kv), _ptr(len_dev),
            int(len_offset), _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return PreparedCall("std_dense_verify_attn_batch", args, kv,
                        (shape, kv, q, k, v, out, workspace, len_dev))


def prepare_prefill_text_attn(q_text, k, v, length, text_start, out, lse_out, workspace,
                              stream=None, scale=None):
    _prefill_args(q_text, k, v, out, lse_out)
    _dev(workspace, "workspace")
    hq, n_text, d = q_text.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, v, length)
    args = (ctypes.byref(shape), _ptr(q_text), int(text_start), n_text, ctypes.byref(kv),
            _ptr(out), _ptr(lse_out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return PreparedCall("std_prefill_text_attn", args, kv,
                        (shape, kv, q_text, k, v, out, lse_out, workspace))


def prepare_select_topk(q_text, k, length, text_start, vis_start, vis_len, topk, idx_out,
                        workspace, scores_out=None, lse=None, stream=None, scale=None):
    _select_args(q_text, k, idx_out, scores_out, lse, vis_len, topk)
    _dev(workspace, "workspace")
    hq, n_text, d = q_text.shape
    shape = attn_shape(hq, k.shape[0], d, scale)
    kv = kv_desc(k, k, length)
    args = (ctypes.byref(shape), _ptr(q_text), text_start, n_text, ctypes.byref(kv),
            Vis(vis_start, vis_len), topk, _ptr(lse), _ptr(idx_out), _ptr(scores_out),
            _ptr(workspace), _nbytes(workspace), _stream(stream))
    return PreparedCall("std_select_topk", args, kv,
                        (shape, kv, q_text, k, idx_out, workspace, scores_out, lse))


def prepare_accept(draft, logits, out_tokens, n_out, margins=None, seq_len=None, stream=None):
    _tensor(draft, "draft", torch.int32)
    if draft.dim() != 1:
        raise ValueError("draft must be [gamma] int32")
    gamma = draft.numel()
    _check_accept_io(draft, logits, gamma + 1, (), out_tokens, n_out, margins, seq_len)
    args = (_ptr(draft), gamma, _ptr(logits), logits.shape[1], _dtype_code(logits),
            _ptr(out_tokens), _ptr(n_out), _ptr(margins), _ptr(seq_len), _stream(stream))
    return PreparedCall("std_accept", args, None,
                        (draft, logits, out_tokens, n_out, margins, seq_len))


def prepare_accept_batch(draft, logits, out_tokens, n_out, margins=None, seq_len=None,
                         gamma_dev=None, stream=None):
    """Prepared batched acceptance (see std_accept_batch)."""
    _tensor(draft, "draft", torch.int32)
    if draft.dim() != 2:
        raise ValueError("draft must be [B][gamma] int32")
    B, gamma = draft.shape
    _check_gamma_dev(gamma_dev, B)
    _check_accept_io(draft, logits, gamma + 1, (B,), out_tokens, n_out, margins, seq_len)
    args = (_ptr(draft), gamma, B, _ptr(gamma_dev), _ptr(logits), logits.shape[2],
            _dtype_code(logits), _ptr(out_tokens), _ptr(n_out), _ptr(margins), _ptr(seq_len),
            _stream(stream))
    return PreparedCall("std_accept_batch", args, None,
                        (draft, logits, out_tokens, n_out, margins, seq_len, gamma_dev))
