"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any launch.

Every call below passes a null workspace of 0 bytes, so even a call whose
other arguments were accepted would stop at the workspace check and could
never launch a kernel.
"""

import ctypes
import os
import re

import pytest

from sparse_draft_speculative_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stdspec.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libstdspec.so not built")

FAKE = 0x10000       # a 16-byte aligned non-null address; never dereferenced


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(std_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    names = declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib._SIGS), "binding and header disagree"


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.std_abi_version() == 2
    assert lib.std_status_str(0) == b"STD_OK"
    assert lib.std_status_str(3) == b"STD_ERR_WORKSPACE_TOO_SMALL"
    assert lib.std_status_str(99) == b"STD_ERR_UNKNOWN"


def _shape(hq=28, hkv=4, d=128, scale=0.088):
    return _lib.AttnShape(hq, hkv, d, scale)


def _kv(cap=1000, length=900, dtype=_lib.STD_DTYPE_BF16, k=FAKE, v=FAKE):
    return _lib.KV(k, v, cap, length, dtype)


def _dense(shape, n_q=6, kv=None, q=FAKE, out=FAKE):
    lib = _lib.load()
    kv = kv or _kv()
    return lib.std_dense_verify_attn(ctypes.byref(shape), ctypes.c_void_p(q), n_q,
                                     ctypes.byref(kv), ctypes.c_void_p(out), None, 0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(shape=_shape(hq=28, hkv=5)), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(d=96)), _lib.STD_ERR_UNSUPPORTED),
    (dict(shape=_shape(scale=0.0)), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(scale=float("nan"))), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), n_q=0), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), n_q=901), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), kv=_kv(length=1001)), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), kv=_kv(k=0)), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), kv=_kv(dtype=7)), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), q=0), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), q=FAKE + 2), _lib.STD_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape()), _lib.STD_ERR_WORKSPACE_TOO_SMALL),
])
def test_dense_verify_rejects(kwargs, status):
    assert _dense(**kwargs) == status
    assert _lib.load().std_last_error() != b""


def test_sparse_decode_rejects():
    lib = _lib.load()
    sh = _shape()

    def call(vis=(0, 800), topk=64, idx=FAKE, kv=None):
        kv = kv or _kv()
        return lib.std_sparse_decode_attn(ctypes.byref(sh), ctypes.c_void_p(FAKE), ctypes.byref(kv),
                                          _lib.Vis(*vis), ctypes.c_void_p(idx), topk,
                                          ctypes.c_void_p(FAKE), None, 0, None)

    E = _lib.STD_ERR_INVALID_ARGUMENT
    assert call(topk=801) == E                 # K > vis_len
    assert call(topk=-1) == E
    assert call(vis=(0, 901)) == E             # span beyond len
    assert call(vis=(-1, 10)) == E
    assert call(idx=0) == E                    # K > 0 needs idx
    assert call(vis=(0, 900), topk=0) == E     # empty key set
    assert call() == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    assert call(topk=0, idx=0) == _lib.STD_ERR_WORKSPACE_TOO_SMALL   # K = 0 is legal


def test_device_length_calls_reject():
    """The device-length variants need len_dev and run the host checks of
    their host-length twins (kv->len is the bound)."""
    lib = _lib.load()
    sh = _shape()
    kv = _kv()
    E = _lib.STD_ERR_INVALID_ARGUMENT
    P = ctypes.c_void_p

    def dense(len_dev=FAKE, n_q=6):
        return lib.std_dense_verify_attn_dlen(ctypes.byref(sh), P(FAKE), n_q, ctypes.byref(kv),
                                              P(len_dev), 0, P(FAKE), None, 0, None)

    def sparse(len_dev=FAKE, topk=64):
        return lib.std_sparse_decode_attn_dlen(ctypes.byref(sh), P(FAKE), ctypes.byref(kv),
                                               P(len_dev), 1, _lib.Vis(0, 800), P(FAKE), topk,
                                               P(FAKE), None, 0, None)

    assert dense(len_dev=0) == E
    assert dense(n_q=901) == E
    assert dense() == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    assert sparse(len_dev=0) == E
    assert sparse(topk=801) == E
    assert sparse() == _lib.STD_ERR_WORKSPACE_TOO_SMALL


def test_batched_sparse_decode_rejects():
    """The batched draft call: batch in [1, 65535], bf16 with G <= 16, and
    the host checks of the single-sequence call."""
    lib = _lib.load()
    sh = _shape()
    P = ctypes.c_void_p

    def call(batch=4, kv=None, topk=64, len_dev=0, gamma_dev=0, step=0):
        kv = kv or _kv()
        return lib.std_sparse_decode_attn_batch(ctypes.byref(sh), P(FAKE), batch,
                                                ctypes.byref(kv), P(len_dev), 0,
                                                _lib.Vis(0, 800), P(FAKE), topk, P(gamma_dev),
                                                step, P(FAKE), None, 0, None)

    E = _lib.STD_ERR_INVALID_ARGUMENT
    assert call(batch=0) == E
    assert call(batch=65536) == E
    assert call(topk=801) == E
    assert call(kv=_kv(dtype=_lib.STD_DTYPE_F32)) == _lib.STD_ERR_UNSUPPORTED
    assert call() == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    assert call(len_dev=FAKE) == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    assert call(gamma_dev=FAKE, step=-1) == E            # a draft step is >= 0
    assert call(gamma_dev=FAKE, step=3) == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    assert call(batch=1, kv=_kv(dtype=_lib.STD_DTYPE_F32)) == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    one = lib.std_sparse_decode_batch_workspace(ctypes.byref(sh), 1, ctypes.byref(_kv()),
                                                _lib.Vis(0, 800), 64)
    four = lib.std_sparse_decode_batch_workspace(ctypes.byref(sh), 4, ctypes.byref(_kv()),
                                                 _lib.Vis(0, 800), 64)
    single = lib.std_sparse_decode_workspace(ctypes.byref(sh), ctypes.byref(_kv()),
                                             _lib.Vis(0, 800), 64)
    assert one == single and four > one
    assert lib.std_sparse_decode_batch_workspace(ctypes.byref(sh), 0, ctypes.byref(_kv()),
                                                 _lib.Vis(0, 800), 64) == 0


def test_select_rejects():
    lib = _lib.load()
    sh = _shape()

    def call(text_start=800, n_text=64, vis=(0, 800), topk=128, kv=None):
        kv = kv or _kv()
        return lib.std_select_topk(ctypes.byref(sh), ctypes.c_void_p(FAKE), text_start, n_text,
                                   ctypes.byref(kv), _lib.Vis(*vis), topk, None,
                                   ctypes.c_void_p(FAKE), None, None, 0, None)

    E = _lib.STD_ERR_INVALID_ARGUMENT
    assert call(text_start=799) == E           # text must follow the visual span
    assert call(n_text=0) == E
    assert call(n_text=101) == E               # beyond len 900
    assert call(topk=0) == E
    assert call(topk=801) == E
    assert call() == _lib.STD_ERR_WORKSPACE_TOO_SMALL


def test_accept_rejects():
    lib = _lib.load()
    E = _lib.STD_ERR_INVALID_ARGUMENT
    p = ctypes.c_void_p(FAKE)
    assert lib.std_accept(p, -1, p, 10, 0, p, p, None, None, None) == E
    assert lib.std_accept(p, 3, p, 0, 0, p, p, None, None, None) == E
    assert lib.std_accept(None, 3, p, 10, 0, p, p, None, None, None) == E
    assert lib.std_accept(p, 3, None, 10, 0, p, p, None, None, None) == E
    assert lib.std_accept(p, 3, p, 10, 5, p, p, None, None, None) == E


def test_prefill_text_attn_rejects():
    lib = _lib.load()
    E, U = _lib.STD_ERR_INVALID_ARGUMENT, _lib.STD_ERR_UNSUPPORTED
    sh = _shape()
    p = ctypes.c_void_p(FAKE)

    def call(q=p, text_start=100, n_text=10, kv=None, out=p, lse=None):
        kv = kv if kv is not None else _kv(length=200)
        return lib.std_prefill_text_attn(ctypes.byref(sh), q, text_start, n_text,
                                         ctypes.byref(kv), out, lse, None, 0, None)
    assert call(q=None) == E
    assert call(out=None) == E
    assert call(text_start=-1) == E
    assert call(n_text=0) == E
    assert call(text_start=195, n_text=10) == E           # rows past len
    assert call(q=ctypes.c_void_p(FAKE + 8)) == E          # misaligned
    assert call(lse=ctypes.c_void_p(FAKE + 2)) == E
    assert call(kv=_kv(length=200, dtype=_lib.STD_DTYPE_F32)) == U
    # every argument valid: stops at the empty workspace, launches nothing
    assert call() == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    assert lib.std_prefill_text_attn_workspace(ctypes.byref(sh), 100, 10) > 0
    assert lib.std_prefill_text_attn_workspace(ctypes.byref(sh), 100, 0) == 0


def test_batched_verify_and_accept_reject():
    lib = _lib.load()
    E, U = _lib.STD_ERR_INVALID_ARGUMENT, _lib.STD_ERR_UNSUPPORTED
    sh = _shape()
    p = ctypes.c_void_p(FAKE)

    def verify(batch=2, n_q=6, kv=None, q=p):
        kv = kv if kv is not None else _kv()
        return lib.std_dense_verify_attn_batch(ctypes.byref(sh), q, n_q, batch, ctypes.byref(kv),
                                               None, 0, p, None, 0, None)
    assert verify(batch=0) == E
    assert verify(n_q=0) == E
    assert verify(q=None) == E
    assert verify(batch=70000) == E                       # rows past the grid
    assert verify(kv=_kv(dtype=_lib.STD_DTYPE_F32)) == U
    assert verify() == _lib.STD_ERR_WORKSPACE_TOO_SMALL    # valid: stops at the workspace
    one = lib.std_dense_verify_workspace(ctypes.byref(sh), 6, ctypes.byref(_kv()))
    two = lib.std_dense_verify_batch_workspace(ctypes.byref(sh), 6, 2, ctypes.byref(_kv()))
    assert one > 0 and two > one
    # acceptance: every check fires before a launch
    assert lib.std_accept_batch(p, 3, 0, None, p, 10, 0, p, p, None, None, None) == E
    assert lib.std_accept_batch(p, -1, 2, None, p, 10, 0, p, p, None, None, None) == E
    assert lib.std_accept_batch(None, 3, 2, None, p, 10, 0, p, p, None, None, None) == E
    assert lib.std_accept_batch(p, 3, 2, p, p, 10, 7, p, p, None, None, None) == E


def test_check_idx_rejects():
    lib = _lib.load()
    E = _lib.STD_ERR_INVALID_ARGUMENT
    p = ctypes.c_void_p(FAKE)
    vis = _lib.Vis(0, 100)
    assert lib.std_check_idx(p, 4, 10, vis, None, None) == E
    assert lib.std_check_idx(None, 4, 10, vis, p, None) == E
    assert lib.std_check_idx(p, 0, 10, vis, p, None) == E
    assert lib.std_check_idx(p, 4, -1, vis, p, None) == E
    assert lib.std_check_idx(p, 4, 101, vis, p, None) == E
    assert lib.std_check_idx(p, 4, 10, _lib.Vis(-1, 100), p, None) == E
    assert lib.std_check_idx(p, 4, 10, _lib.Vis(0, 0), p, None) == E


def test_read_probe_rejects():
    lib = _lib.load()
    E = _lib.STD_ERR_INVALID_ARGUMENT
    p = ctypes.c_void_p(FAKE)
    assert lib.std_hbm_read_probe(None, 1 << 20, p, None) == E
    assert lib.std_hbm_read_probe(p, 1 << 20, None, None) == E
    assert lib.std_hbm_read_probe(p, 0, p, None) == E
    assert lib.std_hbm_read_probe(p, 17, p, None) == E
    assert lib.std_hbm_read_probe(ctypes.c_void_p(FAKE + 8), 1 << 20, p, None) == E
    assert lib.std_hbm_read_probe(p, 1 << 20, ctypes.c_void_p(FAKE + 2), None) == E


def test_workspace_sizes():
    lib = _lib.load()
    sh = _shape()
    small = lib.std_dense_verify_workspace(ctypes.byref(sh), 7, ctypes.byref(_kv(200000, 142055)))
    big = lib.std_dense_verify_workspace(ctypes.byref(sh), 7, ctypes.byref(_kv(300000, 284110)))
    assert 0 < small <= big
    # chunking depends on len only: n_q scales the rows linearly
    one = lib.std_dense_verify_workspace(ctypes.byref(sh), 1, ctypes.byref(_kv(200000, 142055)))
    assert one < small
    assert lib.std_dense_verify_workspace(ctypes.byref(sh), 0, ctypes.byref(_kv())) == 0
    s1 = lib.std_sparse_decode_workspace(ctypes.byref(sh), ctypes.byref(_kv(200000, 142049)),
                                         _lib.Vis(0, 140000), 4096)
    s2 = lib.std_sparse_decode_workspace(ctypes.byref(sh), ctypes.byref(_kv(200000, 142049)),
                                         _lib.Vis(0, 140000), 8192)
    assert 0 < s1 < s2
    w = lib.std_select_topk_workspace(ctypes.byref(sh), 2048, _lib.Vis(0, 140000), 4096,
                                      ctypes.byref(_kv(142048, 142048)))
    assert w >= 4 * 140000 * 4                 # room for the scores
    assert lib.std_select_topk_workspace(ctypes.byref(sh), 2048, _lib.Vis(0, 140000), 0,
                                         ctypes.byref(_kv(142048, 142048))) == 0


def test_workspace_queries_follow_their_calls():
    """A query returns 0, with the reason in std_last_error, for arguments its
    call rejects before the workspace check (batched limits and dtypes too)."""
    lib = _lib.load()
    sh = _shape()
    f32 = _kv(dtype=_lib.STD_DTYPE_F32)
    vis = _lib.Vis(0, 800)

    def reason():
        return lib.std_last_error().decode()

    # dense verify: n_q past the length; batch > 1 needs bf16
    assert lib.std_dense_verify_workspace(ctypes.byref(sh), 1001, ctypes.byref(_kv())) == 0
    assert "n_q" in reason()
    assert lib.std_dense_verify_batch_workspace(ctypes.byref(sh), 6, 2, ctypes.byref(f32)) == 0
    assert "bf16" in reason()
    assert lib.std_dense_verify_batch_workspace(ctypes.byref(sh), 6, 1, ctypes.byref(f32)) > 0
    assert lib.std_dense_verify_batch_workspace(ctypes.byref(sh), 6, 70000,
                                                ctypes.byref(_kv())) == 0
    # sparse draft: batch > 1 needs bf16; batch * n_q_heads bounded
    assert lib.std_sparse_decode_batch_workspace(ctypes.byref(sh), 2, ctypes.byref(f32), vis,
                                                 64) == 0
    assert "bf16" in reason()
    assert lib.std_sparse_decode_batch_workspace(ctypes.byref(sh), 1, ctypes.byref(f32), vis,
                                                 64) > 0
    big = _shape(hq=512, hkv=32)
    assert lib.std_sparse_decode_batch_workspace(ctypes.byref(big), 40000, ctypes.byref(_kv()),
                                                 vis, 64) == 0
    assert "2^24" in reason()
    # selection and prefill queries name their reason too
    assert lib.std_select_topk_workspace(ctypes.byref(sh), 16, vis, 64, None) == 0
    assert "kv is null" in reason()
    assert lib.std_prefill_text_attn_workspace(ctypes.byref(sh), -1, 10) == 0
    assert "text_start" in reason()


def test_static_window_idx_rejects():
    lib = _lib.load()
    E = _lib.STD_ERR_INVALID_ARGUMENT
    p = ctypes.c_void_p(FAKE)
    vis = _lib.Vis(0, 100)
    assert lib.std_static_window_idx(0, vis, 4, 10, p, None) == E
    assert lib.std_static_window_idx(2, _lib.Vis(-1, 100), 4, 10, p, None) == E
    assert lib.std_static_window_idx(2, _lib.Vis(0, 0), 4, 10, p, None) == E
    assert lib.std_static_window_idx(2, vis, 4, 101, p, None) == E
    assert lib.std_static_window_idx(2, vis, 4, -1, p, None) == E
    assert lib.std_static_window_idx(2, vis, -1, 10, p, None) == E
    assert lib.std_static_window_idx(2, vis, 4, 10, None, None) == E
    assert lib.std_static_window_idx(2, _lib.Vis(0x7fffff00, 0x1000), 4, 10, p, None) == E
    assert lib.std_last_error() != b""


# ------------------------------------------------------- binding validation
# The Python wrappers check dtypes and shapes before the device, so these
# rejections are reachable with CPU tensors; nothing reaches the library.

import torch  # noqa: E402


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def _raises(fn, what):
    with pytest.raises(ValueError) as e:
        fn()
    assert what in str(e.value), str(e.value)


def test_binding_rejects_mismatched_attention_tensors():
    k, v = _t(4, 300, 128), _t(4, 300, 128)
    q = _t(7, 28, 128)
    _raises(lambda: _lib.std_dense_verify_attn(q.float(), k, v, 200), "q must be")
    _raises(lambda: _lib.std_dense_verify_attn(q, k, _t(4, 299, 128), 200), "v must have shape")
    _raises(lambda: _lib.std_dense_verify_attn(q, k, v.float(), 200), "v must be")
    _raises(lambda: _lib.std_dense_verify_attn(_t(7, 28, 64), k, v, 200), "head_dim 128")
    _raises(lambda: _lib.std_dense_verify_attn(q, k, v, 200, out=_t(7, 28, 128).float()),
            "out must be")
    _raises(lambda: _lib.std_dense_verify_attn(q, k, v, 200, out=_t(6, 28, 128)),
            "out must have shape")
    _raises(lambda: _lib.std_dense_verify_attn(q, _t(4, 300, 128, dtype=torch.float16), v, 200),
            "k must be")
    qs = _t(28, 128)
    idx = torch.zeros(4, 16, dtype=torch.int32)
    _raises(lambda: _lib.std_sparse_decode_attn(qs, k, v, 200, 0, 100, idx.long()),
            "idx must be")
    _raises(lambda: _lib.std_sparse_decode_attn(qs, k, v, 200, 0, 100, idx[:3]), "idx must be")
    _raises(lambda: _lib.std_sparse_decode_attn(qs, k, v, 200, 0, 100, idx,
                                                out=_t(28, 64)), "out must have shape")
    _raises(lambda: _lib.std_sparse_decode_attn_dlen(qs, k, v, 200, torch.zeros(1), 0, 0, 100,
                                                     idx), "len_dev must be")
    kb, vb = _t(2, 4, 300, 128), _t(2, 4, 300, 128)
    _raises(lambda: _lib.std_sparse_decode_attn_batch(_t(3, 28, 128), kb, vb, 200, 0, 100,
                                                      torch.zeros(3, 4, 16, dtype=torch.int32)),
            "same batch")
    _raises(lambda: _lib.std_sparse_decode_attn_batch(
        _t(2, 28, 128), kb, vb, 200, 0, 100, torch.zeros(2, 4, 16, dtype=torch.int32),
        gamma_dev=torch.zeros(3, dtype=torch.int32)), "gamma_dev must have shape")
    _raises(lambda: _lib.std_dense_verify_attn_batch(_t(2, 7, 28, 128), kb, vb, 200,
                                                     len_dev=torch.zeros(3, dtype=torch.int32)),
            "len_dev must hold 2")


def test_binding_rejects_bad_selection_and_prefill_buffers():
    k, v = _t(4, 300, 128), _t(4, 300, 128)
    qt = _t(28, 20, 128)
    _raises(lambda: _lib.std_select_topk(qt, k, 280, 260, 0, 200, 16,
                                         lse=torch.zeros(28 * 19)), "lse must hold")
    _raises(lambda: _lib.std_select_topk(qt, k, 280, 260, 0, 200, 16,
                                         lse=torch.zeros(28, 20, dtype=torch.float64)),
            "lse must be")
    _raises(lambda: _lib.std_select_topk(qt, k, 280, 260, 0, 200, 16,
                                         idx_out=torch.zeros(4, 15, dtype=torch.int32)),
            "idx_out must have shape")
    _raises(lambda: _lib.std_select_topk(qt, k, 280, 260, 0, 200, 16,
                                         scores_out=torch.zeros(4, 199)),
            "scores_out must have shape")
    _raises(lambda: _lib.std_select_topk(qt.float(), k, 280, 260, 0, 200, 16), "q_text must be")
    _raises(lambda: _lib.std_prefill_text_attn(qt, k, v, 280, 260, lse_out=torch.zeros(28, 19)),
            "lse_out must be")
    _raises(lambda: _lib.std_prefill_text_attn(qt, k, v, 280, 260, out=_t(28, 19, 128)),
            "out must have shape")


def test_binding_rejects_bad_acceptance_buffers():
    draft = torch.zeros(4, dtype=torch.int32)
    logits = torch.zeros(5, 100)
    _raises(lambda: _lib.std_accept(draft, torch.zeros(4, 100)), "logits must be")
    _raises(lambda: _lib.std_accept(draft.long(), logits), "draft must be")
    _raises(lambda: _lib.std_accept(draft, logits.double()), "logits must be")
    _raises(lambda: _lib.std_accept(draft, logits, out_tokens=torch.zeros(4, dtype=torch.int32)),
            "out_tokens must have shape")
    _raises(lambda: _lib.std_accept(draft, logits, margins=torch.zeros(4)), "margins must have")
    _raises(lambda: _lib.std_accept(draft, logits, n_out=torch.zeros(0, dtype=torch.int32)),
            "n_out must hold")
    _raises(lambda: _lib.std_accept(draft, logits, seq_len=torch.zeros(1)), "seq_len must be")
    db = torch.zeros(3, 4, dtype=torch.int32)
    _raises(lambda: _lib.std_accept_batch(db, torch.zeros(3, 4, 100)), "logits must be")
    _raises(lambda: _lib.std_accept_batch(db, torch.zeros(3, 5, 100),
                                          n_out=torch.zeros(2, dtype=torch.int32)),
            "n_out must hold")
    _raises(lambda: _lib.std_accept_batch(db, torch.zeros(3, 5, 100),
                                          gamma_dev=torch.zeros(2, dtype=torch.int32)),
            "gamma_dev must have shape")
    _raises(lambda: _lib.std_static_window_idx(4, 0, 100, 8, 16,
                                               idx_out=torch.zeros(4, 15, dtype=torch.int32)),
            "idx_out must have shape")


def test_noalloc_rejects_before_any_hip_call():
    """The no-alloc draft call checks its arguments, the scratch size
    included, before its first HIP call (so these run without a GPU)."""
    lib = _lib.load()
    sh = _shape()
    P = ctypes.c_void_p
    E = _lib.STD_ERR_INVALID_ARGUMENT

    def call(kv=None, topk=64, q=FAKE, out=FAKE, vis=(0, 800)):
        kv = kv or _kv()
        return lib.std_sparse_decode_attn_noalloc(ctypes.byref(sh), P(q), ctypes.byref(kv), None,
                                                  0, _lib.Vis(*vis), P(FAKE), topk, P(out), None)

    assert call(topk=801) == E
    assert call(q=0) == E
    assert call(out=FAKE + 4) == E
    assert call(kv=_kv(k=0)) == E
    # a list of 2^20 visual entries needs 8,192 splits x 28 rows of partials
    # (about 120 MB), past the library's 8 MiB
    big = _kv(cap=(1 << 20) + 100, length=(1 << 20) + 50)
    assert call(kv=big, topk=1 << 20, vis=(0, 1 << 20)) == _lib.STD_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in lib.std_last_error()
