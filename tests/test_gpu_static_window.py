"""The streaming-attention comparator on the GPU: the index lists written by
std_static_window_idx, and the sparse draft call run on them, against the
float64 oracle (technical summary, Experimental results: StD is compared
with a streaming-attention draft; its sink and window sizes are a reading,
the pages give none).

Bars: index lists bit-exact; attention max-abs <= 2e-2 (bf16) / 1e-5 (fp32).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_draft_speculative_amd as sd
    sd.load()
    return sd


def f64(t):
    return t.detach().double().cpu().numpy()


@pytest.mark.parametrize("hkv,vis_start,vis_len,sink,topk", [
    (4, 0, 140000, 64, 4096),       # the long-video shape: sink 64 + window 4032
    (4, 0, 16384, 64, 1024),
    (2, 17, 1000, 0, 100),          # window only, after a prefix
    (1, 5, 300, 500, 120),          # sink larger than the budget: sink only
    (3, 0, 777, 10, 777),           # K = vis_len: the whole span
    (8, 100, 64, 4, 0),             # K = 0: nothing written
    (2, 0, 1, 1, 1),                # one-position span
])
def test_static_window_idx_matches_oracle(lib, hkv, vis_start, vis_len, sink, topk):
    idx = lib.std_static_window_idx(hkv, vis_start, vis_len, sink, topk)
    bad = lib.std_check_idx(idx, vis_start, vis_len) if topk else None
    torch.cuda.synchronize()
    want = oracle.static_window_idx(vis_start, vis_len, sink, topk)
    got = idx.cpu().numpy()
    assert got.shape == (hkv, topk)
    for g in range(hkv):
        assert got[g].tolist() == want.tolist(), g
    if bad is not None:
        assert int(bad.item()) == 0          # a valid list for the draft call


@pytest.mark.parametrize("name,sink", [("c1", 16), ("c2", 64), ("c2", 0)])
def test_draft_on_static_window_matches_oracle(lib, name, sink):
    """The draft call on the comparator's list against the oracle's sparse
    attention over the same positions, for every draft step of a cycle."""
    cfg = synth.config(name)
    lay = synth.attention_layer(cfg, 0, device="cuda")
    idx = lib.std_static_window_idx(cfg.n_kv_heads, cfg.vis_start, cfg.vis_len, sink, cfg.topk)
    torch.cuda.synchronize()
    want = oracle.static_window_idx(cfg.vis_start, cfg.vis_len, sink, cfg.topk)
    idx_np = np.tile(want, (cfg.n_kv_heads, 1))
    assert idx.cpu().numpy().tolist() == idx_np.tolist()
    kf, vf = f64(lay["k"]), f64(lay["v"])
    tol = 1e-5 if cfg.dtype == "f32" else 2e-2
    for j in range(cfg.gamma):
        length = cfg.draft_len(j)
        q = lay["q_draft"][j].contiguous()
        out = lib.std_sparse_decode_attn(q, lay["k"], lay["v"], length, cfg.vis_start,
                                         cfg.vis_len, idx)
        torch.cuda.synchronize()
        ref = oracle.sparse_decode(f64(q), kf, vf, length, cfg.vis_start, cfg.vis_len, idx_np)
        err = float(np.max(np.abs(f64(out) - ref)))
        say(f"{name} sink {sink} step {j}: max abs err {err:.2e}")
        assert err <= tol
