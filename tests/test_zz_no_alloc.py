"""The no-alloc sparse draft call (std_sparse_decode_attn_noalloc), whose
split-K partials live in the library's own static scratch, against the call
with a caller workspace (std_sparse_decode_attn / _dlen) and the float64
oracle: two calls in a row, the second smaller, each bit for bit equal to
the workspace call (same kernels, same split) and within the bf16 bar of
the oracle.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2


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


def case(cfg):
    lay = synth.attention_layer(cfg, 0, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(cfg.vis_len)
    idx = torch.stack([torch.sort(torch.randperm(cfg.vis_len, generator=g)[:cfg.topk])[0]
                       for _ in range(cfg.n_kv_heads)]).to(torch.int32) + cfg.vis_start
    return lay, idx.cuda()


def test_noalloc_equals_workspace_call(lib):
    big = synth.config("c2")                                    # 16,384 + 512, K 1,024
    small = synth.config("c2", vis_len=2000, n_text=64, topk=256)
    for cfg in (big, small):                                    # second call smaller
        lay, idx = case(cfg)
        q = lay["q_draft"][0].contiguous()
        length = cfg.draft_len(0)
        say(f"no-alloc draft call: vis {cfg.vis_len}, K {cfg.topk}, len {length}")
        a = lib.std_sparse_decode_attn_noalloc(q, lay["k"], lay["v"], length, cfg.vis_start,
                                               cfg.vis_len, idx)
        b = lib.std_sparse_decode_attn(q, lay["k"], lay["v"], length, cfg.vis_start,
                                       cfg.vis_len, idx)
        seq = torch.tensor([cfg.ctx], dtype=torch.int32, device="cuda")
        c = lib.std_sparse_decode_attn_noalloc(q, lay["k"], lay["v"], cfg.capacity,
                                               cfg.vis_start, cfg.vis_len, idx, len_dev=seq,
                                               len_offset=1)
        d = lib.std_sparse_decode_attn_dlen(q, lay["k"], lay["v"], cfg.capacity, seq, 1,
                                            cfg.vis_start, cfg.vis_len, idx)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert torch.equal(c, d)
        ref = oracle.sparse_decode(f64(q), f64(lay["k"]), f64(lay["v"]), length, cfg.vis_start,
                                   cfg.vis_len, idx.cpu().numpy())
        err = float(np.max(np.abs(f64(a) - ref)))
        say(f"  bitwise equal to the workspace call; max abs err vs oracle {err:.2e}")
        assert err <= TOL
