"""Batched sparse draft attention (several independent sequences in one
launch) against the float64 oracle, sequence by sequence.

Each sequence has its own cache, its own selected positions and (through
len_dev) its own valid length; with batch 1 the batched call equals the
single-sequence call bit for bit.
"""

import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2            # bf16 KV


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


def make_batch(B, hq, hkv, d, prefix, vis_len, cap, topk, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = torch.randn(B, hkv, cap, d, generator=g).bfloat16()
    v = torch.randn(B, hkv, cap, d, generator=g).bfloat16()
    q = (torch.randn(B, hq, d, generator=g) * 1.5).bfloat16()
    idx = torch.stack([torch.stack([torch.sort(torch.randperm(vis_len, generator=g)[:topk])[0]
                                    for _ in range(hkv)]) for _ in range(B)]) + prefix
    return q.cuda(), k.cuda(), v.cuda(), idx.to(torch.int32).cuda()


@pytest.mark.parametrize("B,hq,hkv,d,prefix,vis_len,topk,lens", [
    (3, 28, 4, 128, 0, 2000, 256, (2100, 2037, 2299)),
    (5, 8, 2, 64, 17, 900, 100, (1000, 917, 950, 999, 1040)),
    (2, 16, 1, 128, 0, 3000, 0, (3001, 3100)),     # K = 0: text keys only
])
def test_batched_sparse_matches_oracle(lib, B, hq, hkv, d, prefix, vis_len, topk, lens):
    cap = max(lens) + 8
    q, k, v, idx = make_batch(B, hq, hkv, d, prefix, vis_len, cap, topk, seed=B * 100 + hq)
    if topk == 0:
        idx = torch.zeros(B, hkv, 0, dtype=torch.int32, device="cuda")
    max_len = max(lens)
    len_dev = torch.tensor(lens, dtype=torch.int32, device="cuda") - 1
    say(f"batched sparse B={B} hq={hq} hkv={hkv} d={d} K={topk} lens={lens}")
    out = lib.std_sparse_decode_attn_batch(q, k, v, max_len, prefix, vis_len, idx,
                                           len_dev=len_dev, len_offset=1)
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle.sparse_decode(f64(q[b]), f64(k[b]), f64(v[b]), lens[b], prefix, vis_len,
                                   idx[b].cpu().numpy())
        err = float(np.max(np.abs(f64(out[b]) - ref)))
        say(f"  sequence {b} len {lens[b]}: max abs err {err:.2e}")
        assert err <= TOL


def test_batched_sparse_without_device_lengths(lib):
    """len_dev NULL: every sequence attends over max_len positions."""
    B, hq, hkv, d, vis_len, topk, L = 4, 28, 4, 128, 1500, 128, 1600
    q, k, v, idx = make_batch(B, hq, hkv, d, 0, vis_len, L + 4, topk, seed=7)
    out = lib.std_sparse_decode_attn_batch(q, k, v, L, 0, vis_len, idx)
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle.sparse_decode(f64(q[b]), f64(k[b]), f64(v[b]), L, 0, vis_len,
                                   idx[b].cpu().numpy())
        assert float(np.max(np.abs(f64(out[b]) - ref))) <= TOL


def test_batch_of_one_equals_single_call(lib):
    hq, hkv, d, vis_len, topk, L = 28, 4, 128, 2000, 256, 2100
    q, k, v, idx = make_batch(1, hq, hkv, d, 0, vis_len, L + 4, topk, seed=11)
    a = lib.std_sparse_decode_attn_batch(q, k, v, L, 0, vis_len, idx)
    b = lib.std_sparse_decode_attn(q[0].contiguous(), k[0].contiguous(), v[0].contiguous(), L, 0,
                                   vis_len, idx[0].contiguous())
    seq = torch.tensor([L - 50], dtype=torch.int32, device="cuda")
    c = lib.std_sparse_decode_attn_batch(q, k, v, L, 0, vis_len, idx, len_dev=seq, len_offset=3)
    e = lib.std_sparse_decode_attn_dlen(q[0].contiguous(), k[0].contiguous(), v[0].contiguous(),
                                        L, seq, 3, 0, vis_len, idx[0].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a[0], b) and torch.equal(c[0], e)
