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
    # grids above one round of resident workgroups (B x H_kv x 128-entry
    # chunks > 512): two chunks per workgroup, the last split's second
    # chunk partly or wholly past each sequence's list
    (6, 28, 4, 128, 0, 20000, 2048, (22001, 21500, 22100, 21337, 22048, 21900)),
    (12, 16, 2, 64, 40, 30000, 3000, tuple(30100 + 37 * b for b in range(12))),
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


# ------------------------------------------------------- batched dense verify
@pytest.mark.parametrize("B,hq,hkv,d,n_q,lens", [
    (3, 28, 4, 128, 7, (2100, 1037, 2299)),
    (4, 8, 2, 64, 5, (600, 517, 650, 701)),
    (2, 32, 1, 128, 3, (4097, 4000)),          # G = 32: several 64-row blocks per sequence
])
def test_batched_dense_verify_matches_oracle(lib, B, hq, hkv, d, n_q, lens):
    cap = max(lens) + 5
    g = torch.Generator(device="cpu").manual_seed(B * 31 + hq)
    k = torch.randn(B, hkv, cap, d, generator=g).bfloat16().cuda()
    v = torch.randn(B, hkv, cap, d, generator=g).bfloat16().cuda()
    q = (torch.randn(B, n_q, hq, d, generator=g) * 1.5).bfloat16().cuda()
    len_dev = torch.tensor(lens, dtype=torch.int32, device="cuda") - 4     # offset 4 below
    say(f"batched dense B={B} hq={hq} hkv={hkv} d={d} n_q={n_q} lens={lens}")
    out = lib.std_dense_verify_attn_batch(q, k, v, max(lens), len_dev=len_dev, len_offset=4)
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle.dense_verify(f64(q[b]), f64(k[b]), f64(v[b]), lens[b])
        assert np.max(np.abs(f64(out[b]) - ref)) <= TOL, b


def test_batched_dense_verify_two_rounds_matches_oracle(lib):
    """A batch whose workgroups would each stream at least 128 tiles in one
    round of 256 (16 sequences x 8 KV heads, 516 tiles of 64 keys) takes
    two rounds of workgroups: every sequence still matches the oracle."""
    B, hq, hkv, d, n_q = 16, 16, 8, 128, 4
    lens = [32800 + 13 * b for b in range(B)]
    cap = max(lens) + 3
    g = torch.Generator(device="cuda").manual_seed(424)
    k = torch.randn(B, hkv, cap, d, generator=g, device="cuda").bfloat16()
    v = torch.randn(B, hkv, cap, d, generator=g, device="cuda").bfloat16()
    q = (torch.randn(B, n_q, hq, d, generator=g, device="cuda") * 1.5).bfloat16()
    len_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    say(f"batched dense two rounds B={B} hq={hq} hkv={hkv} n_q={n_q} max len {max(lens)}")
    out = lib.std_dense_verify_attn_batch(q, k, v, max(lens), len_dev=len_dev, len_offset=0)
    torch.cuda.synchronize()
    for b in (0, 7, B - 1):
        ref = oracle.dense_verify(f64(q[b]), f64(k[b]), f64(v[b]), lens[b])
        assert np.max(np.abs(f64(out[b]) - ref)) <= TOL, b


def test_batched_dense_verify_of_one_equals_single_call(lib):
    g = torch.Generator(device="cpu").manual_seed(5)
    k = torch.randn(1, 4, 3000, 128, generator=g).bfloat16().cuda()
    v = torch.randn(1, 4, 3000, 128, generator=g).bfloat16().cuda()
    q = torch.randn(1, 7, 28, 128, generator=g).bfloat16().cuda()
    out_b = lib.std_dense_verify_attn_batch(q, k, v, 2999)
    out_1 = lib.std_dense_verify_attn(q[0].contiguous(), k[0].contiguous(), v[0].contiguous(),
                                      2999)
    torch.cuda.synchronize()
    assert torch.equal(out_b[0], out_1)


# ------------------------------------------------------------ batched accept
def test_batched_accept_matches_oracle(lib):
    import synth
    B, gamma, vocab = 5, 6, 3000
    cases = [synth.accept_case(gamma, vocab, 0.8, seed=70 + b, dtype=torch.bfloat16,
                               n_ties=b % 2) for b in range(B)]
    draft = torch.stack([c[0] for c in cases]).cuda()
    logits = torch.stack([c[1] for c in cases]).contiguous().cuda()
    seq = torch.tensor([100 * b for b in range(B)], dtype=torch.int32, device="cuda")
    toks, n_out = lib.std_accept_batch(draft, logits, seq_len=seq)
    torch.cuda.synchronize()
    for b in range(B):
        ref_toks, ref_n, _, _ = oracle.accept(cases[b][0].numpy(), f64(cases[b][1]))
        assert toks[b].cpu().numpy().tolist() == ref_toks.tolist(), b
        assert int(n_out[b]) == ref_n
        assert int(seq[b]) == 100 * b + ref_n


# ----------------------------------------------------- one batched cycle
def test_batched_cycle_equals_single_calls(lib):
    """gamma draft steps for three sequences through the batched call equal
    the single-sequence device-length calls with the same bound, bit for bit
    (same kernel and split count, per-sequence offsets).  The batched verify
    pass raises its split count so the grid fills whole rounds, which
    changes the reduction order: it is held to the oracle instead."""
    B, hq, hkv, d, vis_len, topk, gamma = 3, 28, 4, 128, 1500, 128, 4
    ctx = (1700, 1601, 1800)
    cap = max(ctx) + gamma + 2
    q, k, v, idx = make_batch(B, hq, hkv, d, 0, vis_len, cap, topk, seed=99)
    g = torch.Generator(device="cpu").manual_seed(98)
    qv = (torch.randn(B, gamma + 1, hq, d, generator=g) * 1.5).bfloat16().cuda()
    seq = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    max_len = cap
    drafts_b = [lib.std_sparse_decode_attn_batch(q, k, v, max_len, 0, vis_len, idx, len_dev=seq,
                                                 len_offset=1 + j) for j in range(gamma)]
    verify_b = lib.std_dense_verify_attn_batch(qv, k, v, max_len, len_dev=seq,
                                               len_offset=gamma + 1)
    torch.cuda.synchronize()
    for b in range(B):
        kb, vb = k[b].contiguous(), v[b].contiguous()
        for j in range(gamma):
            one = lib.std_sparse_decode_attn_dlen(q[b].contiguous(), kb, vb, max_len,
                                                  seq[b:b + 1], 1 + j, 0, vis_len,
                                                  idx[b].contiguous())
            assert torch.equal(drafts_b[j][b], one), (b, j)
        ref = oracle.dense_verify(f64(qv[b]), f64(kb), f64(vb), ctx[b] + gamma + 1)
        assert np.max(np.abs(f64(verify_b[b]) - ref)) <= TOL, b


# ------------------------------------------------ per-sequence draft lengths
def test_batched_accept_per_sequence_gamma(lib):
    """Each sequence's own gamma_b (a device array; gamma is the row stride):
    sequence b is std_accept on draft[b][:gamma_b] and logit rows
    [b][:gamma_b + 1], against the oracle; unused slots are -1 and unused
    rows' margins NaN; each length advances by its own n + 1."""
    import synth
    B, stride, vocab = 6, 6, 2000
    gam = [6, 0, 3, 1, 6, 4]
    cases = [synth.accept_case(stride, vocab, 0.85, seed=90 + b, dtype=torch.bfloat16,
                               n_ties=b % 2) for b in range(B)]
    draft = torch.stack([c[0] for c in cases]).cuda()
    logits = torch.stack([c[1] for c in cases]).contiguous().cuda()
    gdev = torch.tensor(gam, dtype=torch.int32, device="cuda")
    seq = torch.tensor([10 * b for b in range(B)], dtype=torch.int32, device="cuda")
    margins = torch.zeros(B, stride + 1, dtype=torch.float32, device="cuda")
    toks, n_out = lib.std_accept_batch(draft, logits, seq_len=seq, margins=margins,
                                       gamma_dev=gdev)
    torch.cuda.synchronize()
    m = margins.cpu().numpy()
    for b in range(B):
        g = gam[b]
        ref_toks, ref_n, ref_m, _ = oracle.accept(cases[b][0][:g].numpy(),
                                                  f64(cases[b][1][:g + 1]))
        got = toks[b].cpu().numpy().tolist()
        assert got[:g + 1] == ref_toks.tolist(), b
        assert got[g + 1:] == [-1] * (stride - g), b
        assert int(n_out[b]) == ref_n and 1 <= ref_n <= g + 1
        assert int(seq[b]) == 10 * b + ref_n
        assert np.allclose(m[b, :g + 1], ref_m, rtol=0, atol=1e-6)
        assert np.all(np.isnan(m[b, g + 1:]))
    # with every gamma_b equal to the stride the call is the uniform one
    full = torch.full((B,), stride, dtype=torch.int32, device="cuda")
    t1, n1 = lib.std_accept_batch(draft, logits, gamma_dev=full)
    t2, n2 = lib.std_accept_batch(draft, logits)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2) and torch.equal(n1, n2)


def test_batched_cycle_per_sequence_gamma(lib):
    """A cycle for three sequences drafting 4, 2 and 3 tokens: draft step j
    runs only the sequences with j < gamma_b (bit for bit the single
    device-length call; the others' output rows stay untouched); the verify
    pass takes 1 + max gamma queries and sequence b's first gamma_b + 1 rows
    are its verify rows (against the oracle); acceptance per sequence."""
    B, hq, hkv, d, vis_len, topk = 3, 28, 4, 128, 1500, 128
    gam = (4, 2, 3)
    gmax = max(gam)
    ctx = (1700, 1601, 1800)
    cap = max(ctx) + gmax + 2
    q, k, v, idx = make_batch(B, hq, hkv, d, 0, vis_len, cap, topk, seed=77)
    g = torch.Generator(device="cpu").manual_seed(76)
    qv = (torch.randn(B, gmax + 1, hq, d, generator=g) * 1.5).bfloat16().cuda()
    seq = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    gdev = torch.tensor(gam, dtype=torch.int32, device="cuda")
    sentinel = torch.full_like(q, 7.0)
    drafts = []
    for j in range(gmax):
        o = sentinel.clone()
        lib.std_sparse_decode_attn_batch(q, k, v, cap, 0, vis_len, idx, len_dev=seq,
                                         len_offset=1 + j, gamma_dev=gdev, step=j, out=o)
        drafts.append(o)
    verify = lib.std_dense_verify_attn_batch(qv, k, v, cap, len_dev=seq, len_offset=gmax + 1)
    torch.cuda.synchronize()
    for b in range(B):
        kb, vb = k[b].contiguous(), v[b].contiguous()
        for j in range(gmax):
            if j < gam[b]:
                one = lib.std_sparse_decode_attn_dlen(q[b].contiguous(), kb, vb, cap,
                                                      seq[b:b + 1], 1 + j, 0, vis_len,
                                                      idx[b].contiguous())
                torch.cuda.synchronize()
                assert torch.equal(drafts[j][b], one), (b, j)
            else:
                assert torch.equal(drafts[j][b], sentinel[b]), (b, j)
        rows = gam[b] + 1
        ref = oracle.dense_verify(f64(qv[b][:rows]), f64(kb), f64(vb), ctx[b] + rows)
        assert np.max(np.abs(f64(verify[b][:rows]) - ref)) <= TOL, b


def test_graph_replayed_batch_with_device_gammas(lib):
    """One batched draft step and one batched acceptance captured once in a
    HIP graph and replayed three times with the per-sequence draft lengths
    changed on the device between replays (eager work and synchronisations
    in between): every replay equals the eager calls with that replay's
    lengths (draft outputs bit for bit, acceptance exactly)."""
    import synth
    B, hq, hkv, d, vis_len, topk, stride = 4, 28, 4, 128, 1500, 128, 5
    ctx = (1700, 1601, 1800, 1650)
    cap = max(ctx) + stride + 2
    q, k, v, idx = make_batch(B, hq, hkv, d, 0, vis_len, cap, topk, seed=55)
    cases = [synth.accept_case(stride, 1000, 0.7, seed=300 + b) for b in range(B)]
    draft = torch.stack([c[0] for c in cases]).cuda()
    logits = torch.stack([c[1] for c in cases]).contiguous().cuda()
    seq = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    gdev = torch.zeros(B, dtype=torch.int32, device="cuda")
    step = 1
    out = torch.zeros_like(q)
    toks = torch.empty(B, stride + 1, dtype=torch.int32, device="cuda")
    n_out = torch.empty(B, dtype=torch.int32, device="cuda")
    shape = lib.attn_shape(hq, hkv, d)
    ws = torch.zeros(lib.std_sparse_decode_batch_workspace(shape, B, k, cap, 0, vis_len, topk),
                     dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()
    sp = lib.prepare_sparse_decode_batch(q, k, v, cap, 0, vis_len, idx, out, ws, len_dev=seq,
                                         len_offset=1 + step, gamma_dev=gdev, step=step,
                                         stream=st)
    ac = lib.prepare_accept_batch(draft, logits, toks, n_out, gamma_dev=gdev, stream=st)
    torch.cuda.synchronize()
    with torch.cuda.stream(st):          # warm-up outside the capture
        sp()
        ac()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        sp()
        ac()
    torch.cuda.synchronize()
    for gam in ((5, 0, 3, 1), (2, 2, 2, 2), (0, 5, 1, 4)):
        gdev.copy_(torch.tensor(gam, dtype=torch.int32))
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = torch.full_like(q, 3.0)
        ref_out = lib.std_sparse_decode_attn_batch(q, k, v, cap, 0, vis_len, idx, len_dev=seq,
                                                   len_offset=1 + step, gamma_dev=gdev,
                                                   step=step, out=ref)
        ref_t, ref_n = lib.std_accept_batch(draft, logits, gamma_dev=gdev)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), gam
        for b in range(B):
            if gam[b] <= step:
                assert torch.equal(out[b], torch.full_like(q[b], 3.0)), (gam, b)
        assert torch.equal(toks, ref_t) and torch.equal(n_out, ref_n), gam
        for b in range(B):
            want, want_n, _, _ = oracle.accept(cases[b][0][:gam[b]].numpy(),
                                               f64(cases[b][1][:gam[b] + 1]))
            assert int(n_out[b]) == want_n
            assert toks[b][:gam[b] + 1].cpu().numpy().tolist() == want.tolist()
