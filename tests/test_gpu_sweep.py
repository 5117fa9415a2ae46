"""GPU parity over a seeded random sweep of shapes: each case draws a head
layout, head dim, dtype, prefix, visual span, text length, K and query count,
then runs the selection, the sparse draft call on the selected lists, the
dense verify call, and (bf16) the prefill text attention, each against the
float64 oracle on the same values.  The fixed cases elsewhere pin chosen
corners; this sweep covers the combinations between them (ragged tiles,
several key chunks, G from 1 to 20 with both the MFMA and the vector-ALU
paths, K from 1 to the whole span).

Bars as everywhere: attention max-abs 2e-2 (bf16) / 1e-5 (fp32); selection
scores within 1e-4 relative and index sets exact outside the 1e-6 band;
prefill normaliser within 2e-5.
"""

import sys

import numpy as np
import pytest
import torch

import oracle

TOL = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = 2e-5
N_CASES = 48


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


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def draw(seed):
    """One case's shapes from a seeded generator (host only)."""
    r = np.random.default_rng(seed)
    hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 7, 8, 16, 20]))
    d = int(r.choice([64, 128]))
    dtype = "f32" if r.random() < 0.25 else "bf16"
    prefix = int(r.choice([0, int(r.integers(1, 120))]))
    vis_len = int(r.integers(1, 9)) if r.random() < 0.15 else int(r.integers(1, 6000))
    n_text = int(r.integers(1, 70))
    kind = r.random()
    if kind < 0.15:
        topk = 1
    elif kind < 0.3:
        topk = vis_len                       # the sparse call then equals the dense one
    else:
        topk = int(r.integers(1, vis_len + 1))
        if r.random() < 0.5:
            topk = min(topk, int(r.integers(1, 600)))
    # positions decoded after the prompt
    n_gen = 0 if r.random() < 0.2 else int(r.integers(1, 40))
    n_q = int(r.integers(1, 18))
    slack = int(r.integers(0, 70))
    return dict(hkv=hkv, hq=hkv * G, d=d, dtype=dtype, prefix=prefix, vis_len=vis_len,
                n_text=n_text, topk=topk, n_gen=n_gen, n_q=n_q, slack=slack)


def test_sweep_draws_cover_the_corners():
    """The sweep reaches both attention paths, both head dims and dtypes, and
    small and whole-span K (host-side check of the draws)."""
    cases = [draw(s) for s in range(N_CASES)]
    assert {c["d"] for c in cases} == {64, 128}
    assert {c["dtype"] for c in cases} == {"f32", "bf16"}
    assert any(c["hq"] // c["hkv"] > 16 for c in cases)
    assert any(c["hq"] // c["hkv"] == 1 for c in cases)
    assert any(c["prefix"] > 0 for c in cases) and any(c["prefix"] == 0 for c in cases)
    assert any(c["topk"] == c["vis_len"] > 1 for c in cases)
    assert any(c["topk"] == 1 < c["vis_len"] for c in cases)
    assert any(c["vis_len"] < 9 for c in cases) and any(c["n_gen"] == 0 for c in cases)
    # verify groups past 64 query rows at head_dim 128 (128-row workgroups)
    assert any(c["d"] == 128 and c["dtype"] == "bf16" and c["n_q"] * c["hq"] // c["hkv"] > 64
               for c in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_sweep_case(lib, seed):
    c = draw(seed)
    say(f"sweep seed={seed} {c}")
    hq, hkv, d, dtype = c["hq"], c["hkv"], c["d"], c["dtype"]
    prefix, vis_len, n_text, topk = c["prefix"], c["vis_len"], c["n_text"], c["topk"]
    text_start = prefix + vis_len
    ctx = text_start + n_text
    length = ctx + c["n_gen"]
    cap = length + c["slack"]
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    gen = torch.Generator(device="cpu").manual_seed(10_000 + seed)
    u = torch.randn(d, generator=gen)
    u /= u.norm()
    k = torch.randn(hkv, cap, d, generator=gen)
    k[:, prefix:text_start] += 2.0 * u * (torch.rand(hkv, vis_len, 1, generator=gen) < 0.05)
    v = torch.randn(hkv, cap, d, generator=gen)
    q_text = torch.randn(hq, n_text, d, generator=gen) + 1.5 * u
    q_draft = torch.randn(hq, d, generator=gen) * 1.5
    q_verify = torch.randn(c["n_q"], hq, d, generator=gen) * 1.5
    k, v, q_text, q_draft, q_verify = (t.to(dt) for t in (k, v, q_text, q_draft, q_verify))
    kf, vf = f64(k), f64(v)
    kd, vd = k.cuda(), v.cuda()

    # selection against the oracle's scores and sets
    idx, scores = lib.std_select_topk(q_text.cuda(), kd, ctx, text_start, prefix, vis_len, topk,
                                      want_scores=True)
    torch.cuda.synchronize()
    _, ref_scores = oracle.select_topk(f64(q_text), kf, text_start, prefix, vis_len, topk)
    rel = np.abs(f64(scores) - ref_scores) / ref_scores
    assert rel.max() < 1e-4, rel.max()
    got = idx.cpu().numpy()
    for g in range(hkv):
        sel = got[g] - prefix
        assert len(set(sel.tolist())) == topk and np.all(np.diff(sel) > 0)
        assert sel.min() >= 0 and sel.max() < vis_len
        s = ref_scores[g]
        kth = np.sort(s)[::-1][topk - 1]
        diff = set(oracle.rank_topk(s, topk).tolist()).symmetric_difference(set(sel.tolist()))
        assert all(abs(s[j] - kth) <= 1e-6 * kth for j in diff), (g, sorted(diff)[:5])

    # the draft step on the selected lists, as the decode position length - 1
    out = lib.std_sparse_decode_attn(q_draft.cuda(), kd, vd, length, prefix, vis_len, idx)
    torch.cuda.synchronize()
    ref = oracle.sparse_decode(f64(q_draft), kf, vf, length, prefix, vis_len, got)
    assert max_abs(f64(out), ref) <= TOL[dtype]

    # the verify step over the whole cache
    out = lib.std_dense_verify_attn(q_verify.cuda(), kd, vd, length)
    torch.cuda.synchronize()
    ref = oracle.dense_verify(f64(q_verify), kf, vf, length)
    assert max_abs(f64(out), ref) <= TOL[dtype]

    # the text rows' prefill attention and normalisers (bf16 calls only)
    if dtype == "bf16":
        out, lse = lib.std_prefill_text_attn(q_text.cuda(), kd, vd, ctx, text_start)
        torch.cuda.synchronize()
        qt = f64(q_text).transpose(1, 0, 2)
        ref = oracle.dense_verify(qt, kf, vf, ctx).transpose(1, 0, 2)
        ref_lse = oracle.row_lse(qt, kf, ctx).T
        assert max_abs(f64(out), ref) <= TOL["bf16"]
        assert max_abs(f64(lse), ref_lse) <= TOL_LSE


# ------------------------------------------------------------ batched sweep
N_BATCH_CASES = 16


def draw_batch(seed):
    """One batched case: B sequences of one layer shape, each with its own
    valid length and draft length (host only)."""
    r = np.random.default_rng(5000 + seed)
    B = int(r.integers(2, 10))
    hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 7, 8, 16]))
    d = int(r.choice([64, 128]))
    prefix = int(r.choice([0, int(r.integers(1, 80))]))
    vis_len = int(r.integers(1, 4000))
    kind = r.random()
    if kind < 0.15:
        topk = 0                                 # text keys only
    elif kind < 0.3:
        topk = vis_len
    else:
        topk = int(r.integers(1, vis_len + 1))
        topk = min(topk, int(r.integers(1, 700))) if r.random() < 0.5 else topk
    gamma = int(r.integers(1, 8))
    # every length past the visual span and at least the verify's gamma + 1
    base = prefix + vis_len + int(r.integers(8, 60))
    lens = [base + int(r.integers(0, 300)) for _ in range(B)]
    gammas = [int(r.integers(0, gamma + 1)) for _ in range(B)]
    vocab = int(r.choice([512, 1000, 3001]))
    return dict(B=B, hkv=hkv, hq=hkv * G, d=d, prefix=prefix, vis_len=vis_len, topk=topk,
                gamma=gamma, lens=lens, gammas=gammas, vocab=vocab)


def test_batch_sweep_draws_cover_the_corners():
    cases = [draw_batch(s) for s in range(N_BATCH_CASES)]
    assert {c["d"] for c in cases} == {64, 128}
    assert any(c["topk"] == 0 for c in cases) and any(c["topk"] == c["vis_len"] for c in cases)
    assert any(0 in c["gammas"] for c in cases)
    assert any(c["hq"] // c["hkv"] == 16 for c in cases) and any(c["hq"] == c["hkv"] for c in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_BATCH_CASES))
def test_batch_sweep_case(lib, seed):
    """The batched draft, verify and acceptance calls on one seeded draw,
    every sequence at its own device length (and draft length for the
    acceptance), against the oracle sequence by sequence."""
    c = draw_batch(seed)
    say(f"batch sweep seed={seed} {c}")
    B, hq, hkv, d = c["B"], c["hq"], c["hkv"], c["d"]
    prefix, vis_len, topk, gamma = c["prefix"], c["vis_len"], c["topk"], c["gamma"]
    lens = c["lens"]
    cap = max(lens) + 5
    gen = torch.Generator(device="cpu").manual_seed(7000 + seed)
    k = torch.randn(B, hkv, cap, d, generator=gen).bfloat16()
    v = torch.randn(B, hkv, cap, d, generator=gen).bfloat16()
    q = (torch.randn(B, hq, d, generator=gen) * 1.5).bfloat16()
    n_q = gamma + 1
    qv = (torch.randn(B, n_q, hq, d, generator=gen) * 1.5).bfloat16()
    idx = torch.stack([torch.stack([torch.sort(torch.randperm(vis_len, generator=gen)[:topk])[0]
                                    for _ in range(hkv)]) for _ in range(B)]).to(torch.int32)
    idx = (idx + prefix).reshape(B, hkv, topk)
    kd, vd = k.cuda(), v.cuda()
    len_dev = torch.tensor(lens, dtype=torch.int32, device="cuda") - 1
    out = lib.std_sparse_decode_attn_batch(q.cuda(), kd, vd, max(lens), prefix, vis_len,
                                           idx.cuda(), len_dev=len_dev, len_offset=1)
    outv = lib.std_dense_verify_attn_batch(qv.cuda(), kd, vd, max(lens), len_dev=len_dev,
                                           len_offset=1)
    torch.cuda.synchronize()
    for b in range(B):
        kf, vf = f64(k[b]), f64(v[b])
        ref = oracle.sparse_decode(f64(q[b]), kf, vf, lens[b], prefix, vis_len, idx[b].numpy())
        assert max_abs(f64(out[b]), ref) <= TOL["bf16"], ("draft", b)
        ref = oracle.dense_verify(f64(qv[b]), kf, vf, lens[b])
        assert max_abs(f64(outv[b]), ref) <= TOL["bf16"], ("verify", b)
    # acceptance with each sequence's own draft length
    import synth
    cases = [synth.accept_case(gamma, c["vocab"], 0.8, seed=9000 + 10 * seed + b,
                               dtype=torch.bfloat16, n_ties=b % 2) for b in range(B)]
    draft = torch.stack([x[0] for x in cases]).cuda()
    logits = torch.stack([x[1] for x in cases]).contiguous().cuda()
    gdev = torch.tensor(c["gammas"], dtype=torch.int32, device="cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    toks, n_out = lib.std_accept_batch(draft, logits, seq_len=seq, gamma_dev=gdev)
    torch.cuda.synchronize()
    for b in range(B):
        g = c["gammas"][b]
        ref_toks, ref_n, _, _ = oracle.accept(cases[b][0][:g].numpy(), f64(cases[b][1][:g + 1]))
        got = toks[b].cpu().numpy().tolist()
        assert got[:g + 1] == ref_toks.tolist() and got[g + 1:] == [-1] * (gamma - g), b
        assert int(n_out[b]) == ref_n and int(seq[b]) == lens[b] + ref_n, b
