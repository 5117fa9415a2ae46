"""GPU parity: every call of the HIP library against the float64 oracle.

Inputs are seeded synthetic tensors (synth); the oracle reads back exactly
the values the GPU received.  Bars: attention max-abs <= 2e-2 (bf16 KV) and
<= 1e-5 (fp32 KV); top-K sets exact except for positions whose oracle score
lies within 1e-6 relative of the K-th value (ties to the lower position);
acceptance bit-exact.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


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


def layer(cfg, i=0):
    return synth.attention_layer(cfg, i, device="cuda")


def oracle_idx(cfg, lay):
    idx, scores = oracle.select_topk(f64(lay["q_text"]), f64(lay["k"]), cfg.text_start,
                                     cfg.vis_start, cfg.vis_len, cfg.topk)
    return idx, scores


def check_topk(gpu_idx, ref_scores, topk, vis_start, vis_len, band=1e-6):
    """A15: distinct in-span ascending positions; the symmetric difference with
    the oracle set lies in the 1e-6 band around the oracle's K-th score."""
    gpu_idx = np.asarray(gpu_idx)
    for g in range(gpu_idx.shape[0]):
        sel = gpu_idx[g] - vis_start
        assert len(set(sel.tolist())) == topk
        assert np.all(np.diff(sel) > 0), "not ascending"
        assert sel.min() >= 0 and sel.max() < vis_len
        s = ref_scores[g]
        ref = set(oracle.rank_topk(s, topk).tolist())
        kth = np.sort(s)[::-1][topk - 1]
        diff = ref.symmetric_difference(set(sel.tolist()))
        bad = [j for j in diff if abs(s[j] - kth) > band * kth]
        assert not bad, f"head {g}: {len(bad)} positions outside the tie band, e.g. {bad[:5]}"


# ---------------------------------------------------------------- dense verify
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_dense_verify_matches_oracle(lib, name):
    cfg = synth.config(name)
    lay = layer(cfg)
    say(f"dense verify {name} n_q={cfg.gamma + 1} len={cfg.verify_len}")
    out = lib.std_dense_verify_attn(lay["q_verify"], lay["k"], lay["v"], cfg.verify_len)
    torch.cuda.synchronize()
    ref = oracle.dense_verify(f64(lay["q_verify"]), f64(lay["k"]), f64(lay["v"]), cfg.verify_len)
    err = max_abs(f64(out), ref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_dense_single_query_decode(lib, name):
    cfg = synth.config(name)
    lay = layer(cfg)
    for j in (0, cfg.gamma - 1):
        length = cfg.draft_len(j)
        q = lay["q_draft"][j:j + 1].contiguous()
        out = lib.std_dense_verify_attn(q, lay["k"], lay["v"], length)
        torch.cuda.synchronize()
        ref = oracle.dense_verify(f64(q), f64(lay["k"]), f64(lay["v"]), length)
        assert max_abs(f64(out), ref) <= TOL[cfg.dtype]


@pytest.mark.parametrize("hq,hkv,d,dtype,n_q,length,cap", [
    (8, 2, 64, "bf16", 7, 8390, 8400),      # toy-decoder shape, ragged length
    (28, 4, 128, "bf16", 1, 65, 70),        # tiny cache, single query
    (28, 4, 128, "bf16", 100, 3000, 3001),  # many query rows: several 128-row blocks
    (28, 4, 128, "bf16", 10, 5000, 5003),   # gamma = 9: 70 rows, one 128-row block
    (28, 4, 128, "bf16", 18, 1100, 1118),   # 126 rows, one 128-row block
    (28, 4, 128, "bf16", 19, 1500, 1519),   # 133 rows: two 128-row blocks, the second ragged
    (8, 1, 64, "bf16", 9, 700, 710),        # 72 rows at head_dim 64: two 64-row blocks
    (4, 4, 64, "f32", 3, 777, 800),         # G = 1, fp32
    (32, 1, 128, "bf16", 5, 4097, 4100),    # G = 32
    (6, 2, 128, "f32", 2, 130, 130),
    (4, 1, 64, "f32", 1, 1, 1),             # one key: the output is that key's V row
    (28, 4, 128, "bf16", 1, 1, 8),          # one valid key in a larger cache
])
def test_dense_verify_shapes(lib, hq, hkv, d, dtype, n_q, length, cap):
    g = torch.Generator(device="cuda").manual_seed(hq * 1000 + length)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    k = torch.randn(hkv, cap, d, generator=g, device="cuda").to(dt)
    v = torch.randn(hkv, cap, d, generator=g, device="cuda").to(dt)
    q = (torch.randn(n_q, hq, d, generator=g, device="cuda") * 1.5).to(dt)
    say(f"dense shape hq={hq} hkv={hkv} d={d} {dtype} n_q={n_q} len={length}")
    out = lib.std_dense_verify_attn(q, k, v, length)
    torch.cuda.synchronize()
    ref = oracle.dense_verify(f64(q), f64(k), f64(v), length)
    assert max_abs(f64(out), ref) <= TOL[dtype]


def test_dense_verify_is_deterministic_and_row_invariant(lib):
    cfg = synth.config("c2")
    lay = layer(cfg)
    a = lib.std_dense_verify_attn(lay["q_verify"], lay["k"], lay["v"], cfg.verify_len)
    b = lib.std_dense_verify_attn(lay["q_verify"], lay["k"], lay["v"], cfg.verify_len)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # the last verify row is the dense n_q=1 decode at the same length
    one = lib.std_dense_verify_attn(lay["q_verify"][-1:].contiguous(), lay["k"], lay["v"],
                                    cfg.verify_len)
    torch.cuda.synchronize()
    assert torch.equal(one[0], a[-1])


@pytest.mark.parametrize("n_q", [10, 17])
def test_dense_verify_rows_past_64_are_row_invariant(lib, n_q):
    """Groups of more than 64 query rows (head_dim 128) take 128-row
    workgroups; each row's arithmetic is the same as in a 64-row block, so
    the last verify row equals the single-query call bitwise."""
    g = torch.Generator(device="cuda").manual_seed(n_q)
    k = torch.randn(4, 9000, 128, generator=g, device="cuda").bfloat16()
    v = torch.randn(4, 9000, 128, generator=g, device="cuda").bfloat16()
    q = (torch.randn(n_q, 28, 128, generator=g, device="cuda") * 1.5).bfloat16()
    length = 8990
    a = lib.std_dense_verify_attn(q, k, v, length)
    one = lib.std_dense_verify_attn(q[-1:].contiguous(), k, v, length)
    torch.cuda.synchronize()
    assert torch.equal(one[0], a[-1])
    ref = oracle.dense_verify(f64(q), f64(k), f64(v), length)
    assert max_abs(f64(a), ref) <= TOL["bf16"]


# ---------------------------------------------------------------- sparse draft
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_sparse_decode_matches_oracle(lib, name):
    cfg = synth.config(name)
    lay = layer(cfg)
    idx_ref, _ = oracle_idx(cfg, lay)
    idx = torch.from_numpy(idx_ref.astype(np.int32)).cuda()
    kf, vf = f64(lay["k"]), f64(lay["v"])
    for j in range(cfg.gamma):
        length = cfg.draft_len(j)
        q = lay["q_draft"][j].contiguous()
        say(f"sparse {name} step {j} len={length} K={cfg.topk}")
        out = lib.std_sparse_decode_attn(q, lay["k"], lay["v"], length, cfg.vis_start,
                                         cfg.vis_len, idx)
        torch.cuda.synchronize()
        ref = oracle.sparse_decode(f64(q), kf, vf, length, cfg.vis_start, cfg.vis_len, idx_ref)
        err = max_abs(f64(out), ref)
        assert err <= TOL[cfg.dtype], err


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_sparse_full_selection_equals_dense(lib, name):
    """K = vis_len: the sparse kernel must equal dense attention (oracle)."""
    cfg = synth.config(name)
    lay = layer(cfg)
    hkv = cfg.n_kv_heads
    idx = torch.arange(cfg.vis_start, cfg.vis_end, dtype=torch.int32, device="cuda")
    idx = idx.repeat(hkv, 1).contiguous()
    length = cfg.draft_len(0)
    q = lay["q_draft"][0].contiguous()
    out = lib.std_sparse_decode_attn(q, lay["k"], lay["v"], length, cfg.vis_start, cfg.vis_len, idx)
    torch.cuda.synchronize()
    ref = oracle.dense_verify(f64(q)[None], f64(lay["k"]), f64(lay["v"]), length)[0]
    assert max_abs(f64(out), ref) <= TOL[cfg.dtype]


@pytest.mark.parametrize("hq,hkv,d,dtype,prefix,vis_len,length,topk", [
    (28, 4, 128, "bf16", 0, 16384, 16897, 0),       # K = 0: text only
    (28, 4, 128, "bf16", 37, 5000, 5100, 1),        # prefix before the span, K = 1
    (8, 2, 64, "bf16", 5, 8192, 8330, 512),         # toy-decoder shape
    (32, 2, 128, "bf16", 0, 1000, 1100, 100),       # G = 16
    (34, 2, 128, "bf16", 0, 1000, 1100, 100),       # G = 17: vector-ALU path
    (4, 1, 64, "f32", 10, 1000, 1200, 77),
    (7, 7, 128, "f32", 0, 300, 301, 300),           # G = 1, K = vis_len
    (4, 2, 128, "bf16", 0, 1, 5, 1),                # one-position visual span
    (4, 2, 64, "f32", 3, 1, 9, 1),                  # one-position span after a prefix
])
def test_sparse_decode_shapes(lib, hq, hkv, d, dtype, prefix, vis_len, length, topk):
    gen = torch.Generator(device="cpu").manual_seed(hq * 7 + topk)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    cap = length + 3
    k = torch.randn(hkv, cap, d, generator=gen).to(dt).cuda()
    v = torch.randn(hkv, cap, d, generator=gen).to(dt).cuda()
    q = (torch.randn(hq, d, generator=gen) * 1.5).to(dt).cuda()
    idx_np = np.stack([np.sort(torch.randperm(vis_len, generator=gen)[:topk].numpy()) + prefix
                       for _ in range(hkv)]).astype(np.int32).reshape(hkv, topk)
    idx = torch.from_numpy(idx_np).cuda()
    say(f"sparse shape hq={hq} hkv={hkv} d={d} {dtype} prefix={prefix} K={topk} len={length}")
    out = lib.std_sparse_decode_attn(q, k, v, length, prefix, vis_len, idx)
    torch.cuda.synchronize()
    ref = oracle.sparse_decode(f64(q), f64(k), f64(v), length, prefix, vis_len, idx_np)
    assert max_abs(f64(out), ref) <= TOL[dtype]


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_select_topk_matches_oracle(lib, name):
    cfg = synth.config(name)
    lay = layer(cfg)
    say(f"select {name} n_text={cfg.n_text} vis={cfg.vis_len} K={cfg.topk}")
    idx, scores = lib.std_select_topk(lay["q_text"], lay["k"], cfg.ctx, cfg.text_start,
                                      cfg.vis_start, cfg.vis_len, cfg.topk, want_scores=True)
    torch.cuda.synchronize()
    _, ref_scores = oracle_idx(cfg, lay)
    rel = np.abs(f64(scores) - ref_scores) / ref_scores
    say(f"  score rel err max {rel.max():.2e} median {np.median(rel):.2e}")
    assert rel.max() < 1e-4
    check_topk(idx.cpu().numpy(), ref_scores, cfg.topk, cfg.vis_start, cfg.vis_len)


def test_select_topk_exact_ties_and_prefix(lib):
    """Duplicated key rows tie bitwise and the lower position wins; a
    non-visual prefix before the span; bf16 d=64."""
    gen = torch.Generator(device="cpu").manual_seed(5)
    hq, hkv, d, prefix, vis_len, n_text = 8, 2, 64, 9, 700, 40
    cap = prefix + vis_len + n_text
    k = torch.randn(hkv, cap, d, generator=gen)
    q = torch.randn(hq, n_text, d, generator=gen)
    u = torch.randn(d, generator=gen)
    u /= u.norm()
    q += 2 * u
    for j in (50, 51, 400, 401, 402):
        k[:, prefix + j] = 6 * u + k[:, prefix + 3]     # five copies of one strong row
    k[:, prefix + 3] = 6 * u + k[:, prefix + 3]
    q, k = q.bfloat16(), k.bfloat16()
    for topk in (1, 3, 6, 7, vis_len):
        idx, scores = lib.std_select_topk(q.cuda(), k.cuda(), cap, prefix + vis_len, prefix,
                                          vis_len, topk, want_scores=True)
        torch.cuda.synchronize()
        sc = scores.cpu()
        for g in range(hkv):
            assert sc[g, 3] == sc[g, 50] == sc[g, 401], "identical rows must tie bitwise"
        ref_idx, ref_scores = oracle.select_topk(f64(q), f64(k), prefix + vis_len, prefix,
                                                 vis_len, topk)
        check_topk(idx.cpu().numpy(), ref_scores, topk, prefix, vis_len)
        if topk <= 6:
            want = [prefix + j for j in (3, 50, 51, 400, 401, 402)][:topk]
            assert ref_idx.tolist() == [want] * hkv          # premise of the case
            assert idx.cpu().numpy().tolist() == [want] * hkv


@pytest.mark.parametrize("hq,hkv,d,prefix,vis_len,n_text,topk", [
    (4, 4, 128, 0, 100, 1, 7),          # one text row per head, G = 1
    (8, 2, 128, 5, 1000, 3, 64),        # G = 4, rows < one tile, prefix
    (7, 1, 128, 64, 2000, 17, 500),     # G = 7, a partial query tile
    (16, 2, 128, 0, 9000, 20, 1024),    # G = 8, keys over two LSE chunks
    (28, 4, 128, 3, 777, 41, 777),      # K = vis_len; 287 rows per group
    (8, 8, 64, 0, 385, 9, 33),          # d = 64, a key block past one workgroup
    (12, 3, 64, 100, 3000, 30, 300),    # d = 64, prefix, rows past one row block
    (4, 1, 128, 0, 1, 4, 1),            # one-position visual span, K = 1
    (8, 2, 64, 2, 1, 3, 1),             # the same after a prefix, d = 64
])
def test_select_topk_shapes(lib, hq, hkv, d, prefix, vis_len, n_text, topk):
    """bf16 selection over shapes that leave partial query tiles, partial key
    blocks, text rows past a row block, keys over several LSE chunks, a
    non-visual prefix and row-range splits (small grids use several)."""
    gen = torch.Generator(device="cpu").manual_seed(hq * 1000 + vis_len + n_text)
    cap = prefix + vis_len + n_text + 5
    k = torch.randn(hkv, cap, d, generator=gen).bfloat16()
    q = torch.randn(hq, n_text, d, generator=gen).bfloat16()
    text_start = prefix + vis_len
    say(f"select shape hq={hq} hkv={hkv} d={d} prefix={prefix} vis={vis_len} "
        f"n_text={n_text} K={topk}")
    idx, scores = lib.std_select_topk(q.cuda(), k.cuda(), cap, text_start, prefix, vis_len, topk,
                                      want_scores=True)
    torch.cuda.synchronize()
    _, ref_scores = oracle.select_topk(f64(q), f64(k), text_start, prefix, vis_len, topk)
    rel = np.abs(f64(scores) - ref_scores) / ref_scores
    say(f"  score rel err max {rel.max():.2e}")
    assert rel.max() < 1e-4
    check_topk(idx.cpu().numpy(), ref_scores, topk, prefix, vis_len)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_select_topk_uses_caller_lse(lib, name):
    """The caller's natural-log row LSE replaces step 1 (fp32 and bf16 paths).
    The LSE comes from the oracle's own row normaliser (row_lse), the value a
    prefill attention returns beside its output."""
    cfg = synth.config(name)
    lay = layer(cfg)
    # text row i of head h sits at position text_start + i: the rows of a
    # dense pass of n_text queries ending at text_start + n_text
    qf, kf = f64(lay["q_text"]), f64(lay["k"])
    lse = np.ascontiguousarray(
        oracle.row_lse(qf.transpose(1, 0, 2), kf, cfg.text_start + cfg.n_text).T)
    lse_t = torch.from_numpy(lse.astype(np.float32)).cuda()
    idx, scores = lib.std_select_topk(lay["q_text"], lay["k"], cfg.ctx, cfg.text_start,
                                      cfg.vis_start, cfg.vis_len, cfg.topk, lse=lse_t,
                                      want_scores=True)
    torch.cuda.synchronize()
    _, ref_scores = oracle_idx(cfg, lay)
    assert np.max(np.abs(f64(scores) - ref_scores) / ref_scores) < 1e-4
    check_topk(idx.cpu().numpy(), ref_scores, cfg.topk, cfg.vis_start, cfg.vis_len)


# ---------------------------------------------------------------- acceptance
@pytest.mark.parametrize("gamma,vocab,dtype,agree,ties", [
    (0, 8192, torch.float32, 0.9, 0),
    (4, 8192, torch.float32, 0.95, 0),
    (6, 8192, torch.bfloat16, 0.95, 2),
    (9, 300, torch.float32, 1.0, 3),
    (6, 152064, torch.bfloat16, 0.5, 1),
    (70, 1000, torch.float32, 0.99, 0),
    (5, 1, torch.float32, 1.0, 0),
])
def test_accept_matches_oracle(lib, gamma, vocab, dtype, agree, ties):
    for seed in range(4):
        draft, logits = synth.accept_case(gamma, vocab, agree, seed, dtype=dtype, n_ties=ties)
        seq = torch.tensor([1000], dtype=torch.int32, device="cuda")
        margins = torch.empty(gamma + 1, dtype=torch.float32, device="cuda")
        out, n_out = lib.std_accept(draft.cuda(), logits.cuda(), margins=margins, seq_len=seq)
        torch.cuda.synchronize()
        ref_out, ref_n, ref_m, _ = oracle.accept(draft.numpy(), f64(logits))
        assert out.cpu().numpy().tolist() == ref_out.tolist()
        assert int(n_out.item()) == ref_n
        assert int(seq.item()) == 1000 + ref_n
        assert np.allclose(margins.cpu().numpy(), ref_m, rtol=1e-6, atol=1e-6)
        # without margins the call takes its value-only path: same tokens
        out2, n2 = lib.std_accept(draft.cuda(), logits.cuda())
        torch.cuda.synchronize()
        assert out2.cpu().numpy().tolist() == ref_out.tolist() and int(n2.item()) == ref_n


@pytest.mark.parametrize("vocab", [152064, 1000, 1001, 9])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_accept_argmax_corners(lib, vocab, dtype):
    """Argmax corners against the oracle, with and without margins: a row of
    -inf (the lowest id wins, margin NaN), a maximum repeated across a
    16-byte chunk boundary (ids 7 and 8) and at the ends of the row, the
    maximum on the last id, and a row whose runner-up sits on the last id.
    vocab 1001 and 9 take the element-by-element path."""
    gamma = 5
    gen = torch.Generator(device="cpu").manual_seed(vocab)
    logits = torch.randn(gamma + 1, vocab, generator=gen)
    logits[0] = -float("inf")
    logits[1, 7] = logits[1, 8] = 9.0
    logits[2, vocab - 1] = 9.0
    logits[3, 0] = 9.0
    logits[3, vocab - 1] = 8.5
    logits[4, 0] = logits[4, vocab - 1] = 9.0
    logits = logits.to(dtype)
    draft = torch.tensor([0, 7, vocab - 1, 0, 0], dtype=torch.int32)
    say(f"accept corners vocab={vocab} {dtype}")
    ref_out, ref_n, ref_m, ref_pred = oracle.accept(draft.numpy(), f64(logits))
    assert ref_pred[:5].tolist() == [0, 7, vocab - 1, 0, 0]       # premise of the case
    margins = torch.empty(gamma + 1, dtype=torch.float32, device="cuda")
    out, n_out = lib.std_accept(draft.cuda(), logits.cuda(), margins=margins)
    out2, n2 = lib.std_accept(draft.cuda(), logits.cuda())
    torch.cuda.synchronize()
    assert out.cpu().numpy().tolist() == ref_out.tolist() and int(n_out.item()) == ref_n
    assert out2.cpu().numpy().tolist() == ref_out.tolist() and int(n2.item()) == ref_n
    assert np.allclose(margins.cpu().numpy(), ref_m, rtol=1e-6, atol=1e-6, equal_nan=True)


def test_sparse_decode_reuses_one_workspace(lib):
    """Back-to-back calls of different sizes sharing one (dirty) workspace
    stay correct: the workspace is scratch and needs no initialisation."""
    cfg = synth.config("c2")
    lay = layer(cfg)
    idx_ref, _ = oracle_idx(cfg, lay)
    idx = torch.from_numpy(idx_ref.astype(np.int32)).cuda()
    shape = lib.attn_shape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    nbytes = lib.std_sparse_decode_workspace(shape, lay["k"], cfg.capacity, cfg.vis_start,
                                             cfg.vis_len, cfg.topk)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device="cuda")   # garbage
    kf, vf = f64(lay["k"]), f64(lay["v"])
    for rep in range(3):
        for j in (cfg.gamma - 1, 0, 2):
            length = cfg.draft_len(j)
            sub = idx[:, : cfg.topk - 100 * rep].contiguous()   # shrinking key sets
            q = lay["q_draft"][j].contiguous()
            out = lib.std_sparse_decode_attn(q, lay["k"], lay["v"], length, cfg.vis_start,
                                             cfg.vis_len, sub, workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.sparse_decode(f64(q), kf, vf, length, cfg.vis_start, cfg.vis_len,
                                       idx_ref[:, : cfg.topk - 100 * rep])
            assert max_abs(f64(out), ref) <= TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_sparse_decode_clamps_out_of_span_positions(lib, name):
    """A selected position outside the visual span is read as the nearest end
    of the span: a malformed list never leaves the cache.  The two
    out-of-span values here (3 below, 2 above the span) lie inside the cache,
    and the result must match the clamped list, not the raw one."""
    cfg = synth.config(name)
    lay = layer(cfg)
    vs, vl = 16, cfg.vis_len - 16
    ve, length, topk = vs + vl, cfg.draft_len(0), 64
    rng = np.random.default_rng(7)
    raw, clamped = [], []
    for _ in range(cfg.n_kv_heads):
        mid = np.sort(rng.choice(np.arange(vs + 1, ve - 1), topk - 2, replace=False))
        raw.append(np.concatenate([[vs - 3], mid, [ve + 2]]))
        clamped.append(np.concatenate([[vs], mid, [ve - 1]]))
    idx = torch.tensor(np.array(raw), dtype=torch.int32, device="cuda")
    q = lay["q_draft"][0].contiguous()
    say(f"sparse clamp {name} len={length} span=[{vs},{ve}) K={topk}")
    out = f64(lib.std_sparse_decode_attn(q, lay["k"], lay["v"], length, vs, vl, idx))
    torch.cuda.synchronize()
    qf, kf, vf = f64(q), f64(lay["k"]), f64(lay["v"])
    ref = oracle.sparse_decode(qf, kf, vf, length, vs, vl, np.array(clamped))
    # the raw list read literally (its two rows duplicate prefix/tail keys)
    G, scale = cfg.n_q_heads // cfg.n_kv_heads, 1.0 / np.sqrt(cfg.head_dim)
    ref_raw = np.empty_like(ref)
    for g in range(cfg.n_kv_heads):
        keys = np.concatenate([np.arange(0, vs), raw[g], np.arange(ve, length)])
        for h in range(g * G, (g + 1) * G):
            ref_raw[h] = oracle.attend(qf[h], kf[g, keys], vf[g, keys], scale)
    assert max_abs(ref, ref_raw) > 2 * TOL[cfg.dtype]      # the case discriminates
    assert max_abs(out, ref) <= TOL[cfg.dtype]


def test_every_call_is_bitwise_repeatable(lib):
    """No reduction in the library uses floating-point atomics and every
    merge has a fixed order, so running a call twice on the same inputs
    gives the same bits: selection (scores and positions), the sparse draft
    call, the prefill text attention (output and normalisers) and the
    acceptance (tokens, count, margins)."""
    cfg = synth.config("c2")
    lay = layer(cfg)
    runs = []
    for _ in range(2):
        idx, sc = lib.std_select_topk(lay["q_text"], lay["k"], cfg.ctx, cfg.text_start,
                                      cfg.vis_start, cfg.vis_len, cfg.topk, want_scores=True)
        sp = lib.std_sparse_decode_attn(lay["q_draft"][0].contiguous(), lay["k"], lay["v"],
                                        cfg.draft_len(0), cfg.vis_start, cfg.vis_len, idx)
        pf, lse = lib.std_prefill_text_attn(lay["q_text"], lay["k"], lay["v"], cfg.ctx,
                                            cfg.text_start)
        draft, logits = synth.accept_case(cfg.gamma, 4096, 0.8, seed=9, dtype=torch.bfloat16,
                                          n_ties=1)
        margins = torch.empty(cfg.gamma + 1, dtype=torch.float32, device="cuda")
        toks, n_out = lib.std_accept(draft.cuda(), logits.cuda(), margins=margins)
        torch.cuda.synchronize()
        runs.append([idx, sc, sp, pf, lse, toks, n_out, margins])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
