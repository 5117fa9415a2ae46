"""GPU parity of the prefill text-row attention (std_prefill_text_attn)
against the float64 oracle: the output against dense_verify on the text rows
(each row i as a single query at position text_start + i), the normaliser
against row_lse.  Small shapes are compared in full, larger ones on sampled
rows.  End to end, the selection fed this normaliser returns the oracle's
top-K within the 1e-6 band.

Bars: output max-abs <= 2e-2 (bf16, as every attention call); normaliser
max-abs <= 2e-5 (fp32 scores and sums of bf16 inputs: about 1e-7 relative
per term, the normaliser is O(10)).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_OUT = 2e-2
TOL_LSE = 2e-5


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


def inputs(hq, hkv, d, text_start, n_text, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    cap = text_start + n_text + 3
    k = torch.randn(hkv, cap, d, generator=gen).bfloat16()
    v = torch.randn(hkv, cap, d, generator=gen).bfloat16()
    q = (torch.randn(hq, n_text, d, generator=gen) * 1.5).bfloat16()
    return q, k, v


def oracle_rows(qf, kf, vf, text_start, rows):
    """Oracle output and normaliser of the listed (h, i) text rows, each as a
    single query at its own position."""
    out, lse = [], []
    for h, i in rows:
        q1 = qf[h:h + 1, i][None]                 # [1][1][d] for head h only
        hkv, hq = kf.shape[0], qf.shape[0]
        g = h // (hq // hkv)
        length = text_start + i + 1
        out.append(oracle.dense_verify(q1, kf[g:g + 1], vf[g:g + 1], length)[0, 0])
        lse.append(oracle.row_lse(q1, kf[g:g + 1], length)[0, 0])
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("hq,hkv,d,text_start,n_text", [
    (4, 4, 128, 0, 1),            # one text row at position 0: one key
    (8, 2, 64, 100, 40),          # d = 64, G = 4
    (7, 1, 128, 5, 60),           # G = 7: 420 rows, past one workgroup
    (28, 4, 128, 1000, 37),       # GQA 28/4, ragged rows and keys
])
def test_prefill_full(lib, hq, hkv, d, text_start, n_text):
    q, k, v = inputs(hq, hkv, d, text_start, n_text, seed=hq * 100 + n_text)
    say(f"prefill full hq={hq} hkv={hkv} d={d} text_start={text_start} n_text={n_text}")
    length = text_start + n_text
    out, lse = lib.std_prefill_text_attn(q.cuda(), k.cuda(), v.cuda(), length, text_start)
    torch.cuda.synchronize()
    qf, kf, vf = f64(q), f64(k), f64(v)
    ref = oracle.dense_verify(qf.transpose(1, 0, 2), kf, vf, length).transpose(1, 0, 2)
    ref_lse = oracle.row_lse(qf.transpose(1, 0, 2), kf, length).T
    assert np.max(np.abs(f64(out) - ref)) <= TOL_OUT
    assert np.max(np.abs(f64(lse) - ref_lse)) <= TOL_LSE


@pytest.mark.parametrize("hq,hkv,d,text_start,n_text", [
    (28, 4, 128, 16384 + 100, 300),   # two key chunks, text rows in the second
    (32, 2, 128, 16380, 9),           # text rows straddle the chunk boundary
    (8, 2, 64, 40000, 70),            # three chunks, d = 64
])
def test_prefill_sampled_rows(lib, hq, hkv, d, text_start, n_text):
    q, k, v = inputs(hq, hkv, d, text_start, n_text, seed=hq * 7 + n_text)
    say(f"prefill sampled hq={hq} hkv={hkv} d={d} text_start={text_start} n_text={n_text}")
    length = text_start + n_text
    out, lse = lib.std_prefill_text_attn(q.cuda(), k.cuda(), v.cuda(), length, text_start)
    torch.cuda.synchronize()
    rng = np.random.default_rng(n_text)
    rows = [(int(rng.integers(hq)), int(rng.integers(n_text))) for _ in range(24)]
    rows += [(0, 0), (hq - 1, n_text - 1)]
    ref, ref_lse = oracle_rows(f64(q), f64(k), f64(v), text_start, rows)
    got = f64(out)
    got_lse = f64(lse)
    for n, (h, i) in enumerate(rows):
        assert np.max(np.abs(got[h, i] - ref[n])) <= TOL_OUT, (h, i)
        assert abs(got_lse[h, i] - ref_lse[n]) <= TOL_LSE, (h, i)


def test_prefill_lse_drives_the_selection(lib):
    """The selection fed the prefill's normaliser picks the oracle's top-K
    (differences only inside the 1e-6 band around the K-th score)."""
    cfg = synth.config("c2", vis_len=4096, n_text=128, topk=512)
    lay = synth.attention_layer(cfg, 0, device="cuda")
    say(f"prefill -> selection, vis {cfg.vis_len}, text {cfg.n_text}, K {cfg.topk}")
    _, lse = lib.std_prefill_text_attn(lay["q_text"], lay["k"], lay["v"], cfg.ctx,
                                       cfg.text_start)
    idx, _ = lib.std_select_topk(lay["q_text"], lay["k"], cfg.ctx, cfg.text_start,
                                 cfg.vis_start, cfg.vis_len, cfg.topk, lse=lse,
                                 want_scores=True)
    torch.cuda.synchronize()
    _, ref_scores = oracle.select_topk(f64(lay["q_text"]), f64(lay["k"]), cfg.text_start,
                                       cfg.vis_start, cfg.vis_len, cfg.topk)
    got = idx.cpu().numpy()
    for g in range(cfg.n_kv_heads):
        s = ref_scores[g]
        kth = np.sort(s)[::-1][cfg.topk - 1]
        ref = set(oracle.rank_topk(s, cfg.topk).tolist())
        sel = set((got[g] - cfg.vis_start).tolist())
        assert len(sel) == cfg.topk
        bad = [j for j in ref ^ sel if abs(s[j] - kth) > 1e-6 * kth]
        assert not bad, f"head {g}: {bad[:5]}"


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_running_max_moves_inside_a_chunk(lib, d):
    """Keys whose scores climb by more than 2^8 (in base 2) at points inside
    both key chunks move every row's running max mid-chunk, and each move
    rescales what the row has summed so far; the normaliser exposes a
    missed or wrong rescale.  Text queries share a direction u; planted keys
    a*u with growing a sit inside tiles (none at a tile start).  The
    normaliser reaches 25-45 here, so its bar is the same 2e-6 relative that
    TOL_LSE is at O(10)."""
    hq, hkv, text_start, n_text = 8, 2, 20000, 50
    gen = torch.Generator(device="cpu").manual_seed(2024 + d)
    cap = text_start + n_text + 3
    u = torch.randn(d, generator=gen)
    u = u / u.norm()
    k = torch.randn(hkv, cap, d, generator=gen)
    v = torch.randn(hkv, cap, d, generator=gen)
    q = 0.3 * torch.randn(hq, n_text, d, generator=gen) + 4.0 * u
    # q.u lies in about [3.1, 4.9], so in base-2 units (scale log2 e / sqrt(d))
    # each planted key clears the previous maximum by at least 8.8 here
    scale2 = 1.4426950408889634 / d ** 0.5
    step, a0 = 9.0 / (scale2 * 3.1), 11.5 / (scale2 * 3.1)
    plant = [700, 5003, 9999, 17011]
    for n, pos in enumerate(plant):
        k[:, pos] = (a0 + n * step) * u
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    say(f"prefill max moves d={d} planted at {plant}")
    length = text_start + n_text
    out, lse = lib.std_prefill_text_attn(q.cuda(), k.cuda(), v.cuda(), length, text_start)
    torch.cuda.synchronize()
    qf, kf, vf = f64(q), f64(k), f64(v)
    # every row's scores climb past its running max at each planted key
    G = hq // hkv
    s = np.einsum("hid,hkd->hik", qf, np.repeat(kf, G, axis=0)) * scale2
    seq = [s[:, :, :plant[0]].max(axis=2)] + [s[:, :, p] for p in plant]
    assert min(float(np.min(b - a)) for a, b in zip(seq, seq[1:])) > 8.0
    ref = oracle.dense_verify(qf.transpose(1, 0, 2), kf, vf, length).transpose(1, 0, 2)
    ref_lse = oracle.row_lse(qf.transpose(1, 0, 2), kf, length).T
    assert np.max(np.abs(f64(out) - ref)) <= TOL_OUT
    assert np.max(np.abs(f64(lse) - ref_lse) / np.maximum(np.abs(ref_lse), 10.0)) <= TOL_LSE / 10
