"""End to end on the GPU: a small decoder whose attention runs on the four
calls (sparse_draft_speculative_amd.toy_decoder), in fp32.

Pins (the pages' Key contributions: the acceleration is lossless, the output
is that of the dense model):
  * the GPU's dense-only greedy stream equals the float64 oracle's greedy
    stream on the same weights;
  * the GPU's StD stream equals the GPU's dense-only stream, for several K
    and gamma;
  * with K = vis_len the draft model is the dense model, so every cycle
    accepts all gamma drafts.
Streams are compared up to the first position whose dense argmax margin is
<= 1e-3 (where two correct implementations may pick different tokens);
every stream here is checked to reach well past the first few tokens.
"""

import sys

import numpy as np
import pytest
import torch

import synth
from oracle import toy as oracle_toy

pytestmark = pytest.mark.gpu

MARGIN = 1e-3
N_NEW = 40


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_draft_speculative_amd as sd
    from sparse_draft_speculative_amd.toy_decoder import ToyDecoder
    sd.load()
    cfg = dict(synth.TOY_GPU)
    params = synth.toy_params(cfg, seed=3, std=0.1)
    vis, text = synth.toy_prompt(cfg, seed=3)
    prompt_len = cfg["n_vis"] + cfg["n_text"]
    dec = ToyDecoder(params, prompt_len + N_NEW + 16, dtype=torch.float32, prefill_chunk=256)
    margins = torch.full((N_NEW,), float("inf"), dtype=torch.float32, device="cuda")
    first, q_text = dec.prefill(vis, text, margin=margins[0:1])
    snap = dec.snapshot()
    dense = dec.decode_dense(first, prompt_len, N_NEW, margins=margins)
    torch.cuda.synchronize()
    return dict(cfg=cfg, params=params, vis=vis, text=text, dec=dec, first=first,
                q_text=q_text, snap=snap, dense=dense, margins=margins.cpu().numpy(),
                prompt_len=prompt_len)


def trusted_prefix(margins):
    """Positions before the first dense argmax margin <= MARGIN."""
    low = np.nonzero(margins <= MARGIN)[0]
    return int(low[0]) if low.size else len(margins)


def test_dense_stream_matches_oracle_greedy(setup):
    s = setup
    ref = oracle_toy.toy_greedy(s["params"], s["vis"], s["text"], N_NEW)
    n = trusted_prefix(s["margins"])
    say(f"dense stream: trusted prefix {n} of {N_NEW}")
    assert n >= 8
    assert s["dense"][:n] == ref[:n]


@pytest.mark.parametrize("topk,gamma,sink", [(64, 4, None), (16, 2, None), (256, 6, None),
                                             (64, 4, 8)])
def test_std_stream_equals_dense_stream(setup, topk, gamma, sink):
    """sink None: the attention-ranked top-K lists; a sink size: the
    streaming comparator's lists (sink + recent window) through the same
    draft call.  Either way the output is the dense model's."""
    s = setup
    cfg, dec = s["cfg"], s["dec"]
    dec.restore(s["snap"])
    if sink is None:
        idx = dec.select(s["q_text"], s["prompt_len"], 0, cfg["n_vis"], topk)
    else:
        idx = dec.select_static(0, cfg["n_vis"], sink, topk)
    out, acc = dec.decode_std(s["first"], s["prompt_len"], N_NEW, idx, 0, cfg["n_vis"], gamma)
    n = trusted_prefix(s["margins"])
    say(f"K={topk} gamma={gamma} sink={sink}: accepted per cycle {acc}; trusted prefix {n}")
    assert all(0 <= a <= gamma for a in acc)
    assert out[:n] == s["dense"][:n]


def test_full_selection_accepts_every_draft(setup):
    """K = vis_len: sparse key set == dense key set (the pages' special
    case), so each cycle accepts all gamma drafts while the dense margins
    are clear of the tie band."""
    s = setup
    cfg, dec = s["cfg"], s["dec"]
    gamma = 4
    dec.restore(s["snap"])
    idx = dec.select(s["q_text"], s["prompt_len"], 0, cfg["n_vis"], cfg["n_vis"])
    out, acc = dec.decode_std(s["first"], s["prompt_len"], N_NEW, idx, 0, cfg["n_vis"], gamma)
    n = trusted_prefix(s["margins"])
    say(f"K=vis_len: accepted per cycle {acc}; trusted prefix {n}")
    assert out[:n] == s["dense"][:n]
    pos = 1                                  # stream index of the first draft
    for a in acc:
        if pos + gamma > n:                  # cycle reaches the tie band
            break
        assert a == gamma
        pos += a + 1



# ------------------------------------------------------------------ bf16
# The toy decoder of the long-video toy workload (4 layers, hidden 512,
# 8/2/64, vocab 8,192, K = 512) with a bf16 cache, so every attention runs on
# the bf16 MFMA kernels the benchmark uses; projections in fp32 keep each row
# independent of the forward's row count.  Weights N(0, 0.04^2) make the
# attention peaked enough that the top-K draft departs from the dense model
# now and then: cycles accept anything from 0 to gamma drafts.
N_NEW_BF16 = 96


@pytest.fixture(scope="module")
def setup_bf16():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_draft_speculative_amd as sd
    from sparse_draft_speculative_amd.toy_decoder import ToyDecoder
    sd.load()
    cfg = dict(synth.TOY_C5)
    params = synth.toy_params(cfg, seed=0, std=0.04)
    vis, text = synth.toy_prompt(cfg, seed=0)
    prompt_len = cfg["n_vis"] + cfg["n_text"]
    dec = ToyDecoder(params, prompt_len + N_NEW_BF16 + 16, dtype=torch.bfloat16,
                     matmul_dtype=torch.float32, prefill_chunk=512)
    margins = torch.full((N_NEW_BF16,), float("inf"), dtype=torch.float32, device="cuda")
    first, q_text = dec.prefill(vis, text, margin=margins[0:1])
    snap = dec.snapshot()
    dense = dec.decode_dense(first, prompt_len, N_NEW_BF16, margins=margins)
    torch.cuda.synchronize()
    return dict(cfg=cfg, dec=dec, first=first, q_text=q_text, snap=snap, dense=dense,
                margins=margins.cpu().numpy(), prompt_len=prompt_len)


def cycles_inside(acc, gamma, n_trusted):
    """Accepted counts of the cycles whose tokens all lie in the trusted
    prefix (the stream's token 0 comes from the prefill)."""
    out, pos = [], 1
    for a in acc:
        if pos + a + 1 > n_trusted:
            break
        out.append(a)
        pos += a + 1
    return out


@pytest.mark.parametrize("gamma,static", [(4, False), (6, False), (4, True)])
def test_bf16_std_stream_equals_dense_stream(setup_bf16, gamma, static):
    s = setup_bf16
    cfg, dec = s["cfg"], s["dec"]
    dec.restore(s["snap"])
    if static:
        idx = dec.select_static(0, cfg["n_vis"], 64, cfg["topk"])
    else:
        idx = dec.select(s["q_text"], s["prompt_len"], 0, cfg["n_vis"], cfg["topk"])
    out, acc = dec.decode_std(s["first"], s["prompt_len"], N_NEW_BF16, idx, 0, cfg["n_vis"],
                              gamma)
    n = trusted_prefix(s["margins"])
    inside = cycles_inside(acc, gamma, n)
    say(f"bf16 gamma={gamma} static={static}: accepted per cycle {acc}; trusted prefix {n}")
    assert n >= 32
    assert out[:n] == s["dense"][:n]
    assert all(0 <= a <= gamma for a in acc)
    if not static:
        # the stream check covers partly accepted drafts, not only all-or-none
        # (the comparator's lists on this random-init model accept nearly
        # every draft, so only the attention-ranked lists are held to this)
        assert any(0 < a < gamma for a in inside), inside
