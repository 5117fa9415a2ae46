"""Losslessness pins for the oracle's StD loop on a tiny float64 decoder."""

import numpy as np
import pytest

import synth
from oracle import toy


@pytest.fixture(scope="module")
def tiny():
    cfg = dict(synth.TOY_TINY)
    # weights N(0, 0.1^2): large enough that attention changes the logits, so
    # a small K drafts wrong tokens and the rejection path is exercised
    return cfg, synth.toy_params(cfg, seed=1, std=0.1), synth.toy_prompt(cfg, seed=1)


def test_std_stream_equals_greedy_stream(tiny):
    """The StD output equals plain greedy decoding token for token
    (Key contributions: lossless acceleration), for several K and gamma."""
    cfg, p, (vis, text) = tiny
    n_new = 24
    ref = toy.toy_greedy(p, vis, text, n_new)
    for topk, gamma in [(8, 2), (32, 4), (64, 3), (4, 6)]:
        out, acc = toy.toy_std(p, vis, text, n_new, topk, gamma)
        assert out == ref, (topk, gamma)
        assert all(0 <= a <= gamma for a in acc)


def test_full_selection_accepts_every_draft(tiny):
    """K = vis_len makes the sparse model the dense model: every cycle
    accepts all gamma drafts."""
    cfg, p, (vis, text) = tiny
    gamma = 3
    out, acc = toy.toy_std(p, vis, text, 22, cfg["n_vis"], gamma)
    assert acc == [gamma] * len(acc)
    assert out == toy.toy_greedy(p, vis, text, 22)


def test_small_k_rejects_sometimes(tiny):
    """With a very small K the draft model is a different model: the loop
    still reproduces greedy decoding while rejecting some drafts (this also
    checks that the rejection path is exercised)."""
    cfg, p, (vis, text) = tiny
    out, acc = toy.toy_std(p, vis, text, 30, 1, 5)
    assert out == toy.toy_greedy(p, vis, text, 30)
    assert min(acc) < 5
