"""Pins for the oracle's prefill-time top-K selection, CPU only."""

import json
import math
import os

import numpy as np
import pytest

import oracle
import synth


def _hand_case(w):
    """Keys [ln w_j, 0] and one text query [1, 0] at position len(w)-1."""
    n = len(w)
    k = np.zeros((1, n, 2))
    k[0, :, 0] = np.log(np.asarray(w, dtype=np.float64))
    q = np.array([[[1.0, 0.0]]])                    # [H_q=1][n_text=1][d=2]
    return q, k


def test_golden_hand_cases(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "selection_hand.json")))
    for case in g["cases"]:
        q, k = _hand_case(case["w"])
        vis_len = len(case["scores"])
        s = oracle.selection_scores(q, k, text_start=vis_len, vis_start=0,
                                    vis_len=vis_len, scale=1.0)
        np.testing.assert_allclose(s[0], case["scores"], atol=g["tol"], rtol=0)
        for kk, want in case["topk"].items():
            idx, _ = oracle.select_topk(q, k, vis_len, 0, vis_len, int(kk), scale=1.0)
            assert idx[0].tolist() == want


def test_ranking_matches_brute_force_sort():
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(1, 64))
        s = rng.integers(0, 6, size=n).astype(np.float64) / 7.0   # many exact ties
        for kk in {1, n, int(rng.integers(1, n + 1))}:
            got = oracle.rank_topk(s, kk)
            want = sorted(sorted(range(n), key=lambda j: (-s[j], j))[:kk])
            assert got.tolist() == want
            chosen = set(got.tolist())
            lo = min(s[j] for j in chosen)
            assert all(s[j] <= lo for j in range(n) if j not in chosen)


def test_zero_queries_give_closed_form_uniform_scores():
    """Q = 0: each text row is uniform over its pos+1 keys.

    score_j = (1/n_text) sum_i 1/(text_start + i + 1) for every visual j, so
    all visual scores tie and the lowest positions are chosen.
    """
    rng = np.random.default_rng(12)
    hq, hkv, d, vis_start, vis_len, n_text = 4, 2, 8, 3, 20, 5
    k = rng.standard_normal((hkv, vis_start + vis_len + n_text, d))
    q = np.zeros((hq, n_text, d))
    ts = vis_start + vis_len
    idx, s = oracle.select_topk(q, k, ts, vis_start, vis_len, 6)
    want = np.mean([1.0 / (ts + i + 1) for i in range(n_text)])
    np.testing.assert_allclose(s, want, atol=1e-15, rtol=0)
    assert idx.tolist() == [list(range(vis_start, vis_start + 6))] * hkv


def test_identical_keys_tie_exactly_and_lower_index_wins():
    rng = np.random.default_rng(13)
    hq, hkv, d, vis_len, n_text = 2, 1, 8, 12, 4
    k = rng.standard_normal((hkv, vis_len + n_text, d))
    q = rng.standard_normal((hq, n_text, d))
    k[0, 9] = k[0, 4]
    k[0, 4] *= 1.0
    k[0, 4] += 6.0 * q[0, 0] / np.linalg.norm(q[0, 0])    # make key 4 (and 9) strong
    k[0, 9] = k[0, 4]
    idx, s = oracle.select_topk(q, k, vis_len, 0, vis_len, 1)
    assert s[0, 4] == s[0, 9]
    assert idx[0].tolist() == [4]
    idx2, _ = oracle.select_topk(q, k, vis_len, 0, vis_len, 2)
    assert idx2[0].tolist() == [4, 9]


def test_scores_are_probability_mass_on_visual_keys():
    rng = np.random.default_rng(14)
    hq, hkv, d, vs, vl, nt = 6, 2, 16, 5, 30, 7
    k = rng.standard_normal((hkv, vs + vl + nt, d)) * 2
    q = rng.standard_normal((hq, nt, d)) * 2
    s = oracle.selection_scores(q, k, vs + vl, vs, vl)
    assert np.all(s > 0)
    assert np.all(s.sum(axis=1) < 1.0)
    # no prefix and no text: all mass of a single text row sits on... the
    # visual span plus the row itself, so the mass is at most 1
    k2 = rng.standard_normal((1, vl + 1, d))
    q2 = np.zeros((1, 1, d))
    s2 = oracle.selection_scores(q2, k2, vl, 0, vl)
    np.testing.assert_allclose(s2.sum(), vl / (vl + 1), atol=1e-14, rtol=0)


def test_mean_over_duplicated_rows_is_unchanged():
    """Mean over rows and the head group: duplicating every text row (and
    every query head of the group) leaves the scores unchanged."""
    rng = np.random.default_rng(15)
    d, vl = 8, 16
    k = rng.standard_normal((1, vl + 4, d))
    q = rng.standard_normal((1, 2, d))
    a = oracle.selection_scores(q, k, vl, 0, vl)
    q2 = np.concatenate([q, q], axis=0)                   # G = 2, identical heads
    b = oracle.selection_scores(q2, k, vl, 0, vl)
    np.testing.assert_allclose(a, b, atol=1e-15, rtol=0)


def test_per_head_sets_differ_when_heads_differ():
    """Selection is per KV head (and per layer)."""
    rng = np.random.default_rng(16)
    d, vl, nt = 8, 32, 4
    k = rng.standard_normal((2, vl + nt, d))
    k[0, 3] += 10 * np.ones(d) / math.sqrt(d)
    k[1, 17] += 10 * np.ones(d) / math.sqrt(d)
    q = np.tile(np.ones(d) / math.sqrt(d) * 3, (2, nt, 1))
    idx, _ = oracle.select_topk(q, k, vl, 0, vl, 1)
    assert idx[:, 0].tolist() == [3, 17]


def test_text_rows_must_follow_visual_span():
    k = np.zeros((1, 10, 2))
    q = np.zeros((1, 2, 2))
    with pytest.raises(ValueError):
        oracle.selection_scores(q, k, text_start=4, vis_start=0, vis_len=6)


def test_generator_planted_keys_are_selected():
    """Sanity of the c1 generator (not parity): the top-128 picks most of the
    64 planted keys."""
    cfg = synth.config("c1")
    lay = synth.attention_layer(cfg, 0)
    q = lay["q_text"].double().numpy()
    k = lay["k"].double().numpy()
    idx, _ = oracle.select_topk(q, k, cfg.text_start, cfg.vis_start, cfg.vis_len, cfg.topk)
    planted = set(np.nonzero(lay["planted"][0].numpy())[0].tolist())
    hit = len(planted & set(idx[0].tolist()))
    assert hit >= 56, hit


# ------------------------------------------------ streaming comparator lists
def test_static_window_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "static_window_cases.json")))
    for c in g["cases"]:
        got = oracle.static_window_idx(c["vis_start"], c["vis_len"], c["sink"], c["topk"])
        assert got.tolist() == c["idx"], c["derivation"]


def test_static_window_invariants():
    """A valid draft index list of K positions; the first min(sink, K) are
    the span's first positions and the rest one run ending at the span's
    end; brute force over every position of the span gives the same set."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        vis_start = int(rng.integers(0, 50))
        vis_len = int(rng.integers(1, 80))
        topk = int(rng.integers(0, vis_len + 1))
        sink = int(rng.integers(0, 90))
        got = oracle.static_window_idx(vis_start, vis_len, sink, topk)
        assert len(got) == topk and len(set(got.tolist())) == topk
        assert np.all(np.diff(got) > 0)
        if topk:
            assert got.min() >= vis_start and got.max() < vis_start + vis_len
        s = min(sink, topk)
        assert got[:s].tolist() == list(range(vis_start, vis_start + s))
        if topk > s:
            assert got[-1] == vis_start + vis_len - 1
            assert np.all(np.diff(got[s:]) == 1)
        # brute force: position p of the span is kept iff it is among the
        # first s or the last topk - s positions
        keep = [p for p in range(vis_start, vis_start + vis_len)
                if p - vis_start < s or (vis_start + vis_len - 1 - p) < topk - s]
        assert got.tolist() == keep


def test_static_window_full_budget_is_the_span():
    """K = vis_len keeps the whole span for any sink, so the draft over that
    list is the dense model (the sparse == dense special case)."""
    for sink in (0, 1, 7, 100):
        assert oracle.static_window_idx(5, 40, sink, 40).tolist() == list(range(5, 45))


def test_static_window_rejects():
    for args in ((0, 10, 2, 11), (0, 10, -1, 3), (-1, 10, 2, 3), (0, 10, 2, -1)):
        with pytest.raises(ValueError):
            oracle.static_window_idx(*args)
