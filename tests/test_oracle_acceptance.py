"""Pins for the oracle's greedy acceptance rule, CPU only."""

import itertools
import json
import os

import numpy as np

import oracle


def _one_hot_logits(pred, vocab):
    logits = np.zeros((len(pred), vocab))
    for i, p in enumerate(pred):
        logits[i, p] = 1.0
    return logits


def test_golden_cases(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "accept_cases.json")))
    for case in g["cases"]:
        logits = _one_hot_logits(case["pred"], g["vocab"])
        out, n_out, margins, pred = oracle.accept(np.array(case["draft"], dtype=np.int64), logits)
        assert out.tolist() == case["out"], case["name"]
        assert n_out == case["n_out"], case["name"]
        assert pred.tolist() == case["pred"]
        np.testing.assert_allclose(margins, 1.0)


def test_exhaustive_small_vocab():
    """Every draft sequence x every prediction sequence, vocab 4, gamma <= 4.

    Checked against properties that characterise the rule: 1 <= n_out <=
    gamma+1; the emitted prefix equals the drafts; the last emitted token is
    the dense prediction at that point; either every draft was accepted or
    the first rejected draft differs from the prediction; the emitted tokens
    equal the dense predictions (greedy decoding would emit exactly these).
    """
    vocab = 4
    for gamma in range(0, 5):
        for draft in itertools.product(range(vocab), repeat=gamma):
            for pred in itertools.product(range(vocab), repeat=gamma + 1):
                logits = _one_hot_logits(pred, vocab)
                out, n_out, _, _ = oracle.accept(np.array(draft, dtype=np.int64), logits)
                n = n_out - 1
                assert 1 <= n_out <= gamma + 1
                assert list(out[:n]) == list(draft[:n])
                assert out[n] == pred[n]
                assert n == gamma or draft[n] != pred[n]
                assert list(out[:n_out]) == list(pred[:n_out])
                assert all(x == -1 for x in out[n_out:])
                if draft == pred[:gamma]:
                    assert n_out == gamma + 1
                if gamma and draft[0] != pred[0]:
                    assert n_out == 1


def test_argmax_ties_go_to_lowest_id_and_margin():
    row = np.array([0.5, 2.0, -1.0, 2.0, 1.5])
    assert oracle.argmax_margin(row) == (1, 0.0)
    row2 = np.array([0.5, 3.0, -1.0, 2.0, 1.5])
    best, m = oracle.argmax_margin(row2)
    assert best == 1 and m == 1.0
    # ties decide acceptance through the lowest id
    logits = np.array([[0.0, 1.0, 1.0], [0.0, 0.0, 0.0]])
    out, n_out, _, _ = oracle.accept(np.array([2]), logits)
    assert out.tolist() == [1, -1] and n_out == 1
    out, n_out, _, _ = oracle.accept(np.array([1]), logits)
    assert out.tolist() == [1, 0] and n_out == 2
