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


# ---- pins of the decoder's pieces (closed forms, hand values, invariants) ----

def test_rms_norm_hand_value_and_scale_invariance():
    """[3, -4] has mean square 12.5: with weights [1, 2] and eps 0 the output
    is [3, -8] / sqrt(12.5); scaling the input leaves it unchanged, a constant
    vector maps to its sign times the weights, and eps enters under the root."""
    out = toy.rms_norm(np.array([3.0, -4.0]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(out, [0.848528137423857, -2.262741699796952], rtol=1e-14)
    x = np.random.default_rng(0).standard_normal((3, 8))
    w = np.linspace(0.5, 2.0, 8)
    assert np.allclose(toy.rms_norm(7.5 * x, w, 0.0), toy.rms_norm(x, w, 0.0), rtol=1e-13)
    assert np.allclose(toy.rms_norm(np.full(4, -2.5), w[:4], 0.0), -w[:4], rtol=1e-14)
    # x = [1, 1]: mean square 1, so the output is 1 / sqrt(1 + eps)
    assert np.allclose(toy.rms_norm(np.ones(2), np.ones(2), 0.25), 1 / np.sqrt(1.25), rtol=1e-14)


def test_rope_hand_values_pin_convention_and_frequencies():
    """Rotate-half pairs (i, i + d/2) with frequency theta^(-2i/d): at d = 4,
    theta = 100, position 3, pair 0 turns by 3 rad and pair 1 by 0.3 rad; the
    first half takes x1 cos - x2 sin, the second x2 cos + x1 sin."""
    x = np.array([[[1.0, 0.0, 0.0, 0.0]], [[0.0, 1.0, 0.0, 0.0]], [[0.0, 0.0, 1.0, 0.0]]])
    out = toy.rope(x, [3, 3, 3], 100.0)
    c3, s3, c03, s03 = np.cos(3.0), np.sin(3.0), np.cos(0.3), np.sin(0.3)
    assert np.allclose(out[0, 0], [c3, 0.0, s3, 0.0], atol=1e-15)
    assert np.allclose(out[1, 0], [0.0, c03, 0.0, s03], atol=1e-15)
    assert np.allclose(out[2, 0], [-s3, 0.0, c3, 0.0], atol=1e-15)
    assert np.allclose(out[0, 0, [0, 2]], [-0.9899924966004454, 0.1411200080598672], atol=1e-15)


def test_rope_identity_at_zero_norms_and_relative_position():
    """Position 0 leaves vectors unchanged, every pair keeps its length, and
    q.k after rotation depends on the positions only through their offset."""
    rng = np.random.default_rng(1)
    d, theta = 16, 1e4
    x = rng.standard_normal((5, 2, d))
    assert np.allclose(toy.rope(x, np.zeros(5), theta), x, atol=0)
    r = toy.rope(x, np.arange(5) + 11, theta)
    h = d // 2
    assert np.allclose(x[..., :h] ** 2 + x[..., h:] ** 2, r[..., :h] ** 2 + r[..., h:] ** 2,
                       rtol=1e-12)
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    def dot(m, n):
        return float(np.sum(toy.rope(q, [m], theta) * toy.rope(k, [n], theta)))
    assert np.isclose(dot(7, 3), dot(107, 103), rtol=1e-10)
    assert np.isclose(dot(0, 0), float(np.sum(q * k)), rtol=1e-13)
    assert not np.isclose(dot(7, 3), dot(7, 4), rtol=1e-6)


def test_silu_hand_value_and_odd_part():
    """silu(x) = x * sigmoid(x): silu(0) = 0, silu(1) = 1 / (1 + 1/e), and
    silu(x) - silu(-x) = x for every x; large x passes through."""
    assert toy.silu(0.0) == 0.0
    assert np.isclose(toy.silu(1.0), 0.7310585786300049, rtol=1e-15)
    x = np.linspace(-20, 20, 81)
    assert np.allclose(toy.silu(x) - toy.silu(-x), x, atol=1e-12)
    assert np.isclose(toy.silu(40.0), 40.0, rtol=1e-15)


def _tiny_model(seed=3, std=0.1):
    cfg = dict(synth.TOY_TINY)
    return cfg, synth.toy_params(cfg, seed=seed, std=std)


def test_forward_prompt_pass_equals_token_by_token_with_the_cache():
    """One dense pass over T tokens gives the same logits as T single-token
    passes that read the cache the earlier ones wrote (positions, causal
    masking and cache writes agree)."""
    cfg, p = _tiny_model()
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, cfg["hidden"]))
    c1 = toy.Cache(cfg["n_layers"], cfg["n_kv_heads"], 16, cfg["head_dim"])
    full = toy.forward(p, x, np.arange(9), c1)
    c2 = toy.Cache(cfg["n_layers"], cfg["n_kv_heads"], 16, cfg["head_dim"])
    step = np.concatenate([toy.forward(p, x[i:i + 1], [i], c2) for i in range(9)])
    assert np.allclose(full, step, rtol=1e-11, atol=1e-12)
    assert np.allclose(c1.k, c2.k) and np.allclose(c1.v, c2.v)


def test_forward_is_causal_and_zero_projections_leave_the_residual():
    """A later token cannot change earlier logits; with every attention
    output and MLP down projection zero the layers add nothing, so the
    logits equal those of the same model with no layers."""
    cfg, p = _tiny_model()
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, cfg["hidden"]))
    cache = lambda: toy.Cache(cfg["n_layers"], cfg["n_kv_heads"], 8, cfg["head_dim"])  # noqa: E731
    a = toy.forward(p, x, np.arange(6), cache())
    x2 = x.copy()
    x2[5] += 3.0
    b = toy.forward(p, x2, np.arange(6), cache())
    assert np.allclose(a[:5], b[:5], rtol=0, atol=0) and not np.allclose(a[5], b[5])
    z = dict(p, layers=[dict(lp, wo=np.zeros_like(lp["wo"]), w_down=np.zeros_like(lp["w_down"]))
                        for lp in p["layers"]])
    bare = dict(p, layers=[])
    assert np.allclose(toy.forward(z, x, np.arange(6), cache()),
                       toy.forward(bare, x, np.arange(6), cache()), rtol=1e-14, atol=0)


def test_forward_sparse_over_every_visual_key_is_dense():
    """The draft model with every visual position selected is the dense
    model (forward level of sparse(K = vis_len) = dense)."""
    cfg, p = _tiny_model()
    rng = np.random.default_rng(6)
    n_vis, n = 12, 15
    x = rng.standard_normal((n, cfg["hidden"]))
    c = toy.Cache(cfg["n_layers"], cfg["n_kv_heads"], 20, cfg["head_dim"])
    toy.forward(p, x[:n - 1], np.arange(n - 1), c)
    c_s = toy.Cache(cfg["n_layers"], cfg["n_kv_heads"], 20, cfg["head_dim"])
    c_s.k, c_s.v, c_s.length = c.k.copy(), c.v.copy(), c.length
    dense = toy.forward(p, x[n - 1:], [n - 1], c)
    idx = [np.tile(np.arange(n_vis), (cfg["n_kv_heads"], 1)) for _ in range(cfg["n_layers"])]
    sparse = toy.forward(p, x[n - 1:], [n - 1], c_s, "sparse", idx, (0, n_vis))
    assert np.allclose(dense, sparse, rtol=1e-12, atol=1e-13)
    idx_small = [np.tile(np.arange(2), (cfg["n_kv_heads"], 1)) for _ in range(cfg["n_layers"])]
    c_t = toy.Cache(cfg["n_layers"], cfg["n_kv_heads"], 20, cfg["head_dim"])
    c_t.k, c_t.v, c_t.length = c.k.copy(), c.v.copy(), c.length
    assert not np.allclose(dense, toy.forward(p, x[n - 1:], [n - 1], c_t, "sparse", idx_small,
                                              (0, n_vis)))
