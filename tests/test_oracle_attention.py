"""Pins for the oracle's attention (sparse draft and dense verify), CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_golden_three_keys(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attention_three_keys.json")))
    q = np.array(g["q"])[None, None]                      # n_q=1, H_q=1
    k = np.array(g["k"])[None]
    v = np.array(g["v"])[None]
    out = oracle.dense_verify(q, k, v, length=3, scale=g["scale"])
    np.testing.assert_allclose(out[0, 0], g["out"], atol=g["tol"], rtol=0)


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(1)
    k, v = _rand(rng, 2, 5, 8), _rand(rng, 2, 5, 8)
    q = _rand(rng, 5, 4, 8)                               # n_q = length = 5
    out = oracle.dense_verify(q, k, v, length=5)
    # the first query sits at position 0 and sees only key 0
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[h // 2, 0], atol=1e-15, rtol=0)


def test_equal_logits_give_mean_of_visible_values():
    rng = np.random.default_rng(2)
    k, v = _rand(rng, 1, 9, 16), _rand(rng, 1, 9, 16)
    q = np.zeros((3, 2, 16))                              # all logits 0
    out = oracle.dense_verify(q, k, v, length=9)
    for i in range(3):
        pos = 9 - 3 + i
        for h in range(2):
            np.testing.assert_allclose(out[i, h], v[0, : pos + 1].mean(0), atol=1e-14, rtol=0)


def test_constant_values_pass_through():
    """Softmax rows sum to 1: with every value row equal to c the output is c."""
    rng = np.random.default_rng(3)
    k = _rand(rng, 2, 40, 8) * 4
    v = np.broadcast_to(np.arange(8.0), (2, 40, 8)).copy()
    q = _rand(rng, 4, 6, 8) * 4
    out = oracle.dense_verify(q, k, v, length=37)
    np.testing.assert_allclose(out, np.broadcast_to(np.arange(8.0), out.shape), atol=1e-12, rtol=0)
    idx = np.array([[1, 5, 9], [0, 2, 30]])
    o2 = oracle.sparse_decode(q[0], k, v, 37, 0, 31, idx)
    np.testing.assert_allclose(o2, np.broadcast_to(np.arange(8.0), o2.shape), atol=1e-12, rtol=0)


def test_causality_future_keys_do_not_matter():
    rng = np.random.default_rng(4)
    k, v = _rand(rng, 2, 30, 8), _rand(rng, 2, 30, 8)
    q = _rand(rng, 4, 4, 8)
    a = oracle.dense_verify(q, k, v, length=30)
    k2, v2 = k.copy(), v.copy()
    k2[:, 28:] += 5.0                                     # positions after query 1 (pos 27)
    v2[:, 28:] -= 3.0
    b = oracle.dense_verify(q, k2, v2, length=30)
    assert np.array_equal(a[:2], b[:2])                   # queries at 26, 27 unchanged
    assert not np.allclose(a[2:], b[2:])


def test_verify_row_equals_single_query_dense_decode():
    """Row i of the verify pass is the dense n_q=1 decode at that length."""
    rng = np.random.default_rng(5)
    k, v = _rand(rng, 2, 64, 16), _rand(rng, 2, 64, 16)
    q = _rand(rng, 6, 6, 16)
    out = oracle.dense_verify(q, k, v, length=60)
    for i in range(6):
        one = oracle.dense_verify(q[i:i + 1], k, v, length=60 - 6 + i + 1)
        np.testing.assert_allclose(out[i], one[0], atol=1e-12, rtol=0)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (7, 1)])
def test_dense_matches_torch_sdpa_float64(hq, hkv):
    """Independent library routine: torch SDPA in float64 on the CPU."""
    rng = np.random.default_rng(6 + hq)
    d, length, n_q = 32, 50, 5
    k, v = _rand(rng, hkv, 55, d), _rand(rng, hkv, 55, d)
    q = _rand(rng, n_q, hq, d)
    out = oracle.dense_verify(q, k, v, length=length)
    G = hq // hkv
    kt = torch.from_numpy(k[:, :length]).repeat_interleave(G, dim=0)   # [hq][L][d]
    vt = torch.from_numpy(v[:, :length]).repeat_interleave(G, dim=0)
    qt = torch.from_numpy(q).permute(1, 0, 2)                           # [hq][n_q][d]
    pos = torch.arange(length - n_q, length)[:, None]
    mask = torch.arange(length)[None, :] <= pos                         # bottom-right causal
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt.contiguous(), kt.contiguous(), vt.contiguous(), attn_mask=mask)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


def test_sparse_with_all_visual_equals_dense():
    """Special case: selecting every visual key makes the sparse model dense."""
    rng = np.random.default_rng(7)
    hkv, hq, d = 2, 6, 16
    vis_start, vis_len, length = 3, 40, 52
    k, v = _rand(rng, hkv, 60, d), _rand(rng, hkv, 60, d)
    q = _rand(rng, hq, d)
    idx = np.tile(np.arange(vis_start, vis_start + vis_len), (hkv, 1))
    s = oracle.sparse_decode(q, k, v, length, vis_start, vis_len, idx)
    dn = oracle.dense_verify(q[None], k, v, length)[0]
    np.testing.assert_allclose(s, dn, atol=1e-12, rtol=0)


def test_sparse_matches_sdpa_on_compacted_cache():
    """The sparse key set, built by hand, fed to torch SDPA (float64)."""
    rng = np.random.default_rng(8)
    hkv, hq, d = 2, 4, 8
    vis_start, vis_len, length = 2, 20, 30
    k, v = _rand(rng, hkv, 32, d), _rand(rng, hkv, 32, d)
    q = _rand(rng, hq, d)
    idx = np.array([[3, 7, 8, 21], [2, 10, 11, 12]])
    s = oracle.sparse_decode(q, k, v, length, vis_start, vis_len, idx)
    for g in range(hkv):
        keep = [0, 1] + list(idx[g]) + list(range(22, 30))  # prefix, picks, text
        kt = torch.from_numpy(k[g, keep])[None]
        vt = torch.from_numpy(v[g, keep])[None]
        for h in range(g * 2, g * 2 + 2):
            qt = torch.from_numpy(q[h])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0]
            np.testing.assert_allclose(s[h], ref.numpy(), atol=1e-12, rtol=0)


def test_sparse_rejects_bad_index_sets():
    rng = np.random.default_rng(9)
    k, v = _rand(rng, 1, 20, 4), _rand(rng, 1, 20, 4)
    q = _rand(rng, 1, 4)
    with pytest.raises(ValueError):
        oracle.sparse_decode(q, k, v, 20, 0, 10, np.array([[3, 3]]))    # duplicate
    with pytest.raises(ValueError):
        oracle.sparse_decode(q, k, v, 20, 0, 10, np.array([[3, 12]]))   # outside span


def test_scale_default_is_inverse_sqrt_d():
    rng = np.random.default_rng(10)
    k, v = _rand(rng, 1, 10, 16), _rand(rng, 1, 10, 16)
    q = _rand(rng, 2, 1, 16)
    a = oracle.dense_verify(q, k, v, 10)
    b = oracle.dense_verify(q, k, v, 10, scale=1 / math.sqrt(16))
    assert np.array_equal(a, b)
    c = oracle.dense_verify(q, k, v, 10, scale=1.0)
    assert not np.allclose(a, c)


# ------------------------------------------------------------------ row LSE
def test_row_lse_single_key_is_the_logit():
    """One visible key: the normaliser is that key's scaled logit exactly."""
    rng = np.random.default_rng(41)
    q = rng.standard_normal((1, 3, 16))
    k = rng.standard_normal((1, 4, 16))
    lse = oracle.row_lse(q, k, 1, scale=0.3)
    assert np.allclose(lse[0], 0.3 * (q[0] @ k[0, 0]), rtol=0, atol=1e-15)


def test_row_lse_equal_logits_is_log_count():
    """q = 0 makes every logit 0, so row i (position p) has lse = log(p + 1)."""
    q = np.zeros((5, 4, 8))
    k = np.random.default_rng(42).standard_normal((2, 30, 8))
    lse = oracle.row_lse(q, k, 23)
    pos = 23 - 5 + np.arange(5)
    assert np.allclose(lse, np.log(pos + 1.0)[:, None], rtol=0, atol=1e-14)


def test_row_lse_shift_by_a_direction_of_q():
    """Adding t * u to every key, with u a unit vector along q, shifts every
    logit by scale * t * |q| and so the normaliser by the same amount."""
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 50, 32))
    u = q[0, 0] / np.linalg.norm(q[0, 0])
    t, scale = 2.5, 0.2
    base = oracle.row_lse(q, k, 50, scale=scale)
    moved = oracle.row_lse(q, k + t * u, 50, scale=scale)
    assert abs(moved[0, 0] - base[0, 0] - scale * t * np.linalg.norm(q[0, 0])) < 1e-12


def test_row_lse_normalises_the_dense_rows():
    """exp(s - lse) over each row's visible keys sums to 1, and weighting the
    values with it reproduces dense_verify: the normaliser is the softmax
    denominator of the same rows (GQA, several queries, causal rows)."""
    rng = np.random.default_rng(44)
    hq, hkv, d, n_q, length = 6, 2, 16, 4, 37
    q = rng.standard_normal((n_q, hq, d)) * 1.3
    k = rng.standard_normal((hkv, 40, d))
    v = rng.standard_normal((hkv, 40, d))
    lse = oracle.row_lse(q, k, length)
    out = oracle.dense_verify(q, k, v, length)
    for i in range(n_q):
        pos = length - n_q + i
        for h in range(hq):
            g = h // (hq // hkv)
            w = np.exp(k[g, : pos + 1] @ q[i, h] / np.sqrt(d) - lse[i, h])
            assert abs(w.sum() - 1.0) < 1e-12
            assert np.max(np.abs(w @ v[g, : pos + 1] - out[i, h])) < 1e-12


def test_row_lse_matches_scipy_logsumexp():
    """An independent library routine on the masked logits."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(45)
    hq, hkv, d, n_q, length = 4, 1, 8, 3, 20
    q = rng.standard_normal((n_q, hq, d)) * 2.0
    k = rng.standard_normal((hkv, 25, d))
    lse = oracle.row_lse(q, k, length, scale=0.7)
    for i in range(n_q):
        pos = length - n_q + i
        for h in range(hq):
            assert abs(lse[i, h] - logsumexp(0.7 * (k[0, : pos + 1] @ q[i, h]))) < 1e-12
