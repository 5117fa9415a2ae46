"""Oracle: a tiny float64 decoder running plain greedy decoding and the StD loop.

Test infrastructure only (see the package docstring).

The StD loop follows the technical summary, Methodology item 3 ("decoding
procedure"): the sparse model M_s drafts gamma tokens autoregressively, the
dense model M checks them in one parallel pass over the full KV cache, the
longest agreeing prefix plus a bonus token is accepted and appended to the
context.  Item 4: the top-K visual KV per layer and KV head are chosen once,
at prefill, and never re-chosen.  Key contributions, "lossless
acceleration": the output is that of the dense model, which the tests pin by
comparing ``toy_std`` with ``toy_greedy`` token by token.

The decoder itself is not on the pages; it is a small standard pre-norm
transformer (RMSNorm, rotary position embedding, grouped-query attention,
SwiGLU MLP, untied LM head) whose weights are inputs (random, from the
seeded input generators).  The draft model is the same weights with the
attention switched to the sparse key set (Methodology item 2).

Cache handling (reading of "appended to the context"): drafted tokens write
their K/V at their own positions in the one shared cache; the dense pass
rewrites positions t..t+gamma; after acceptance the valid length becomes
t+n+1, so rejected positions are simply overwritten later.
"""

import math

import numpy as np

from .acceptance import accept, argmax_margin
from .attention import dense_verify, sparse_decode
from .selection import select_topk


def rms_norm(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rope(x, positions, theta):
    """Rotary embedding, rotate-half convention: pairs (i, i + d/2)."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    cos, sin = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


class Cache:
    """Per-layer K and V, [H_kv][capacity][d], plus the valid length."""

    def __init__(self, n_layers, hkv, capacity, d):
        self.k = np.zeros((n_layers, hkv, capacity, d))
        self.v = np.zeros((n_layers, hkv, capacity, d))
        self.length = 0


def forward(p, x, positions, cache, mode="dense", idx=None, vis=None,
            want_q_text=None):
    """Run the decoder on embeddings x [T][hidden] at contiguous positions.

    Writes K/V of every layer at ``positions`` and returns logits [T][vocab].
    mode "dense": causal attention over the full cache (dense model M).
    mode "sparse": T must be 1; attention over the sparse key set given by
    ``idx[layer]`` and ``vis`` = (vis_start, vis_len) (sparse model M_s).
    ``want_q_text`` = (row0, row1): also return the rotated queries of those
    rows for every layer (the prefill's text queries).
    """
    cfg = p["cfg"]
    hq, hkv, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    positions = np.asarray(positions, dtype=np.int64)
    n = positions.size
    if n > 1 and not np.all(np.diff(positions) == 1):
        raise ValueError("positions must be contiguous")
    length = int(positions[-1]) + 1
    q_text = []
    for li, lp in enumerate(p["layers"]):
        h = rms_norm(x, lp["attn_norm"], cfg["eps"])
        q = (h @ lp["wq"]).reshape(n, hq, d)
        k = (h @ lp["wk"]).reshape(n, hkv, d)
        v = (h @ lp["wv"]).reshape(n, hkv, d)
        q = rope(q, positions, cfg["rope_theta"])
        k = rope(k, positions, cfg["rope_theta"])
        cache.k[li][:, positions] = k.transpose(1, 0, 2)
        cache.v[li][:, positions] = v.transpose(1, 0, 2)
        if want_q_text is not None:
            q_text.append(q[want_q_text[0]:want_q_text[1]].transpose(1, 0, 2))
        if mode == "dense":
            o = dense_verify(q, cache.k[li], cache.v[li], length)
        elif mode == "sparse":
            if n != 1:
                raise ValueError("the sparse model drafts one token at a time")
            o = sparse_decode(q[0], cache.k[li], cache.v[li], length,
                              vis[0], vis[1], idx[li])[None]
        else:
            raise ValueError(mode)
        x = x + o.reshape(n, hq * d) @ lp["wo"]
        h = rms_norm(x, lp["mlp_norm"], cfg["eps"])
        x = x + (silu(h @ lp["w_gate"]) * (h @ lp["w_up"])) @ lp["w_down"]
    logits = rms_norm(x, p["final_norm"], cfg["eps"]) @ p["lm_head"]
    cache.length = max(cache.length, length)
    return (logits, q_text) if want_q_text is not None else logits


def _greedy_token(row):
    return int(argmax_margin(row)[0])


def prefill(p, vis_emb, text_ids, capacity):
    """Dense prefill of [visual embeddings; text token embeddings].

    Returns (cache, per-layer rotated text queries [H_q][n_text][d], first
    generated token).
    """
    cfg = p["cfg"]
    vis_emb = np.asarray(vis_emb, dtype=np.float64)
    text_ids = np.asarray(text_ids, dtype=np.int64)
    x = np.concatenate([vis_emb, p["embed"][text_ids]], axis=0)
    n_vis = vis_emb.shape[0]
    cache = Cache(len(p["layers"]), cfg["n_kv_heads"], capacity, cfg["head_dim"])
    logits, q_text = forward(p, x, np.arange(x.shape[0]), cache,
                             want_q_text=(n_vis, x.shape[0]))
    return cache, q_text, _greedy_token(logits[-1])


def toy_greedy(p, vis_emb, text_ids, n_new):
    """Plain greedy decoding with the dense model: the losslessness target."""
    prompt_len = len(vis_emb) + len(text_ids)
    cache, _, tok = prefill(p, vis_emb, text_ids, prompt_len + n_new + 1)
    out = [tok]
    t = prompt_len
    while len(out) < n_new:
        logits = forward(p, p["embed"][[tok]], [t], cache)
        tok = _greedy_token(logits[0])
        out.append(tok)
        t += 1
    return out


def toy_std(p, vis_emb, text_ids, n_new, topk, gamma):
    """Sparse-to-Dense decoding.  Returns (tokens, accepted counts per cycle).

    Selection: ``select_topk`` per layer on the prefill's text queries and
    the cached keys (Methodology item 4).  Each cycle: gamma sparse single-
    token steps from the pending token x_t, one dense pass over
    (x_t, d_1..d_gamma), then greedy acceptance (Methodology item 3).
    """
    n_vis = len(vis_emb)
    prompt_len = n_vis + len(text_ids)
    capacity = prompt_len + n_new + gamma + 2
    cache, q_text, x_t = prefill(p, vis_emb, text_ids, capacity)
    idx = [select_topk(q_text[li], cache.k[li], n_vis, 0, n_vis, topk)[0]
           for li in range(len(p["layers"]))]
    out = [x_t]
    accepted = []
    t = prompt_len                                 # position of x_t
    while len(out) < n_new:
        drafts = []
        tok = x_t
        for j in range(gamma):                     # sparse model drafts
            logits = forward(p, p["embed"][[tok]], [t + j], cache, "sparse",
                             idx, (0, n_vis))
            tok = _greedy_token(logits[0])
            drafts.append(tok)
        seq = [x_t] + drafts                       # dense model verifies
        logits = forward(p, p["embed"][seq], np.arange(t, t + gamma + 1), cache)
        toks, n_out, _, _ = accept(np.array(drafts, dtype=np.int64), logits)
        emitted = [int(z) for z in toks[:n_out]]
        accepted.append(n_out - 1)
        out.extend(emitted)
        x_t = emitted[-1]                          # bonus becomes pending
        t += n_out
        cache.length = t
    return out[:n_new], accepted


def model_dims_ok(p):
    cfg = p["cfg"]
    return (cfg["n_q_heads"] % cfg["n_kv_heads"] == 0
            and cfg["head_dim"] % 2 == 0
            and math.isfinite(cfg["eps"]))
