"""Oracle: the sparse draft attention and the dense verify attention (float64).

Test infrastructure only (see the package docstring).

Shared conventions (readings where the pages are silent):
* GQA grouping: query head h reads KV head floor(h / G), G = H_q / H_kv.
* scale defaults to 1/sqrt(d); no soft-cap, no positional bias.  Q and K are
  taken as given (already rotated, if the model rotates them).
* ``length`` counts every valid cache position, including the positions of
  the queries being processed; queries are bottom-right aligned, so query i
  of n_q sits at position length - n_q + i and sees keys [0, that position].
"""

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attend(q, keys, values, scale):
    """Textbook softmax attention of one query over a list of key rows.

    out = sum_j softmax_j(scale * q.k_j) v_j, computed with the max subtracted
    before exponentiation (exact in real arithmetic, overflow-free in f64).
    """
    q, keys, values = _f64(q), _f64(keys), _f64(values)
    if keys.shape[0] == 0:
        raise ValueError("attention over an empty key set is undefined")
    s = scale * (keys @ q)
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ values


def dense_verify(q, k, v, length, scale=None):
    """Dense model M: causal attention of n_q queries over the full KV cache.

    Follows the StD technical summary, Methodology item 2 (the dense model
    uses the full KV cache, i.e. standard attention) and item 3 (the dense
    model verifies the gamma drafted tokens in parallel).  The single pass
    over the cache is a property of the GPU kernel, not of the result, so
    this is the plain definition evaluated query by query.

    q: [n_q][H_q][d]; k, v: [H_kv][capacity][d].  Returns [n_q][H_q][d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_q, hq, d = q.shape
    hkv = k.shape[0]
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    if not (1 <= n_q <= length <= k.shape[1]):
        raise ValueError("need 1 <= n_q <= length <= capacity")
    g_size = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.empty((n_q, hq, d))
    for i in range(n_q):
        pos = length - n_q + i
        for h in range(hq):
            g = h // g_size
            out[i, h] = attend(q[i, h], k[g, : pos + 1], v[g, : pos + 1], scale)
    return out


def row_lse(q, k, length, scale=None):
    """Natural-log softmax normaliser of every query row of ``dense_verify``.

    Query i of n_q (position length - n_q + i) of head h has
    lse = log sum_{j <= position} exp(scale * q.k_j), the log of the
    denominator of its causal softmax: the value a prefill attention returns
    beside its output, which the selection's first step (the text rows'
    normalisers; technical summary, Methodology item 4) then need not
    recompute.  Evaluated with the row maximum taken out before the
    exponentials (exact in real arithmetic).

    q: [n_q][H_q][d]; k: [H_kv][capacity][d].  Returns [n_q][H_q].
    """
    q, k = _f64(q), _f64(k)
    n_q, hq, d = q.shape
    hkv = k.shape[0]
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    if not (1 <= n_q <= length <= k.shape[1]):
        raise ValueError("need 1 <= n_q <= length <= capacity")
    g_size = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.empty((n_q, hq))
    for i in range(n_q):
        pos = length - n_q + i
        for h in range(hq):
            s = scale * (k[h // g_size, : pos + 1] @ q[i, h])
            mx = s.max()
            out[i, h] = mx + math.log(np.exp(s - mx).sum())
    return out


def sparse_key_set(length, vis_start, vis_len, idx_g):
    """Positions seen by the sparse model M_s for one KV head.

    All non-visual positions are kept and the visual span is replaced by the
    selected top-K visual positions (technical summary, Methodology item 2:
    top-K attention keeps only the most relevant visual KV; item 4: selection
    is over the visual KV).  Reading: prefix text, prompt text and every
    generated or drafted position are all kept.
    """
    vis_end = vis_start + vis_len
    idx_g = np.asarray(idx_g, dtype=np.int64)
    if idx_g.size and (idx_g.min() < vis_start or idx_g.max() >= vis_end):
        raise ValueError("selected positions must lie inside the visual span")
    if len(np.unique(idx_g)) != idx_g.size:
        raise ValueError("selected positions must be distinct")
    return np.concatenate([
        np.arange(0, vis_start, dtype=np.int64),
        np.sort(idx_g),
        np.arange(vis_end, length, dtype=np.int64),
    ])


def sparse_decode(q, k, v, length, vis_start, vis_len, idx, scale=None):
    """Sparse model M_s: one decode query over the sparse key set.

    The query sits at position length-1 and attends, per KV head g, to
    [0, vis_start) + idx[g] + [vis_start+vis_len, length) with textbook
    softmax attention (technical summary, Methodology items 2 and 3: the
    sparse model drafts autoregressively with top-K attention).

    q: [H_q][d]; k, v: [H_kv][capacity][d]; idx: [H_kv][K].  Returns [H_q][d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    hq, d = q.shape
    hkv = k.shape[0]
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    if not (vis_start + vis_len <= length <= k.shape[1]):
        raise ValueError("the visual span must end before length")
    g_size = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    idx = np.asarray(idx).reshape(hkv, -1)
    out = np.empty((hq, d))
    for g in range(hkv):
        keep = sparse_key_set(length, vis_start, vis_len, idx[g])
        for h in range(g * g_size, (g + 1) * g_size):
            out[h] = attend(q[h], k[g, keep], v[g, keep], scale)
    return out
