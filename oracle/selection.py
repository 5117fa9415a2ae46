"""Oracle: prefill-time top-K visual KV selection (float64).

Test infrastructure only (see the package docstring).

Follows the StD technical summary, Methodology item 4 ("KV cache
selection"): the top-K visual KV are chosen once, during prefill, from the
average attention score that text tokens direct at visual tokens, and the
choice differs per layer and per attention head; item 2 names the basis as
the attention weights from text tokens to visual tokens.

Readings where the pages leave a step open:
* score = post-softmax probability of the prefill's own causal attention row
  of each text query (normalised over every key that query sees: the prefix,
  the whole visual span and the text up to and including itself), summed over
  the visual columns only;
* text queries = the prompt text tokens that follow the visual span;
* one index set per (layer, KV head): the mean runs over the text rows and
  the G query heads that share the KV head (the mean, not the sum, but the
  ranking is the same);
* ties in the ranking go to the lower position, and the selected set is
  returned in ascending position order.

This is a heuristic, so the oracle takes the algorithm's steps in order:
(1) softmax of each text row, (2) mean over rows and the head group,
(3) rank by (-score, position) and keep the first K.
"""

import math

import numpy as np


def selection_scores(q_text, k, text_start, vis_start, vis_len, scale=None,
                     row_block=256):
    """Mean text->visual softmax probability per (KV head, visual position).

    q_text: [H_q][n_text][d], the text queries of the prefill (text row i sits
    at position text_start + i).  k: [H_kv][capacity][d].
    Returns scores [H_kv][vis_len] (float64).

    Rows are evaluated ``row_block`` at a time only to bound memory; each row
    is an independent softmax and the per-row arithmetic is the definition.
    """
    q_text = np.asarray(q_text, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, n_text, d = q_text.shape
    hkv = k.shape[0]
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    vis_end = vis_start + vis_len
    if n_text < 1 or vis_len < 1:
        raise ValueError("need at least one text row and one visual position")
    if text_start < vis_end:
        raise ValueError("text rows must follow the visual span")
    if text_start + n_text > k.shape[1]:
        raise ValueError("text rows exceed the cache")
    g_size = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    scores = np.zeros((hkv, vis_len))
    for h in range(hq):
        g = h // g_size
        for r0 in range(0, n_text, row_block):
            r1 = min(n_text, r0 + row_block)
            pos = text_start + np.arange(r0, r1)          # position of each row
            n_keys = int(pos[-1]) + 1
            logits = scale * (q_text[h, r0:r1] @ k[g, :n_keys].T)
            visible = np.arange(n_keys)[None, :] <= pos[:, None]
            logits = np.where(visible, logits, -np.inf)
            logits = logits - logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p = p / p.sum(axis=1, keepdims=True)          # softmax of each row
            scores[g] += p[:, vis_start:vis_end].sum(axis=0)
    scores /= g_size * n_text
    return scores


def rank_topk(scores_g, topk):
    """Positions (0-based within the visual span) of the K largest scores.

    Order is (-score, position): ties go to the lower position.  The chosen
    set is returned sorted ascending.
    """
    s = np.asarray(scores_g, dtype=np.float64)
    if not (1 <= topk <= s.size):
        raise ValueError("need 1 <= topk <= vis_len")
    order = np.lexsort((np.arange(s.size), -s))   # primary key: -score
    return np.sort(order[:topk])


def select_topk(q_text, k, text_start, vis_start, vis_len, topk, scale=None):
    """Top-K visual positions per KV head, as absolute cache positions.

    Returns (idx [H_kv][K] int64 ascending absolute positions,
             scores [H_kv][vis_len] float64).
    """
    scores = selection_scores(q_text, k, text_start, vis_start, vis_len, scale)
    idx = np.stack([rank_topk(scores[g], topk) for g in range(scores.shape[0])])
    return idx + vis_start, scores


def static_window_idx(vis_start, vis_len, sink, topk):
    """Visual positions kept by the streaming-attention comparator.

    The pages compare StD with a streaming-attention draft (technical
    summary, Experimental results) without stating its sizes.  Reading: such
    a policy keeps the first ``sink`` positions of the visual span (the
    attention sink) and, for the rest of a budget of ``topk`` positions, the
    most recent ones (the window); the text KV is kept whole, as for StD.
    Written from that description: the sink is the first s = min(sink, topk)
    positions of the span, the window the last topk - s.

    Returns the absolute positions as an int64 array of length topk, sorted
    ascending.
    """
    if not (0 <= topk <= vis_len) or sink < 0 or vis_start < 0:
        raise ValueError("need 0 <= topk <= vis_len, sink >= 0, vis_start >= 0")
    s = min(sink, topk)
    sink_part = list(range(vis_start, vis_start + s))
    vis_end = vis_start + vis_len
    window_part = list(range(vis_end - (topk - s), vis_end))
    return np.array(sorted(sink_part + window_part), dtype=np.int64)
