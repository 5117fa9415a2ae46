"""Oracle: greedy longest-prefix acceptance plus the bonus token.

Test infrastructure only (see the package docstring).

Follows the StD technical summary, Methodology item 3 ("decoding
procedure"): verification finds the longest prefix of drafted tokens that
agrees with the dense model's predictions (n tokens) and accepts one extra
"bonus" token; the accepted sequence is appended to the context.  The French
lay explanation ("draft and verify team") gives the same rule in words: the
editor keeps the correct words and, at the first wrong one, corrects it and
stops there.

Readings: the dense prediction is the greedy argmax, ties to the lowest
token id; row i of the verify logits is the prediction made after the i-th
verify input (x_t, d_1, ..., d_gamma), so it is compared with d_{i+1}; the
bonus is the dense prediction after the last accepted token (the correction
when n < gamma, an extra token when n == gamma).
"""

import numpy as np


def argmax_margin(row):
    """(argmax with ties to the lowest index, top1 - top2) of one logit row."""
    row = np.asarray(row, dtype=np.float64)
    best = 0
    for j in range(1, row.size):
        if row[j] > row[best]:
            best = j
    if row.size == 1:
        return best, np.inf
    rest = np.delete(row, best)
    with np.errstate(invalid="ignore"):        # a row of -inf: the margin is NaN
        return best, float(row[best] - rest.max())


def accept(draft, logits):
    """Greedy acceptance of ``gamma`` drafted tokens against gamma+1 rows.

    draft: [gamma] int; logits: [gamma+1][vocab].
    Returns (out_tokens [gamma+1] int64, n_out, margins [gamma+1], pred).
    out_tokens[0..n] = d_1..d_n followed by the bonus pred[n]; the entries
    after position n are -1.  n_out = n + 1 lies in [1, gamma + 1].
    """
    draft = np.asarray(draft, dtype=np.int64).reshape(-1)
    logits = np.asarray(logits, dtype=np.float64)
    gamma = draft.size
    if logits.shape[0] != gamma + 1:
        raise ValueError("need gamma+1 logit rows")
    pred = np.empty(gamma + 1, dtype=np.int64)
    margins = np.empty(gamma + 1)
    for i in range(gamma + 1):
        pred[i], margins[i] = argmax_margin(logits[i])
    n = 0
    while n < gamma and draft[n] == pred[n]:
        n += 1
    out = np.full(gamma + 1, -1, dtype=np.int64)
    out[:n] = draft[:n]
    out[n] = pred[n]
    return out, n + 1, margins, pred
