"""Oracle for the MoE routing cascade: row softmax, then top-k, then renormalise.

Test infrastructure only (see the package docstring).

The cascade is named in "RedFuser episode transcript", cue 11 (MoE routing is
softmax followed by top-k) and in the bookshelf explainer's section "Problem";
"Online normalizer calculation for softmax" (abstract) reports softmax and
top-k fused into one pass. The pages do not say how ties are broken or in which
order the k results are returned; the reading taken is: experts are ordered by
logit descending, equal logits by expert index ascending, and the first k are
returned in that order. Ordering by the fp32 logit is the same as ordering by
the probability because the softmax is strictly increasing within a row, and it
keeps distinct logits distinct where their probabilities might collide.

Weights: with ``renormalize`` the selected probabilities are divided by their
own sum (so they sum to 1), otherwise they are the softmax probabilities
themselves.

Parity: pinned by brute force (Python ``sorted`` over (-x, j)) on tiny rows,
by tie-heavy rows drawn from a few values, by torch.softmax in float64, and
by the invariants sum(w) = 1 and w non-increasing along the output.
"""

import numpy as np


def softmax_rows(x):
    """Three-stage safe softmax of each row of x (float64)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)          # stage 1: max
    e = np.exp(x - m)
    l = e.sum(axis=-1, keepdims=True)          # stage 2: denominator
    return e / l                               # stage 3: divide


def softmax_topk(logits, k, renormalize=True):
    """logits: [T, E] float32 values. Returns (weights [T, k] float64, idx [T, k] int32)."""
    x = np.asarray(logits, dtype=np.float64)
    T, E = x.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    p = softmax_rows(x)
    # Stable sort of -x keeps equal logits in ascending index order.
    order = np.argsort(-x, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, order, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w, order.astype(np.int32)
