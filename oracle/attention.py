"""Oracle for attention, split-KV decode partials and the merge of partial states.

Test infrastructure only (see the package docstring).

What is computed, and where the pages define it:

* ``attention`` -- the unfused three-stage safe softmax of the scaled scores
  followed by the product with V ("RedFuser episode transcript", cue 9: row
  max, then the sum of exponentials relative to it, then the division; the
  cascade is GEMM, softmax, GEMM). The log-sum-exp is m + ln(l) of the scaled
  scores (natural log; the pages do not define it, so this is the plainest
  reading). Parity: pinned by the worked example of cue 15, by closed forms
  (causal first row, zero queries, a single key) and by torch's
  scaled_dot_product_attention run in float64 on the CPU.

* ``attention_online`` -- the one-pass form: a running max m, a running
  denominator l and a running accumulator, all rescaled by exp(m_old - m_new)
  when a tile raises the max, divided by l once at the end (transcript cues
  15, 17, 19; visual explainer "Online softmax, step by step" and "Rescale the
  output accumulator too"). It is a self-check of the oracle: it must equal
  ``attention`` to float64 rounding. When the running max is still -inf the
  correction factor is taken as 1 (transcript cue 29: where the factor is not
  invertible the identity element is substituted).

* ``decode_partials`` -- the per-segment partial states (m_s, l_s, acc_s) of
  the Multi-Segment strategy (transcript cue 39; visual explainer
  "Single-Segment vs Multi-Segment"). Segment s covers keys
  [s*L_s, min((s+1)*L_s, Lk)) with L_s = ceil(Lk / S); an empty segment is the
  identity state (-inf, 0, 0). acc_s is NOT normalised and is relative to m_s.

* ``merge_states`` -- the merge of partial states, each with its own max,
  by rescaling to the common max and adding (transcript cue 21; visual
  explainer "Merging partial states across blocks (FlashDecoding-style)").
  A state with m_s = -inf has weight 0; if every state is the identity the
  output row is 0 and its log-sum-exp is -inf. Parity: pinned by the
  invariant that every segmentation of the keys, merged, equals the unsplit
  attention (brute force over all compositions of small Lk), by associativity
  and commutativity of the merge (transcript cue 27: the combining operator
  is a commutative monoid with an identity) and by the worked example.

GQA head mapping: query head h reads key/value head h // (Hq // Hkv)
(contiguous groups). Causal masking: key j is visible to query i iff j <= i,
with Lq == Lk.
"""

import math

import numpy as np

NEG_INF = -math.inf


def _f64(x):
    """Exact upcast of a numpy array or a torch CPU tensor to float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only for the dtype conversion of torch inputs

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, scale, causal=False):
    """Unfused safe-softmax attention.

    q: [B, Hq, Lq, d]; k: [B, Hkv, Lk, d]; v: [B, Hkv, Lk, dv] (any float
    dtype, upcast exactly; dv may differ from d, as in multi-latent attention
    where the values are the first dv columns of the shared latent rows).
    Returns (o [B, Hq, Lq, dv] float64, lse [B, Hq, Lq] float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    dv = v.shape[-1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and Lq != Lk:
        raise ValueError("causal attention is defined here for Lq == Lk only")
    group = Hq // Hkv
    o = np.zeros((B, Hq, Lq, dv))
    lse = np.zeros((B, Hq, Lq))
    if causal:
        visible = np.tril(np.ones((Lq, Lk), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            # GEMM 1: the score matrix.
            s = scale * (q[b, h] @ k[b, hk].T)
            if causal:
                s = np.where(visible, s, NEG_INF)
            # Stage 1: row max.
            m = s.max(axis=1)
            # Stage 2: denominator relative to that max.
            e = np.exp(s - m[:, None])
            l = e.sum(axis=1)
            # Stage 3: divide, then GEMM 2 with V.
            p = e / l[:, None]
            o[b, h] = p @ v[b, hk]
            lse[b, h] = m + np.log(l)
    return o, lse


def attention_online(q, k, v, scale, causal=False, tile=64):
    """One-pass attention over key tiles of ``tile`` keys with running (m, l, acc).

    Same arguments and results as ``attention``. Also returns the list of
    per-tile running states of head (0, 0), row 0, as (m, l, acc[0]) tuples
    after each tile, so the worked example can check the intermediate values.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    dv = v.shape[-1]
    group = Hq // Hkv
    o = np.zeros((B, Hq, Lq, dv))
    lse = np.zeros((B, Hq, Lq))
    trace = []
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            for i in range(Lq):
                m = NEG_INF
                l = 0.0
                acc = np.zeros(dv)
                for t0 in range(0, Lk, tile):
                    t1 = min(t0 + tile, Lk)
                    scores = scale * (k[b, hk, t0:t1] @ q[b, h, i])
                    if causal:
                        keys = np.arange(t0, t1)
                        scores = np.where(keys <= i, scores, NEG_INF)
                    m_new = max(m, scores.max())
                    # Correction factor for everything accumulated so far.
                    alpha = 1.0 if m_new == NEG_INF else math.exp(m - m_new)
                    if m_new == NEG_INF:
                        p = np.zeros_like(scores)
                    else:
                        p = np.exp(scores - m_new)
                    l = alpha * l + p.sum()
                    acc = alpha * acc + p @ v[b, hk, t0:t1]
                    m = m_new
                    if b == 0 and h == 0 and i == 0:
                        trace.append((m, l, acc[0]))
                o[b, h, i] = acc / l
                lse[b, h, i] = m + math.log(l)
    return o, lse, trace


def segment_bounds(Lk, S):
    """Key ranges of the S segments: ceil-div length, trailing ranges may be empty."""
    seg = -(-Lk // S)
    return [(min(s * seg, Lk), min((s + 1) * seg, Lk)) for s in range(S)]


def decode_partials(q, k, v, scale, S, bounds=None):
    """Per-segment partial states for single-query decode.

    q: [B, Hq, d]; k: [B, Hkv, Lk, d]; v: [B, Hkv, Lk, dv]. ``bounds``
    optionally replaces the ceil-div segmentation by an explicit list of S
    (start, end) key ranges. Returns m [B, Hq, S], l [B, Hq, S],
    acc [B, Hq, S, dv] (float64), acc unnormalised and relative to m.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    dv = v.shape[-1]
    group = Hq // Hkv
    if bounds is None:
        bounds = segment_bounds(Lk, S)
    if len(bounds) != S:
        raise ValueError("need one key range per segment")
    m = np.full((B, Hq, S), NEG_INF)
    l = np.zeros((B, Hq, S))
    acc = np.zeros((B, Hq, S, dv))
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            for s, (t0, t1) in enumerate(bounds):
                if t0 == t1:
                    continue  # identity state
                scores = scale * (k[b, hk, t0:t1] @ q[b, h])
                m_s = scores.max()
                e = np.exp(scores - m_s)
                m[b, h, s] = m_s
                l[b, h, s] = e.sum()
                acc[b, h, s] = e @ v[b, hk, t0:t1]
    return m, l, acc


def merge_states(m, l, acc):
    """Merge S partial states per row.

    m, l: [..., S]; acc: [..., S, d]. Returns (o [..., d], lse [...]) float64.
    """
    m, l, acc = _f64(m), _f64(l), _f64(acc)
    m_star = m.max(axis=-1)
    finite = np.isfinite(m_star)
    safe_star = np.where(finite, m_star, 0.0)
    w = np.where(np.isfinite(m), np.exp(m - safe_star[..., None]), 0.0)
    w = np.where(finite[..., None], w, 0.0)
    l_tot = (w * l).sum(axis=-1)
    num = (w[..., None] * acc).sum(axis=-2)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l_tot[..., None] > 0, num / np.where(l_tot > 0, l_tot, 1.0)[..., None], 0.0)
        lse = np.where(finite, m_star + np.log(np.where(l_tot > 0, l_tot, 1.0)), NEG_INF)
    return o, lse


def merge_pair(a, b):
    """Merge two single-row states (m, l, acc) into one; the monoid's operation."""
    ma, la, acca = a
    mb, lb, accb = b
    m = max(ma, mb)
    if m == NEG_INF:
        return (NEG_INF, 0.0, np.zeros_like(acca))
    wa = 0.0 if ma == NEG_INF else math.exp(ma - m)
    wb = 0.0 if mb == NEG_INF else math.exp(mb - m)
    return (m, wa * la + wb * lb, wa * np.asarray(acca) + wb * np.asarray(accb))
