"""Dense-mask twin of the selected-set attention (TEST INFRASTRUCTURE).

Written independently of oracle.c, in numpy fp64: it materializes the full
[T, T] logit matrix of one (batch, head), builds a boolean mask from the
selection and the causal rule, and runs a masked softmax.  The technical
report page ("Monodratic: a reproducible sparse attention mixer", section
"Evidence", and the news page's section "Why Learned Product-Hash Routing
Matters Now") compares sparse gathering against exactly such an
independently built dense-mask computation over the same selected positions.
"""
import numpy as np


def _rotate(x, cos, sin):
    """Rotate-half rotary embedding in fp64: x [T, d], cos/sin [T, d/2]."""
    x = np.asarray(x, np.float64)
    h = x.shape[-1] // 2
    c = np.asarray(cos, np.float64)
    s = np.asarray(sin, np.float64)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def dense_masked_attention(q, k, v, cos, sin, sel, beta, L, rows=None):
    """One (batch, q-head): q [T, d], k/v [T, d] of its kv-head, sel [T, R]
    (selected remote blocks, -1 = empty).  Returns [len(rows), d] fp64 for
    the query rows `rows` (all rows if None)."""
    T, d = q.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    qr = _rotate(q[rows], cos[rows], sin[rows])
    kr = _rotate(k, cos[:T], sin[:T])
    logits = (qr @ kr.T) / np.sqrt(d)
    blk_of = np.arange(T) // beta
    mask = np.zeros((len(rows), T), dtype=bool)
    for i, t in enumerate(rows):
        qb = t // beta
        allowed = set(int(x) for x in sel[t] if x >= 0)
        allowed.update(range(max(0, qb - L + 1), qb + 1))
        mask[i] = np.isin(blk_of, list(allowed)) & (np.arange(T) <= t)
    logits = np.where(mask, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    w /= w.sum(axis=1, keepdims=True)
    return w @ np.asarray(v, np.float64)


def dense_causal_attention(q, k, v, cos, sin, rows=None):
    """Textbook dense causal softmax attention of one (batch, head), fp64."""
    T, d = q.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    qr = _rotate(q[rows], cos[rows], sin[rows])
    kr = _rotate(k, cos[:T], sin[:T])
    logits = (qr @ kr.T) / np.sqrt(d)
    causal = np.arange(T)[None, :] <= rows[:, None]
    logits = np.where(causal, logits, -np.inf)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ np.asarray(v, np.float64)
