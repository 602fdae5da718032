"""Oracle for the MoE router (test infrastructure only; the product path
never imports it).

The toolchain write-up ("MetaX-TileLang工具链", section 2.4, the PyTorch
reference of the fused-MoE case) defines the router as: logits from a linear
gate over the token, a softmax over all experts, then the top-k expert ids
with their scores.  It states no renormalisation of the k scores, so none is
applied; the scores are the softmax probabilities themselves.

Readings where the page is silent: logits and softmax in float64 here (the
kernel's are float32; the page fixes no precision); among equal scores the
lower expert index ranks first; the k results are in decreasing score order.
"""
from __future__ import annotations

import numpy as np


def router_logits(x16, w16) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W[e, h] in float64 (x [T, H] and W [E, H]
    fp16 values, widened exactly)."""
    x = np.asarray(x16, dtype=np.float64)
    w = np.asarray(w16, dtype=np.float64)
    return x @ w.T


def softmax(logits) -> np.ndarray:
    """Row-wise softmax over the experts, shifted by the row maximum."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def topk(scores, k: int):
    """The k largest scores per row, decreasing; equal scores by ascending
    expert index.  Returns (ids [T, k] int32, values [T, k] float64)."""
    s = np.asarray(scores, dtype=np.float64)
    if not 0 <= k <= s.shape[1]:
        raise ValueError("k out of range")
    order = np.argsort(-s, axis=1, kind="stable")[:, :k]
    return order.astype(np.int32), np.take_along_axis(s, order, axis=1)


def route(x16, w16, k: int):
    """Router of one batch: (ids, scores, all softmax scores)."""
    p = softmax(router_logits(x16, w16))
    ids, vals = topk(p, k)
    return ids, vals, p
