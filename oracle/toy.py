"""Scalar chunk-and-merge on Python floats (TEST INFRASTRUCTURE ONLY).

The www.2kiu.com/news/6053916 article, section "用 log-sum-exp 给块结果定权重",
works a one-dimensional example: each chunk keeps its softmax-normalised
weighted value and the log of its exponent sum; the merge takes a softmax over
those log-sums and uses it to weight the chunk outputs. Its section
"为什么这个反例特别容易看出平均法错误" explains why averaging the chunk outputs
is wrong. These functions restate that procedure for scalar values.
"""
from __future__ import annotations

import math


def chunk_partial(scores, values):
    """Normalised weighted value of one non-empty chunk and its log-sum-exp."""
    if not scores or len(scores) != len(values):
        raise ValueError("a chunk needs at least one key and one value per key")
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = math.fsum(weights)
    mean = math.fsum(w * x for w, x in zip(weights, values)) / total
    return mean, top + math.log(total)


def merge(partials):
    """Combine (output, lse) pairs with weights exp(lse - max lse)."""
    if not partials:
        raise ValueError("nothing to merge: no chunk had a valid key")
    top = max(l for _, l in partials)
    weights = [math.exp(l - top) for _, l in partials]
    return math.fsum(w * o for w, (o, _) in zip(weights, partials)) / math.fsum(weights)


def naive_average(partials):
    """The wrong merge the article rejects: the plain mean of chunk outputs."""
    return sum(o for o, _ in partials) / len(partials)
