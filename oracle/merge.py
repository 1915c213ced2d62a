"""Log-sum-exp merge of attention computed over disjoint token sets (fp64).

TEST INFRASTRUCTURE ONLY.  Softmax attention over a union of token sets is
a weighted combination of the attention over each set: with o_s the
normalised output and lse_s = ln(sum of exp(score)) over set s,

    lse = ln(sum_s exp(lse_s)),   o = sum_s exp(lse_s - lse) * o_s.

This is the algebra behind blockwise exact attention ("FlashAttention"
tiling, described in "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践"
§4.2 and in "Transformer架构优化实战2026" §三).  Empty sets have
lse_s = -inf and weight zero.
"""
import numpy as np


def lse_merge(outs, lses):
    """outs: [S, ..., D]; lses: [S, ...]  ->  (out [..., D], lse [...])."""
    outs = np.asarray(outs, np.float64)
    lses = np.asarray(lses, np.float64)
    top = np.max(lses, axis=0)
    safe = np.where(np.isfinite(top), top, 0.0)
    w = np.exp(lses - safe[None])                       # 0 for empty sets
    total = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.einsum("s...,s...d->...d", w, outs) / total[..., None]
        lse = safe + np.log(total)
    out = np.where(total[..., None] > 0, out, 0.0)
    lse = np.where(total > 0, lse, -np.inf)
    return out, lse
