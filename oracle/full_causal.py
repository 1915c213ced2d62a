"""Causal self-attention recomputed from scratch, fp64 NumPy (tiny inputs).

TEST INFRASTRUCTURE ONLY.  Written independently of ``kvoracle.c``: here
RoPE is a complex multiplication of the (real, imag) pairs, the GQA
broadcast is an explicit ``np.repeat`` on the head axis, and the causal mask
is applied to the whole T x T score matrix.  Agreement of the C decode loop
(one query per step over the cache) with this full recompute pins both.

Pages cited by title:
  [KVGR] "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践"
  [OPT]  "Transformer架构优化实战2026：注意力机制、KV Cache与推理加速完整指南"
"""
import numpy as np


def rope_complex(x, positions, base=10000.0, style="interleaved"):
    """Rotate x [T, heads, D] at positions [T] by e^{i * pos * theta_k}.

    The pair k is the complex number x[2k] + i x[2k+1] (interleaved) or
    x[k] + i x[k + D/2] (half); theta_k = 1 / base^(2k / D) ([KVGR] §3,
    the arange(0, dim, 2) / dim form of the frequency).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    freqs = 1.0 / (base ** (np.arange(0, D, 2, dtype=np.float64) / D))
    angles = np.asarray(positions, dtype=np.float64)[:, None] * freqs[None, :]  # [T, D/2]
    rot = np.exp(1j * angles)[:, None, :]                                        # [T, 1, D/2]
    if style == "interleaved":
        z = x[..., 0::2] + 1j * x[..., 1::2]
    else:
        z = x[..., : D // 2] + 1j * x[..., D // 2:]
    z = z * rot
    y = np.empty_like(x)
    if style == "interleaved":
        y[..., 0::2], y[..., 1::2] = z.real, z.imag
    else:
        y[..., : D // 2], y[..., D // 2:] = z.real, z.imag
    return y


def full_causal_attention(q, k, v, base=10000.0, style="interleaved", scale=None,
                          mask_value=None):
    """Outputs of every position of one sequence, recomputed from scratch.

    q: [T, H, D]; k, v: [T, G, D] (un-rotated, fp64).  Token t sits at
    position t.  Returns (out [T, H, D], weights [H, T, T]).

    mask_value=None excludes future tokens (weight exactly 0); a finite value
    (the pages use -1e9, [OPT] §二) fills the masked scores instead.
    """
    T, H, D = q.shape
    G = k.shape[1]
    n_rep = H // G
    pos = np.arange(T)
    qr = rope_complex(q, pos, base, style)
    kr = rope_complex(k, pos, base, style)
    # GQA: K/V of group g serve query heads g*n_rep ... g*n_rep + n_rep - 1
    # (repeat_interleave on the head axis, [KVGR] §2.2, [OPT] §六)
    kr = np.repeat(kr, n_rep, axis=1)
    vv = np.repeat(np.asarray(v, np.float64), n_rep, axis=1)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    scores = np.einsum("thd,shd->hts", qr, kr) * scale        # [H, T, T]
    causal = np.tril(np.ones((T, T), dtype=bool))             # j <= i visible
    if mask_value is None:
        scores = np.where(causal[None], scores, -np.inf)
    else:
        scores = np.where(causal[None], scores, mask_value)
    scores = scores - scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=-1, keepdims=True)
    out = np.einsum("hts,shd->thd", w, vv)
    return out, w
