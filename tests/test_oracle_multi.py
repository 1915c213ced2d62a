"""Pins of the oracle's multi-token step (no GPU): T = gamma + 1 new tokens
per sequence, all appended, each attending the cache and the new tokens up
to its own position.

"Transformer架构优化实战2026" §五: in speculative decoding the target model
checks all gamma draft tokens in one forward pass (gamma = 4 in the page's
code).  With a KV cache that pass is one step with several queries per
sequence under the causal mask of [KVGR] §5.1 b.v.  Pins: the step equals T
single-token steps taken one after the other (the pinned decode step), and
equals the last T rows of causal attention recomputed from scratch by the
independent NumPy program.
"""
import numpy as np
import pytest

import oracle
from oracle.full_causal import full_causal_attention
from kv_cache_gqa_decode_amd import workloads as W

RNG = np.random.default_rng(41)


@pytest.mark.parametrize("T", [1, 2, 5])
@pytest.mark.parametrize("G", [1, 2, 8])
@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_window_step_equals_full_causal_tail(T, G, style):
    N, H, D = 29, 8, 16
    q = RNG.standard_normal((N, H, D))
    k = RNG.standard_normal((N, G, D))
    v = RNG.standard_normal((N, G, D))
    ref, _ = full_causal_attention(q, k, v, style=style)
    g = oracle.Geometry(1, H, G, D, "f64", max_seq_len=N)
    kc = np.full((1, N, G, D), np.nan)
    vc = np.full((1, N, G, D), np.nan)
    P = N - T
    # history: one token per step (the pinned single-token path)
    for t in range(P):
        oracle.rope_append(g, None, np.ascontiguousarray(k[t][None]),
                           np.ascontiguousarray(v[t][None]), kc, vc, np.array([t], np.int32),
                           style=style)
    q_rot = oracle.rope_append(g, np.ascontiguousarray(q[P:][None]), np.ascontiguousarray(k[P:][None]),
                               np.ascontiguousarray(v[P:][None]), kc, vc, np.array([P], np.int32),
                               style=style, n_query=T) if T > 1 else \
        oracle.rope_append(g, np.ascontiguousarray(q[P][None]), np.ascontiguousarray(k[P][None]),
                           np.ascontiguousarray(v[P][None]), kc, vc, np.array([P], np.int32),
                           style=style)
    out, lse = oracle.decode_attn(g, q_rot, kc, vc, np.array([N], np.int32), n_query=T)
    got = out[0] if T > 1 else out
    np.testing.assert_allclose(got.reshape(T, H, D), ref[P:], atol=1e-12)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("paged", [False, True])
def test_window_step_equals_sequential_steps(dtype, paged):
    """One step with T = 5 new tokens per sequence = five single-token steps,
    bit for bit in the caches and to rounding in the outputs."""
    T, B, H, G, D = 5, 3, 8, 2, 64
    if paged:
        s = W.spec("c4", batch=B, n_heads=H, n_kv_heads=G, head_dim=D, num_blocks=40,
                   max_blocks_per_seq=8, q_gain=6.0, value_scale=0.125)
    else:
        s = W.spec("c3", batch=B, n_heads=H, n_kv_heads=G, head_dim=D, max_seq_len=128,
                   q_gain=6.0, value_scale=0.125)
    s = s.replace(dtype=dtype)
    L = np.array([T, 40, 128], np.int32)         # tokens after the step
    p = W.make_problem(s, lengths=L - T + 1)      # history of L - T tokens
    g = oracle.Geometry(B, H, G, D, dtype, max_seq_len=s.max_seq_len, block_size=s.block_size,
                        num_blocks=s.num_blocks, max_blocks_per_seq=s.max_blocks_per_seq)
    sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if dtype == "i8" else {}
    qw = RNG.standard_normal((B, T, H, D)).astype(np.float32) * 0.8
    kw = RNG.standard_normal((B, T, G, D)).astype(np.float32) * 0.2
    vw = RNG.standard_normal((B, T, G, D)).astype(np.float32) * 0.2
    cast = lambda a: W._to_storage(a, "bf16")
    qw, kw, vw = cast(qw), cast(kw), cast(vw)
    P = (L - T).astype(np.int32)
    # one window step
    k1, v1 = p.k_cache.copy(), p.v_cache.copy()
    q_rot = oracle.rope_append(g, qw, kw, vw, k1, v1, P, p.block_table, n_query=T, **sc)
    out, lse = oracle.decode_attn(g, q_rot, k1, v1, L, p.block_table, n_query=T, **sc)
    # T single-token steps
    k2, v2 = p.k_cache.copy(), p.v_cache.copy()
    for t in range(T):
        qr = oracle.rope_append(g, np.ascontiguousarray(qw[:, t]), np.ascontiguousarray(kw[:, t]),
                                np.ascontiguousarray(vw[:, t]), k2, v2, (P + t).astype(np.int32),
                                p.block_table, **sc)
        o, l = oracle.decode_attn(g, qr, k2, v2, (P + t + 1).astype(np.int32), p.block_table,
                                  **sc)
        np.testing.assert_allclose(q_rot[:, t], qr, rtol=0, atol=0)
        np.testing.assert_allclose(out[:, t], o, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[:, t], l, rtol=0, atol=1e-13)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_window_mask_is_needed():
    """Dropping the in-window mask (every query sees all T new tokens) is
    caught: query 0 must not see tokens 1 .. T-1."""
    N, H, G, D, T = 20, 4, 2, 16, 5
    q = RNG.standard_normal((N, H, D))
    k = RNG.standard_normal((N, G, D))
    v = RNG.standard_normal((N, G, D))
    ref, _ = full_causal_attention(q, k, v)
    g = oracle.Geometry(1, H, G, D, "f64", max_seq_len=N)
    kc = np.zeros((1, N, G, D)); vc = np.zeros((1, N, G, D))
    for t in range(N - T):
        oracle.rope_append(g, None, np.ascontiguousarray(k[t][None]),
                           np.ascontiguousarray(v[t][None]), kc, vc, np.array([t], np.int32))
    q_rot = oracle.rope_append(g, np.ascontiguousarray(q[N - T:][None]),
                               np.ascontiguousarray(k[N - T:][None]),
                               np.ascontiguousarray(v[N - T:][None]), kc, vc,
                               np.array([N - T], np.int32), n_query=T)
    # all queries over the full length: what an unmasked window would give
    flat = oracle.Geometry(T, H, G, D, "f64", max_seq_len=N)
    kk = np.repeat(kc, T, axis=0); vv = np.repeat(vc, T, axis=0)
    unmasked, _ = oracle.decode_attn(flat, np.ascontiguousarray(q_rot[0]), kk, vv,
                                     np.full(T, N, np.int32))
    assert np.abs(unmasked[0] - ref[N - T]).max() > 1e-3
    masked, _ = oracle.decode_attn(g, q_rot, kc, vc, np.array([N], np.int32), n_query=T)
    np.testing.assert_allclose(masked[0], ref[N - T:], atol=1e-12)
