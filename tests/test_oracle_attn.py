"""Pins of the oracle's decode attention (no GPU).

Definitions followed: softmax(q K^T / sqrt(d_k)) V with d_k the per-head
dimension and each weight row summing to 1 ("Transformer推理核心：KV Cache、
GQA与RoPE原理与工程实践" §2.1; "4. 自注意力机制推理" §4.1); GQA shares K/V head
h // n_rep across the n_rep query heads of a group, the repeat_interleave
broadcast (§2.2 of the first page; "Transformer架构优化实战2026" §六).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.full_causal import full_causal_attention
from oracle.merge import lse_merge

RNG = np.random.default_rng(99)


def _geom(B, H, G, D, S, dtype="f64"):
    return oracle.Geometry(B, H, G, D, dtype, max_seq_len=S)


def _rand_problem(B=2, H=8, G=2, D=16, S=40, lens=(40, 13)):
    q = RNG.standard_normal((B, H, D))
    k = RNG.standard_normal((B, S, G, D))
    v = RNG.standard_normal((B, S, G, D))
    return q, k, v, np.array(lens, np.int32)


def test_single_token_returns_its_value_exactly():
    q, k, v, _ = _rand_problem()
    L = np.array([1, 1], np.int32)
    out, lse = oracle.decode_attn(_geom(2, 8, 2, 16, 40), q, k, v, L)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(out[b, h], v[b, 0, h // 4])
            assert lse[b, h] == pytest.approx(q[b, h] @ k[b, 0, h // 4] / 4.0, rel=1e-14)


def test_equal_keys_give_mean_of_values():
    q, k, v, L = _rand_problem()
    k[:] = k[:, :1]
    out, lse = oracle.decode_attn(_geom(2, 8, 2, 16, 40), q, k, v, L)
    for b in range(2):
        n = L[b]
        for h in range(8):
            np.testing.assert_allclose(out[b, h], v[b, :n, h // 4].mean(axis=0), atol=1e-13)
            s = q[b, h] @ k[b, 0, h // 4] / 4.0
            assert lse[b, h] == pytest.approx(s + np.log(n), abs=1e-12)


def test_dominant_key_selects_its_value():
    q, k, v, L = _rand_problem(B=1, H=4, G=1, D=16, S=30, lens=(30,))
    k[0, 11, 0] = q[0, 0] * 40.0          # score ~ 40 * |q|^2 / 4 >> others
    out, _ = oracle.decode_attn(_geom(1, 4, 1, 16, 30), q, k, v, L)
    np.testing.assert_allclose(out[0, 0], v[0, 11, 0], atol=1e-12)


def test_weights_sum_to_one_and_output_is_convex_combination():
    q, k, v, L = _rand_problem()
    q *= 3.0
    out, lse, p = oracle.decode_attn(_geom(2, 8, 2, 16, 40), q, k, v, L, want_probs=True)
    for b in range(2):
        n = L[b]
        np.testing.assert_allclose(p[b, :, :n].sum(-1), 1.0, atol=1e-14)
        assert (p[b, :, n:] == 0).all()
        for h in range(8):
            vv = v[b, :n, h // 4]
            assert (out[b, h] <= vv.max(0) + 1e-12).all()
            assert (out[b, h] >= vv.min(0) - 1e-12).all()


def test_permuting_cached_tokens_leaves_output_unchanged():
    # the cache holds already-rotated K, so the order of rows is irrelevant to
    # one query's attention
    q, k, v, L = _rand_problem(lens=(40, 40))
    perm = RNG.permutation(40)
    g = _geom(2, 8, 2, 16, 40)
    out1, lse1 = oracle.decode_attn(g, q, k, v, L)
    out2, lse2 = oracle.decode_attn(g, q, np.ascontiguousarray(k[:, perm]),
                                    np.ascontiguousarray(v[:, perm]), L)
    np.testing.assert_allclose(out2, out1, atol=1e-13)
    np.testing.assert_allclose(lse2, lse1, atol=1e-13)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_equals_mha_on_repeat_interleaved_cache(G):
    H, D, S = 8, 16, 33
    q, k, v, L = _rand_problem(B=2, H=H, G=G, D=D, S=S, lens=(33, 20))
    out_g, lse_g = oracle.decode_attn(_geom(2, H, G, D, S), q, k, v, L)
    kr = np.ascontiguousarray(np.repeat(k, H // G, axis=2))
    vr = np.ascontiguousarray(np.repeat(v, H // G, axis=2))
    out_m, lse_m = oracle.decode_attn(_geom(2, H, H, D, S), q, kr, vr, L)
    assert np.array_equal(out_g, out_m) and np.array_equal(lse_g, lse_m)
    if 1 < G < H:
        # the other plausible mapping (head h -> K/V head h % G) is different
        kt = np.ascontiguousarray(np.tile(k, (1, 1, H // G, 1)))
        vt = np.ascontiguousarray(np.tile(v, (1, 1, H // G, 1)))
        out_t, _ = oracle.decode_attn(_geom(2, H, H, D, S), q, kt, vt, L)
        assert np.abs(out_t - out_g).max() > 1e-3


@pytest.mark.parametrize("G", [1, 4, 8])
def test_matches_torch_sdpa_fp64(G):
    """MHA (G = H), GQA and MQA (G = 1) against torch's fp64 CPU attention,
    with K/V expanded by repeat_interleave on the head axis."""
    H, D, S = 8, 32, 50
    q, k, v, L = _rand_problem(B=2, H=H, G=G, D=D, S=S, lens=(50, 7))
    q *= 2.0
    out, _ = oracle.decode_attn(_geom(2, H, G, D, S), q, k, v, L)
    for b in range(2):
        n = int(L[b])
        qt = torch.from_numpy(q[b][:, None, :])                              # [H, 1, D]
        kt = torch.from_numpy(k[b, :n]).permute(1, 0, 2).repeat_interleave(H // G, dim=0)
        vt = torch.from_numpy(v[b, :n]).permute(1, 0, 2).repeat_interleave(H // G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous())
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), atol=1e-13)


def test_zero_length_gives_zero_output_and_minus_inf_lse():
    q, k, v, _ = _rand_problem()
    out, lse = oracle.decode_attn(_geom(2, 8, 2, 16, 40), q, k, v, np.array([0, 3], np.int32))
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(lse[1]).all()


def test_sampled_units_equal_full_run():
    q, k, v, L = _rand_problem()
    g = _geom(2, 8, 2, 16, 40)
    out, lse = oracle.decode_attn(g, q, k, v, L)
    units = [(1, 7), (0, 0), (1, 2)]
    o2, l2 = oracle.decode_attn_units(g, q, k, v, L, units)
    for i, (b, h) in enumerate(units):
        assert np.array_equal(o2[i], out[b, h]) and l2[i] == lse[b, h]


def test_nan_in_unread_slots_does_not_leak():
    q, k, v, L = _rand_problem()
    k[0, L[0]:] = np.nan
    k[1, L[1]:] = np.nan
    v[1, L[1]:] = np.nan
    out, lse = oracle.decode_attn(_geom(2, 8, 2, 16, 40), q, k, v, L)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_lse_merge_of_token_partitions_equals_unsplit():
    """Attention over any partition of the tokens (empty parts included),
    merged by log-sum-exp, equals attention over all of them."""
    H, G, D, S = 4, 2, 16, 64
    q, k, v, _ = _rand_problem(B=1, H=H, G=G, D=D, S=S, lens=(64,))
    q *= 4.0
    g = _geom(1, H, G, D, S)
    full_o, full_l = oracle.decode_attn(g, q, k, v, np.array([S], np.int32))
    for cuts in ([0, 16, 16, 48, 64], [0, 1, 63, 64], [0, 64], [0, 5, 9, 30, 31, 64, 64]):
        outs, lses = [], []
        for a, bnd in zip(cuts[:-1], cuts[1:]):
            n = bnd - a
            kk = np.zeros((1, S, G, D)); vv = np.zeros((1, S, G, D))
            kk[0, :n], vv[0, :n] = k[0, a:bnd], v[0, a:bnd]
            o, l = oracle.decode_attn(g, q, kk, vv, np.array([n], np.int32))
            outs.append(o); lses.append(l)
        mo, ml = lse_merge(np.stack(outs), np.stack(lses))
        np.testing.assert_allclose(mo, full_o, atol=1e-13)
        np.testing.assert_allclose(ml, full_l, atol=1e-13)


@pytest.mark.parametrize("D", [8, 64])
@pytest.mark.parametrize("G", [1, 2, 8])
@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_decode_loop_equals_full_causal_recompute(D, G, style):
    """Cached decode, one token per step (RoPE at the step's position, append
    at that slot, attend over the prefix), equals causal attention recomputed
    from scratch over the whole sequence by an independent NumPy program."""
    T, H = 24 if D == 64 else 48, 8
    q = RNG.standard_normal((T, H, D))
    k = RNG.standard_normal((T, G, D))
    v = RNG.standard_normal((T, G, D))
    ref, w = full_causal_attention(q, k, v, style=style)
    # the recompute's weights are lower-triangular (no future token visible)
    assert np.all(np.triu(w, k=1) == 0.0)
    g = _geom(1, H, G, D, T)
    kc = np.full((1, T, G, D), np.nan)
    vc = np.full((1, T, G, D), np.nan)
    for t in range(T):
        q_rot = oracle.rope_append(g, np.ascontiguousarray(q[t][None]),
                                   np.ascontiguousarray(k[t][None]),
                                   np.ascontiguousarray(v[t][None]), kc, vc,
                                   np.array([t], np.int32), style=style)
        out, _ = oracle.decode_attn(g, q_rot, kc, vc, np.array([t + 1], np.int32))
        np.testing.assert_allclose(out[0], ref[t], atol=1e-12)


def test_mask_fill_value_form_matches_exclusion():
    # filling masked scores with -1e9 (the pages' code) gives the same result
    # as excluding them, for finite scores
    q = RNG.standard_normal((10, 4, 8))
    k = RNG.standard_normal((10, 2, 8))
    v = RNG.standard_normal((10, 2, 8))
    a, _ = full_causal_attention(q, k, v)
    b, _ = full_causal_attention(q, k, v, mask_value=-1e9)
    np.testing.assert_array_equal(a, b)
