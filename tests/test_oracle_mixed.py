"""Pins of the oracle's mixed-precision cache (no GPU).

"Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §4.3 names caches that keep
the most recent tokens at high precision and quantise the older history.
Reading adopted: the W newest tokens of a sequence in a bf16 ring (token p
in row p mod W), every older token as INT8 codes (per-head scales, the INT8
cache's layout) at its own position; the token that leaves the ring is
quantised from its stored bf16 values.  The pins tie the oracle to things
outside itself:

* appending token by token leaves the ring equal, bit for bit, to the last W
  rows of a bf16 cache filled by the (separately pinned) bf16 append, and
  the INT8 history equal to an exhaustive nearest-code search over those
  rows' values;
* attention equals a numpy softmax over the history's dequantised codes and
  the ring's values, gathered by position;
* with a ring as long as the cache nothing is quantised and the step equals
  the bf16 step exactly;
* a paged INT8 history holds the same codes as a contiguous one.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_i8 import _nearest_codes


def _bf16_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16           # nearest even
    return u.astype(np.uint16)


def _bf16_val(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _geoms(B, H, G, D, S, block_size=0):
    gi = oracle.Geometry(B, H, G, D, "i8", max_seq_len=S)
    if block_size:
        nbps = S // block_size
        gi = oracle.Geometry(B, H, G, D, "i8", block_size=block_size, num_blocks=B * nbps + 3,
                             max_blocks_per_seq=nbps)
    gb = oracle.Geometry(B, H, G, D, "bf16", max_seq_len=S)
    return gi, gb


def _scales(rng, G):
    return ((rng.uniform(0.75, 1.25, G) / 40).astype(np.float32),
            (rng.uniform(0.75, 1.25, G) / 40).astype(np.float32))


def _codes_at(gi, kc, vc, b, p, table=None):
    """K and V codes [G, D] of token p of sequence b (independent regrouping)."""
    if gi.block_size:
        blk = table[b, p // gi.block_size]
        grp = blk * (gi.block_size // 16) + (p % gi.block_size) // 16
        kflat = kc.reshape(-1, gi.n_kv_heads, 16, gi.head_dim)
        vflat = vc.reshape(-1, gi.n_kv_heads, gi.head_dim, 16)
        return kflat[grp, :, p % 16, :], vflat[grp, :, :, p % 16]
    return kc[b, p // 16, :, p % 16, :], vc[b, p // 16, :, :, p % 16]


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_token_by_token_ring_and_history(style):
    B, H, G, D, S, Wn, N = 2, 4, 2, 8, 64, 16, 41
    rng = np.random.default_rng(101)
    gi, gb = _geoms(B, H, G, D, S)
    ks, vs = _scales(rng, G)
    kc = np.zeros(gi.cache_shape(), np.int8)
    vc = np.zeros(gi.v_cache_shape(), np.int8)
    kr = np.zeros(oracle.recent_shape(gi, Wn), np.uint16)
    vr = np.zeros_like(kr)
    kb = np.zeros(gb.cache_shape(), np.uint16)
    vb = np.zeros_like(kb)
    start = np.array([0, 5], np.int32)                # sequence 1 starts at position 5
    for step in range(N):
        pos = (start + step).astype(np.int32)
        q = _bf16_bits(rng, (B, H, D), 0.3)
        k = _bf16_bits(rng, (B, G, D), 0.3)
        v = _bf16_bits(rng, (B, G, D), 0.3)
        qm = oracle.rope_append_mixed(gi, Wn, q, k, v, kc, vc, kr, vr, pos, style=style,
                                      k_scale=ks, v_scale=vs)
        qb = oracle.rope_append(gb, q, k, v, kb, vb, pos, style=style)
        assert np.array_equal(qm, qb)
    for b in range(B):
        end = int(start[b]) + N                          # tokens start[b] .. end - 1 written
        for p in range(int(start[b]), end):
            if p >= end - Wn:                           # still in the ring, as written
                assert np.array_equal(kr[b, p % Wn], kb[b, p]), (b, p)
                assert np.array_equal(vr[b, p % Wn], vb[b, p]), (b, p)
            else:                                       # left the ring: nearest codes
                kq, vq = _codes_at(gi, kc, vc, b, p)
                for g in range(G):
                    assert np.array_equal(kq[g], _nearest_codes(_bf16_val(kb[b, p, g]), ks[g]))
                    assert np.array_equal(vq[g], _nearest_codes(_bf16_val(vb[b, p, g]), vs[g]))
        for p in list(range(0, int(start[b]))) + list(range(end - Wn, S)):
            kq, vq = _codes_at(gi, kc, vc, b, p)        # never quantised: untouched
            assert not kq.any() and not vq.any(), (b, p)


def _numpy_mixed_attention(gi, Wn, q_rot, kc, vc, kr, vr, lens, ks, vs, table=None):
    B, H, G, D = gi.batch, gi.n_heads, gi.n_kv_heads, gi.head_dim
    out = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        K = np.zeros((L, G, D))
        V = np.zeros((L, G, D))
        for j in range(L):
            if j >= L - Wn:
                K[j], V[j] = _bf16_val(kr[b, j % Wn]), _bf16_val(vr[b, j % Wn])
            else:
                kq, vq = _codes_at(gi, kc, vc, b, j, table)
                K[j] = ks[:, None] * kq.astype(np.float64)
                V[j] = vs[:, None] * vq.astype(np.float64)
        for h in range(H):
            g = h // (H // G)
            s = K[:, g, :] @ q_rot[b, h] / np.sqrt(D)
            m = s.max()
            e = np.exp(s - m)
            out[b, h] = (e / e.sum()) @ V[:, g, :]
            lse[b, h] = m + np.log(e.sum())
    return out, lse


@pytest.mark.parametrize("block_size", [0, 16, 32])
def test_attention_is_softmax_over_history_and_ring(block_size):
    B, H, G, D, S, Wn = 5, 8, 2, 16, 128, 32
    rng = np.random.default_rng(102)
    gi, _ = _geoms(B, H, G, D, S, block_size)
    ks, vs = _scales(rng, G)
    kc = rng.integers(-127, 128, gi.cache_shape()).astype(np.int8)
    vc = rng.integers(-127, 128, gi.v_cache_shape()).astype(np.int8)
    kr = _bf16_bits(rng, oracle.recent_shape(gi, Wn), 0.09)
    vr = _bf16_bits(rng, oracle.recent_shape(gi, Wn), 0.09)
    table = None
    if block_size:
        table = rng.permutation(gi.num_blocks)[:B * gi.max_blocks_per_seq]
        table = table.reshape(B, -1).astype(np.int32)
    lens = np.array([0, 1, Wn - 1, Wn, 117], np.int32)   # none, all in the ring, history too
    q_rot = rng.standard_normal((B, H, D))
    o, l = oracle.decode_attn_mixed(gi, Wn, q_rot, kc, vc, kr, vr, lens, table, k_scale=ks,
                                    v_scale=vs)
    eo, el = _numpy_mixed_attention(gi, Wn, q_rot, kc, vc, kr, vr, lens, ks, vs, table)
    np.testing.assert_allclose(o, eo, rtol=0, atol=1e-13)
    assert np.isneginf(l[0]).all()
    np.testing.assert_allclose(l[1:], el[1:], rtol=1e-13, atol=0)
    # listed units agree with the whole batch
    units = [(4, 7), (2, 0), (4, 1)]
    uo, ul = oracle.decode_attn_mixed(gi, Wn, q_rot, kc, vc, kr, vr, lens, table, k_scale=ks,
                                      v_scale=vs, units=units)
    for i, (b, h) in enumerate(units):
        assert np.array_equal(uo[i], o[b, h]) and ul[i] == l[b, h]


def test_ring_as_long_as_the_cache_is_the_bf16_step():
    """W = S_max: token p stays in ring row p, nothing is quantised, and the
    step (append and attention) equals the bf16 step exactly."""
    B, H, G, D, S = 3, 8, 4, 16, 48
    rng = np.random.default_rng(103)
    gi, gb = _geoms(B, H, G, D, S)
    ks, vs = _scales(rng, G)
    kc = np.zeros(gi.cache_shape(), np.int8)
    vc = np.zeros(gi.v_cache_shape(), np.int8)
    kb = _bf16_bits(rng, gb.cache_shape(), 0.09)
    vb = _bf16_bits(rng, gb.cache_shape(), 0.09)
    kr, vr = kb.copy(), vb.copy()
    pos = np.array([0, 20, S - 1], np.int32)
    q = _bf16_bits(rng, (B, H, D))
    k = _bf16_bits(rng, (B, G, D))
    v = _bf16_bits(rng, (B, G, D))
    qm = oracle.rope_append_mixed(gi, S, q, k, v, kc, vc, kr, vr, pos, k_scale=ks, v_scale=vs)
    qb = oracle.rope_append(gb, q, k, v, kb, vb, pos)
    assert np.array_equal(qm, qb) and np.array_equal(kr, kb) and np.array_equal(vr, vb)
    assert not kc.any() and not vc.any()
    lens = pos + 1
    om, lm = oracle.decode_attn_mixed(gi, S, qm, kc, vc, kr, vr, lens, k_scale=ks, v_scale=vs)
    ob, lb = oracle.decode_attn(gb, qb, kb, vb, lens)
    assert np.array_equal(om, ob) and np.array_equal(lm, lb)


def test_paged_history_holds_the_contiguous_codes():
    B, H, G, D, S, Wn, N = 2, 4, 2, 8, 64, 16, 50
    rng = np.random.default_rng(104)
    gc, _ = _geoms(B, H, G, D, S)
    gp, _ = _geoms(B, H, G, D, S, block_size=32)
    ks, vs = _scales(rng, G)
    table = rng.permutation(gp.num_blocks)[:B * gp.max_blocks_per_seq].reshape(B, -1)
    table = table.astype(np.int32)
    state = {}
    for name, g in (("c", gc), ("p", gp)):
        state[name] = [np.zeros(g.cache_shape(), np.int8), np.zeros(g.v_cache_shape(), np.int8),
                       np.zeros(oracle.recent_shape(g, Wn), np.uint16),
                       np.zeros(oracle.recent_shape(g, Wn), np.uint16)]
    for step in range(N):
        pos = np.full(B, step, np.int32)
        q = _bf16_bits(rng, (B, H, D))
        k = _bf16_bits(rng, (B, G, D))
        v = _bf16_bits(rng, (B, G, D))
        oracle.rope_append_mixed(gc, Wn, q, k, v, *state["c"], pos, k_scale=ks, v_scale=vs)
        oracle.rope_append_mixed(gp, Wn, q, k, v, *state["p"], pos, table, k_scale=ks,
                                 v_scale=vs)
    kc, vc, krc, vrc = state["c"]
    kp, vp, krp, vrp = state["p"]
    assert np.array_equal(krc, krp) and np.array_equal(vrc, vrp)
    for b in range(B):
        for p in range(N - Wn):
            a = _codes_at(gc, kc, vc, b, p)
            c = _codes_at(gp, kp, vp, b, p, table)
            assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_out_of_range_position_is_refused():
    B, H, G, D, S, Wn = 1, 2, 1, 8, 32, 16
    gi, _ = _geoms(B, H, G, D, S)
    ks = vs = np.ones(G, np.float32)
    bufs = [np.zeros(gi.cache_shape(), np.int8), np.zeros(gi.v_cache_shape(), np.int8),
            np.zeros(oracle.recent_shape(gi, Wn), np.uint16),
            np.zeros(oracle.recent_shape(gi, Wn), np.uint16)]
    z = np.zeros((B, G, D), np.uint16)
    with pytest.raises(ValueError):
        oracle.rope_append_mixed(gi, Wn, None, z, z, *bufs, np.array([S], np.int32),
                                 k_scale=ks, v_scale=vs)
    assert not any(b.any() for b in bufs)
