"""Pins of the oracle's KV-cache append (no GPU).

"4. 自注意力机制推理：单步计算、KV Cache的引入与原理" §4.5: the cache is
preallocated and the new K/V are written at index `step`, nothing else
moves.  "Transformer架构优化实战2026" §四: the same update at start_pos for a
[batch, seq, heads, dim] cache, and the paged variant whose blocks are
gathered through a per-sequence block table.
"""
import numpy as np
import pytest

import oracle
from kv_cache_gqa_decode_amd import workloads as W


def _geom(s):
    return oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                           max_seq_len=s.max_seq_len, block_size=s.block_size,
                           num_blocks=s.num_blocks, max_blocks_per_seq=s.max_blocks_per_seq)


def _small(dtype="bf16", paged=False, G=2, poison=True, block_size=16):
    if paged:
        nb = 640 // block_size
        return W.spec("c4", batch=3, n_heads=4, n_kv_heads=G, head_dim=64, len_lo=1,
                      len_hi=70, num_blocks=nb, max_blocks_per_seq=128 // block_size,
                      block_size=block_size, poison=poison)
    s = W.spec("c3", batch=3, n_heads=4, n_kv_heads=G, head_dim=64, len_lo=1, len_hi=70,
               max_seq_len=80, poison=poison)
    return s.replace(dtype=dtype)


def _slot(s, p, b):
    pos = int(p.positions[b])
    if s.block_size:
        return p.block_table[b, pos // s.block_size], pos % s.block_size
    return b, pos


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("paged", [False, True])
def test_only_appended_slots_change(dtype, paged):
    s = _small(dtype, paged)
    s = s.replace(dtype=dtype)
    p = W.make_problem(s, lengths=np.array([1, 17, 70], np.int32))
    k0, v0 = p.k_cache.copy(), p.v_cache.copy()
    oracle.rope_append(_geom(s), p.q, p.k_new, p.v_new, p.k_cache, p.v_cache,
                       p.positions, p.block_table)
    changed = np.zeros(p.k_cache.shape[:2], bool)
    for b in range(s.batch):
        changed[_slot(s, p, b)] = True
    raw = lambda a: a.view(np.uint32 if a.dtype == np.float32 else np.uint16)
    # brute-force diff: outside the B appended rows the caches are bit-identical
    assert np.array_equal(raw(p.k_cache)[~changed], raw(k0)[~changed])
    assert np.array_equal(raw(p.v_cache)[~changed], raw(v0)[~changed])
    for b in range(s.batch):
        sl = _slot(s, p, b)
        # V is a bit copy of v_new; K holds finite rotated values (the slot was NaN)
        assert np.array_equal(raw(p.v_cache[sl]), raw(p.v_new[b]))
        kf = p.k_cache[sl].astype(np.float64) if dtype == "f32" else \
            (p.k_cache[sl].astype(np.uint32) << 16).view(np.float32)
        assert np.isfinite(kf).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_position_zero_stores_k_unchanged(dtype):
    s = _small(dtype)
    p = W.make_problem(s, lengths=np.array([1, 1, 1], np.int32))
    oracle.rope_append(_geom(s), p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions)
    assert np.array_equal(p.k_cache[:, 0], p.k_new)


def _to64(a, dtype):
    if dtype == "f32":
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stored_k_is_rotation_rounded_once(dtype):
    """The stored K row is the fp64 rotation of k_new rounded once."""
    s = _small(dtype)
    p = W.make_problem(s, lengths=np.array([5, 33, 64], np.int32))
    oracle.rope_append(_geom(s), p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions)
    for b in range(s.batch):
        pos = int(p.positions[b])
        exact = oracle.rope_rotate(_to64(p.k_new[b], dtype), pos)
        stored = _to64(p.k_cache[b, pos], dtype)
        # nearest representable: error at most half a unit in the last place
        if dtype == "f32":
            ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
        else:
            ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
        assert (np.abs(stored - exact) <= 0.5 * ulp).all()


@pytest.mark.parametrize("block_size", [16, 32])
def test_paged_gather_equals_contiguous(block_size):
    """Gathering the paged pool through the table (the concatenation of a
    sequence's blocks) reproduces the contiguous cache, before and after the
    append, for 16- and 32-token blocks."""
    G = 2
    sp = _small("bf16", paged=True, G=G, block_size=block_size)
    sc = _small("bf16", paged=False, G=G).replace(cfg_id=sp.cfg_id, max_seq_len=128)
    L = np.array([3, 16, 70], np.int32)
    pp = W.make_problem(sp, lengths=L)
    pc = W.make_problem(sc, lengths=L)
    for arrs in ((pp.k_cache, pc.k_cache), (pp.v_cache, pc.v_cache)):
        pool, cont = arrs
        for b in range(3):
            n = int(L[b]) - 1
            gathered = np.concatenate([pool[i] for i in pp.block_table[b]])[:n]
            assert np.array_equal(gathered, cont[b, :n])
    oracle.rope_append(_geom(sp), pp.q, pp.k_new, pp.v_new, pp.k_cache, pp.v_cache,
                       pp.positions, pp.block_table)
    oracle.rope_append(_geom(sc), pc.q, pc.k_new, pc.v_new, pc.k_cache, pc.v_cache,
                       pc.positions)
    for b in range(3):
        n = int(L[b])
        gathered = np.concatenate([pp.k_cache[i] for i in pp.block_table[b]])[:n]
        assert np.array_equal(gathered, pc.k_cache[b, :n])
        gathered = np.concatenate([pp.v_cache[i] for i in pp.block_table[b]])[:n]
        assert np.array_equal(gathered, pc.v_cache[b, :n])


def test_step_counter_advances_one_slot_per_step():
    """Appending at position t, t+1, ... fills consecutive slots; inspecting
    K_cache[0, :, 0, 0] after each step shows exactly one new entry at the end
    (the check "Transformer推理核心" §5.3 recommends)."""
    s = _small("f32").replace(batch=1, poison=False)
    p = W.make_problem(s, lengths=np.array([1], np.int32))
    g = _geom(s)
    rng = np.random.default_rng(3)
    for t in range(6):
        k_new = rng.standard_normal((1, s.n_kv_heads, s.head_dim)).astype(np.float32)
        v_new = rng.standard_normal((1, s.n_kv_heads, s.head_dim)).astype(np.float32)
        before = p.k_cache[0, :, 0, 0].copy()
        oracle.rope_append(g, None, k_new, v_new, p.k_cache, p.v_cache,
                           np.array([t], np.int32))
        after = p.k_cache[0, :, 0, 0]
        diff = np.flatnonzero(before != after)
        assert list(diff) == [t]
        assert np.array_equal(p.v_cache[0, t], v_new[0])


def test_out_of_range_position_is_rejected_and_skipped():
    s = _small("bf16")
    p = W.make_problem(s, lengths=np.array([2, 3, 4], np.int32))
    pos = p.positions.copy()
    pos[1] = s.max_seq_len          # one past the end
    k0 = p.k_cache.copy()
    with pytest.raises(ValueError):
        oracle.rope_append(_geom(s), p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, pos)
    assert np.array_equal(p.k_cache[1], k0[1])
