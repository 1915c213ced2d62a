"""Pins of the oracle's paged caches beyond one private 16-token block per
slot (no GPU): 32-token blocks, and block tables that share a prompt prefix.

"Transformer架构优化实战2026" §九 recommends 32-token blocks for long
sequences and 16 for short ones, and prefix caching where requests share a
system prompt (§八 enables it in the vLLM configuration); §四 describes the
block table.  Here the shared prefix blocks are read only: every sequence
appends into a block of its own.  The pin: attention through any table
equals attention over the contiguous cache that an independent numpy gather
of the same blocks builds (the already pinned contiguous path).
"""
import numpy as np
import pytest

import oracle
from kv_cache_gqa_decode_amd import workloads as W


def _geom(s):
    return oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                           max_seq_len=s.max_seq_len, block_size=s.block_size,
                           num_blocks=s.num_blocks, max_blocks_per_seq=s.max_blocks_per_seq)


def _paged(dtype, block_size, B=4, nb=None):
    per = 512 // block_size                      # blocks per sequence (512 tokens)
    s = W.spec("c4", batch=B, n_heads=8, n_kv_heads=2, head_dim=64, len_lo=1, len_hi=512,
               num_blocks=nb or B * per + 8, max_blocks_per_seq=per, block_size=block_size,
               q_gain=6.0, value_scale=0.125)
    return s.replace(dtype=dtype)


def _token_major(s, cache, v=False):
    """[num_blocks * block_size, G, D] view of a pool (INT8 pools regrouped)."""
    G, D, bs = s.n_kv_heads, s.head_dim, s.block_size
    if s.dtype != "i8":
        return cache.reshape(-1, G, D)
    m = bs // 16
    c = cache.reshape(s.num_blocks * m, G, D, 16) if v else cache.reshape(s.num_blocks * m, G, 16, D)
    c = c.transpose(0, 3, 1, 2) if v else c.transpose(0, 2, 1, 3)
    return np.ascontiguousarray(c).reshape(-1, G, D)


def _gathered(s, p, table):
    """Contiguous fp64 caches [B, S, G, D] gathered through the table."""
    bs = s.block_size
    kt, vt = _token_major(s, p.k_cache), _token_major(s, p.v_cache, v=True)
    B, S = s.batch, s.max_seq_len
    k = np.zeros((B, S, s.n_kv_heads, s.head_dim))
    v = np.zeros_like(k)
    for b in range(B):
        for j in range(S // bs):
            blk = table[b, j]
            k[b, j * bs:(j + 1) * bs] = _values(s, p, kt[blk * bs:(blk + 1) * bs], "k")
            v[b, j * bs:(j + 1) * bs] = _values(s, p, vt[blk * bs:(blk + 1) * bs], "v")
    return k, v


def _values(s, p, a, which):
    if s.dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if s.dtype == "i8":
        sc = (p.k_scale if which == "k" else p.v_scale).astype(np.float64)
        return a.astype(np.float64) * sc[None, :, None]
    return a.astype(np.float64)


def _scales(s, p):
    return dict(k_scale=p.k_scale, v_scale=p.v_scale) if s.dtype == "i8" else {}


def _share_prefix(s, p, n_shared):
    """Rows 1.. of the table start with row 0's first n_shared blocks; every
    sequence's append slot stays in a block of its own."""
    t = p.block_table.copy()
    t[1:, :n_shared] = t[0, :n_shared]
    assert (p.positions // s.block_size >= n_shared).all()
    return t


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("shared", [0, 3])
def test_paged_attention_equals_gathered_contiguous(dtype, block_size, shared):
    s = _paged(dtype, block_size)
    L = np.array([200, 511, 130, 300], np.int32)
    p = W.make_problem(s, lengths=L)
    table = _share_prefix(s, p, shared) if shared else p.block_table
    g = _geom(s)
    q_rot = oracle.rope_append(g, p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions, table,
                               **_scales(s, p))
    out, lse = oracle.decode_attn(g, q_rot, p.k_cache, p.v_cache, p.seq_lens, table,
                                  **_scales(s, p))
    k, v = _gathered(s, p, table)
    gc = oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, "f64",
                         max_seq_len=s.max_seq_len)
    ref, ref_lse = oracle.decode_attn(gc, q_rot, k, v, p.seq_lens)
    assert np.abs(out - ref).max() <= 1e-13 * np.abs(ref).max()
    assert np.abs(lse - ref_lse).max() <= 1e-12
    if shared:
        # the shared prefix is really read by every sequence: zeroing one of
        # its values changes every sequence's output
        kz = p.k_cache.copy()
        kz[p.block_table[0, 0]] = 0
        out2, _ = oracle.decode_attn(g, q_rot, kz, p.v_cache, p.seq_lens, table, **_scales(s, p))
        assert all(np.abs(out2[b] - out[b]).max() > 0 for b in range(s.batch))


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_block_32_equals_block_16(dtype):
    """The same logical cache in 32-token and in 16-token blocks gives the
    same attention (each block size with its own seeded table)."""
    L = np.array([200, 511, 130, 300], np.int32)
    res = []
    for bs in (16, 32):
        s = _paged(dtype, bs).replace(cfg_id=7)
        p = W.make_problem(s, lengths=L)
        g = _geom(s)
        q_rot = oracle.rope_append(g, p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions,
                                   p.block_table, **_scales(s, p))
        res.append(oracle.decode_attn(g, q_rot, p.k_cache, p.v_cache, p.seq_lens, p.block_table,
                                      **_scales(s, p)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
