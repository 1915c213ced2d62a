"""Pins of the oracle's INT8 KV cache (no GPU).

"Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §4.3: the cached K and V
vectors are held as 8-bit integers instead of bf16, with quantisation
parameters calibrated per attention head.  Reading adopted: symmetric codes
n in [-127, 127] with one fp32 scale per KV head for K and one for V; a new
element x is stored as the code nearest to x / scale; attention reads
scale * n.  The pins below check the oracle against that definition written
differently: the nearest code found by exhaustive search (exact rational
arithmetic at the ties), the cache layout through an independent numpy
regrouping, and attention against the already pinned fp64 path on the
dequantised cache.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from kv_cache_gqa_decode_amd import workloads as W

CODES = np.arange(-127, 128)


def _nearest_code_exact(x: float, s: float) -> int:
    """argmin over n in [-127, 127] of |x - n s| in exact arithmetic, ties to
    the even n (infinite x saturates, NaN gives 0)."""
    if np.isnan(x):
        return 0
    if np.isinf(x):
        return 127 if (x > 0) == (s > 0) else -127
    fx, fs = Fraction(x), Fraction(s)
    best, best_d = None, None
    for n in range(-127, 128):
        d = abs(fx - n * fs)
        if best is None or d < best_d or (d == best_d and n % 2 == 0):
            best, best_d = n, d
    return best


def _nearest_codes(x: np.ndarray, s: float) -> np.ndarray:
    """Vectorised exhaustive search for generic (tie-free) inputs."""
    d = np.abs(np.asarray(x, np.float64)[..., None] - CODES * np.float64(s))
    return CODES[np.argmin(d, axis=-1)]


def test_quantiser_is_the_nearest_code():
    rng = np.random.default_rng(7)
    cases = []
    for s in (0.5, 0.25, float(np.float32(0.0021937)), float(np.float32(3.3e-3)), 1.0):
        cases += [(n * s, s) for n in (-127, -64, -3, -1, 0, 1, 2, 5, 126, 127)]
        cases += [((n + 0.5) * s, s) for n in (-128, -4, -3, -1, 0, 1, 2, 125, 126)]   # ties
        cases += [(f * s, s) for f in (127.4, 127.5, 127.6, 500.0, -127.5, -900.0)]
        cases += [(float(x), s) for x in rng.standard_normal(40) * 60 * s]
    cases += [(float("inf"), 0.5), (float("-inf"), 0.5), (float("nan"), 0.5), (-0.0, 0.5)]
    for x, s in cases:
        assert oracle.quantize_i8(x, s) == _nearest_code_exact(x, s), (x, s)


def test_quantiser_error_bound():
    """Within range the dequantised code is within half a scale step of x."""
    rng = np.random.default_rng(8)
    s = float(np.float32(0.0123))
    xs = rng.uniform(-127.5 * s, 127.5 * s, 3000)
    got = np.array([oracle.quantize_i8(x, s) for x in xs])
    assert (np.abs(xs - got * s) <= 0.5 * s * (1 + 1e-12)).all()
    assert np.array_equal(got, _nearest_codes(xs, s))


def _small_i8(paged=False, G=2, B=3):
    if paged:
        s = W.spec("c4", batch=B, n_heads=4, n_kv_heads=G, head_dim=64, len_lo=1, len_hi=70,
                   num_blocks=40, max_blocks_per_seq=8)
    else:
        s = W.spec("c3", batch=B, n_heads=4, n_kv_heads=G, head_dim=64, len_lo=1, len_hi=70,
                   max_seq_len=80)
    return s.replace(dtype="i8")


def _geom(s):
    return oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                           max_seq_len=s.max_seq_len, block_size=s.block_size,
                           num_blocks=s.num_blocks, max_blocks_per_seq=s.max_blocks_per_seq)


def _bf16_to64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _logical_v(s, v_cache):
    """Token-major view [.., 16, G, D] of a group-transposed INT8 V cache."""
    if s.block_size:
        return np.ascontiguousarray(v_cache.transpose(0, 3, 1, 2))
    B, n, G, D, _ = v_cache.shape
    return np.ascontiguousarray(v_cache.transpose(0, 1, 4, 2, 3).reshape(B, n * 16, G, D))


def _logical_k(s, k_cache):
    """Token-major view [.., 16, G, D] of a group-major INT8 K cache."""
    if s.block_size:
        return np.ascontiguousarray(k_cache.transpose(0, 2, 1, 3))
    B, n, G, _, D = k_cache.shape
    return np.ascontiguousarray(k_cache.transpose(0, 1, 3, 2, 4).reshape(B, n * 16, G, D))


def _slot(s, p, b):
    pos = int(p.positions[b])
    if s.block_size:
        return int(p.block_table[b, pos // 16]), pos % 16
    return b, pos


@pytest.mark.parametrize("paged", [False, True])
def test_append_stores_nearest_codes_and_nothing_else(paged):
    s = _small_i8(paged)
    p = W.make_problem(s, lengths=np.array([1, 17, 70], np.int32))
    k0, v0 = _logical_k(s, p.k_cache), _logical_v(s, p.v_cache)
    q_rot = oracle.rope_append(_geom(s), p.q, p.k_new, p.v_new, p.k_cache, p.v_cache,
                               p.positions, p.block_table, k_scale=p.k_scale, v_scale=p.v_scale)
    kl, vl = _logical_k(s, p.k_cache), _logical_v(s, p.v_cache)
    changed = np.zeros(kl.shape[:2], bool)
    for b in range(s.batch):
        changed[_slot(s, p, b)] = True
    assert np.array_equal(kl[~changed], k0[~changed])
    assert np.array_equal(vl[~changed], v0[~changed])
    for b in range(s.batch):
        sl = _slot(s, p, b)
        pos = int(p.positions[b])
        for g in range(s.n_kv_heads):
            k_rot = oracle.rope_rotate(_bf16_to64(p.k_new[b, g]), pos)
            assert np.array_equal(kl[sl][g], _nearest_codes(k_rot, p.k_scale[g]))
            v = _bf16_to64(p.v_new[b, g])
            assert np.array_equal(vl[sl][g], _nearest_codes(v, p.v_scale[g]))
    # q is rotated as for any other cache dtype
    assert np.allclose(q_rot[1, 0], oracle.rope_rotate(_bf16_to64(p.q[1, 0]), 16), atol=0)


def test_append_saturates():
    s = _small_i8().replace(batch=1)
    p = W.make_problem(s, lengths=np.array([1], np.int32))
    big = np.full_like(p.k_new, 0x4480)     # bf16 1024.0, far beyond 127 * scale
    neg = np.full_like(p.v_new, 0xC480)     # -1024.0
    oracle.rope_append(_geom(s), None, big, neg, p.k_cache, p.v_cache, p.positions,
                       k_scale=p.k_scale, v_scale=p.v_scale)
    assert (_logical_k(s, p.k_cache)[0, 0] == 127).all()   # position 0: no rotation
    assert (_logical_v(s, p.v_cache)[0, 0] == -127).all()


def _dequantised_f64(s, p):
    """fp64 caches holding scale * code, K and V regrouped to token-major."""
    ks = p.k_scale.astype(np.float64)[:, None]
    vs = p.v_scale.astype(np.float64)[:, None]
    k = np.ascontiguousarray(_logical_k(s, p.k_cache).astype(np.float64) * ks)
    v = np.ascontiguousarray(_logical_v(s, p.v_cache).astype(np.float64) * vs)
    return k, v


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_attention_equals_fp64_attention_on_dequantised_cache(paged, G):
    s = _small_i8(paged, G=G).replace(q_gain=8.0)
    p = W.make_problem(s, lengths=np.array([1, 33, 70], np.int32))
    g8 = _geom(s)
    q_rot = oracle.rope_append(g8, p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions,
                               p.block_table, k_scale=p.k_scale, v_scale=p.v_scale)
    out, lse = oracle.decode_attn(g8, q_rot, p.k_cache, p.v_cache, p.seq_lens, p.block_table,
                                  k_scale=p.k_scale, v_scale=p.v_scale)
    k64, v64 = _dequantised_f64(s, p)
    g64 = oracle.Geometry(s.batch, s.n_heads, G, s.head_dim, "f64", max_seq_len=s.max_seq_len,
                          block_size=s.block_size, num_blocks=s.num_blocks,
                          max_blocks_per_seq=s.max_blocks_per_seq)
    ref, ref_lse = oracle.decode_attn(g64, q_rot, k64, v64, p.seq_lens, p.block_table)
    assert np.abs(out - ref).max() <= 1e-13 * np.abs(ref).max()
    assert np.abs(lse - ref_lse).max() <= 1e-12
    # the units entry point agrees with the full one
    units = [(2, 3), (0, 0), (1, 2)]
    uo, ul = oracle.decode_attn_units(g8, q_rot, p.k_cache, p.v_cache, p.seq_lens, units,
                                      p.block_table, k_scale=p.k_scale, v_scale=p.v_scale)
    for i, (b, h) in enumerate(units):
        assert np.array_equal(uo[i], out[b, h]) and ul[i] == lse[b, h]


def test_scales_and_layout_matter():
    """Plausible mistakes change the result far beyond rounding: K and V
    scales swapped, V read token-major instead of group-transposed, or K
    read token-major instead of group-major."""
    s = _small_i8(G=2)
    p = W.make_problem(s, lengths=np.array([40, 64, 70], np.int32))
    g8 = _geom(s)
    q_rot = oracle.rope_append(g8, p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions,
                               k_scale=p.k_scale, v_scale=p.v_scale)
    out, _ = oracle.decode_attn(g8, q_rot, p.k_cache, p.v_cache, p.seq_lens,
                                k_scale=p.k_scale, v_scale=p.v_scale)
    swapped, _ = oracle.decode_attn(g8, q_rot, p.k_cache, p.v_cache, p.seq_lens,
                                    k_scale=p.v_scale, v_scale=p.k_scale)
    assert np.abs(out - swapped).max() > 1e-3 * np.abs(out).max()
    k64, _ = _dequantised_f64(s, p)
    wrong_v = p.v_cache.reshape(s.batch, s.max_seq_len, 2, s.head_dim).astype(np.float64) * \
        p.v_scale.astype(np.float64)[:, None]
    g64 = oracle.Geometry(s.batch, s.n_heads, 2, s.head_dim, "f64", max_seq_len=s.max_seq_len)
    bad, _ = oracle.decode_attn(g64, q_rot, k64, np.ascontiguousarray(wrong_v), p.seq_lens)
    assert np.abs(out - bad).max() > 1e-2 * np.abs(out).max()
    _, v64 = _dequantised_f64(s, p)
    wrong_k = p.k_cache.reshape(s.batch, s.max_seq_len, 2, s.head_dim).astype(np.float64) * \
        p.k_scale.astype(np.float64)[:, None]
    bad, _ = oracle.decode_attn(g64, q_rot, np.ascontiguousarray(wrong_k), v64, p.seq_lens)
    assert np.abs(out - bad).max() > 1e-2 * np.abs(out).max()


def test_paged_equals_contiguous():
    L = np.array([3, 16, 70], np.int32)
    sp = _small_i8(paged=True)
    sc = _small_i8(paged=False).replace(cfg_id=sp.cfg_id, max_seq_len=128)
    pp, pc = W.make_problem(sp, lengths=L), W.make_problem(sc, lengths=L)
    assert np.array_equal(pp.k_scale, pc.k_scale) and np.array_equal(pp.v_scale, pc.v_scale)
    res = []
    for s, p in ((sp, pp), (sc, pc)):
        g8 = _geom(s)
        q_rot = oracle.rope_append(g8, p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions,
                                   p.block_table, k_scale=p.k_scale, v_scale=p.v_scale)
        res.append(oracle.decode_attn(g8, q_rot, p.k_cache, p.v_cache, p.seq_lens,
                                      p.block_table, k_scale=p.k_scale, v_scale=p.v_scale))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def test_scales_required_exactly_for_int8():
    s = _small_i8()
    p = W.make_problem(s, lengths=np.array([2, 3, 4], np.int32))
    with pytest.raises(TypeError):
        oracle.rope_append(_geom(s), p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions)
    sb = s.replace(dtype="bf16")
    pb = W.make_problem(sb, lengths=np.array([2, 3, 4], np.int32))
    with pytest.raises(ValueError):
        oracle.rope_append(_geom(sb), pb.q, pb.k_new, pb.v_new, pb.k_cache, pb.v_cache,
                           pb.positions, k_scale=p.k_scale, v_scale=p.v_scale)
