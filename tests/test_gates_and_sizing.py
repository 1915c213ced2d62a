"""The sizing helper against the cache sizes the pages print, and the parity
gates' power to reject plausible mistakes (planted in oracle outputs, on the
CPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from kv_cache_gqa_decode_amd import sizing
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_sizes.json")


def test_cache_size_formula_matches_printed_numbers():
    g = json.load(open(GOLDEN, encoding="utf-8"))
    for case in g["absolute"]:
        n = sizing.kv_cache_bytes(case["batch"], case["layers"], case["kv_heads"],
                                  case["seq_len"], case["head_dim"], case["dtype_bytes"])
        assert n / 2**30 == case["printed_gib"]
    base = g["absolute"][0]
    mha = sizing.kv_cache_bytes(1, 32, 32, 1024, 128, 2)
    for case in g["relative_to_mha"]:
        n = sizing.kv_cache_bytes(1, 32, case["kv_heads"], 1024, 128, 2)
        assert round(100 * n / mha) == case["printed_percent"]
    ex = g["groups_example"]
    assert ex["num_heads"] // ex["num_groups"] == ex["heads_per_group"]
    assert sizing.kv_cache_bytes(1, 1, ex["num_groups"], 1, 128, 2) / \
        sizing.kv_cache_bytes(1, 1, ex["num_heads"], 1, 128, 2) == ex["fraction_of_mha"]
    assert base["seq_len"] == 1024


def test_decode_read_bytes_sum_over_sequences():
    assert sizing.decode_kv_read_bytes([131072], 8, 128, 2) == 512 * 2**20
    assert sizing.decode_kv_read_bytes([131072], 1, 128, 2) == 64 * 2**20
    assert sizing.decode_kv_read_bytes([256], 2, 64, 4) == 262144
    assert sizing.decode_kv_read_bytes([3, 5], 8, 128, 2) == 8 * 8 * 128 * 2 * 2


def _c2_small():
    s = W.spec("c2", max_seq_len=512, len_lo=512, len_hi=512)
    p = W.make_problem(s)
    g = oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, "bf16",
                        max_seq_len=s.max_seq_len)
    q_rot = oracle.rope_append(g, p.q, p.k_new, p.v_new, p.k_cache, p.v_cache, p.positions)
    return s, p, g, q_rot


def test_gates_reject_planted_mistakes():
    s, p, g, q_rot = _c2_small()
    ref, lse = oracle.decode_attn(g, q_rot, p.k_cache, p.v_cache, p.seq_lens)
    assert gates.out_ok(ref, ref, "bf16") and gates.lse_ok(lse, lse, "bf16")
    # an all-zero output (at 131072 tokens it would pass the absolute gate
    # alone: outputs there are ~1e-3) is rejected by the normwise gate
    zero = np.zeros_like(ref)
    assert gates.out_errors(zero, ref)["normwise"] == 1.0
    assert not gates.out_ok(zero, ref, "bf16")
    # a dropped split (tokens 256..383 never read)
    kk, vv = p.k_cache.copy(), p.v_cache.copy()
    keep = np.r_[0:256, 384:512]
    kk[0, : keep.size] = p.k_cache[0, keep]
    vv[0, : keep.size] = p.v_cache[0, keep]
    dropped, dl = oracle.decode_attn(g, q_rot, kk, vv, np.array([keep.size], np.int32))
    assert not gates.out_ok(dropped, ref, "bf16") or not gates.lse_ok(dl, lse, "bf16")
    # the new token not attended (off-by-one length)
    short, sl = oracle.decode_attn(g, q_rot, p.k_cache, p.v_cache, p.seq_lens - 1)
    assert not gates.out_ok(short, ref, "bf16") or not gates.lse_ok(sl, lse, "bf16")
    # wrong GQA mapping h -> h % G
    H, G = s.n_heads, s.n_kv_heads
    perm = np.array([(h % G) * (H // G) + h // G for h in range(H)])
    wrong, _ = oracle.decode_attn(g, np.ascontiguousarray(q_rot[:, perm]), p.k_cache,
                                  p.v_cache, p.seq_lens)
    assert not gates.out_ok(wrong[:, np.argsort(perm)], ref, "bf16")
    # q left un-rotated
    unrot = (p.q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bad, _ = oracle.decode_attn(g, unrot, p.k_cache, p.v_cache, p.seq_lens)
    assert not gates.out_ok(bad, ref, "bf16")
    # the scale left out
    noscale, _ = oracle.decode_attn(g, q_rot, p.k_cache, p.v_cache, p.seq_lens, scale=1.0)
    assert not gates.out_ok(noscale, ref, "bf16")


def test_fp32_gate_rejects_bf16_level_error():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((8, 64))
    assert gates.out_ok(ref * (1 + 1e-7), ref, "f32")
    assert not gates.out_ok(ref + 2.0**-8 * np.abs(ref).max(), ref, "f32")


def test_prefill_gate_rejects_planted_mistakes():
    """The looser prefill gate (bf16 q and P) still rejects the mistakes a
    causal prefill kernel can make: an off-by-one causal bound, a missing
    mask inside the window, a dropped history and the h mod G mapping."""
    T, B, H, G, D = 24, 2, 8, 2, 64
    s = W.spec("c3", batch=B, n_heads=H, n_kv_heads=G, head_dim=D, max_seq_len=256, q_gain=2.0)
    L = np.array([T, 200], np.int32)
    p = W.make_window(s, T, lengths=L)
    g = oracle.Geometry(B, H, G, D, "bf16", max_seq_len=s.max_seq_len)
    kc, vc = p.k_cache.copy(), p.v_cache.copy()
    q_rot = oracle.rope_append(g, p.q, p.k_new, p.v_new, kc, vc, p.positions, n_query=T)
    ref, lse = oracle.decode_attn(g, q_rot, kc, vc, p.seq_lens, n_query=T)
    assert gates.out_ok(ref, ref, "prefill") and gates.lse_ok(lse, lse, "prefill")
    # one token too few for every query (the bound taken exclusive of the query's own token)
    short, sl = oracle.decode_attn(g, q_rot, kc, vc, p.seq_lens - 1, n_query=T)
    short[0, 0] = 0.0                  # query 0 of an empty history then sees nothing
    assert not gates.out_ok(short, ref, "prefill")
    # no mask inside the window: every query sees all T new tokens
    flat = oracle.Geometry(B * T, H, G, D, "bf16", max_seq_len=s.max_seq_len)
    kk = np.repeat(kc, T, axis=0); vv = np.repeat(vc, T, axis=0)
    unmasked, _ = oracle.decode_attn(flat, np.ascontiguousarray(q_rot.reshape(B * T, H, D)), kk,
                                     vv, np.repeat(p.seq_lens, T))
    assert not gates.out_ok(unmasked.reshape(ref.shape), ref, "prefill")
    # the history of sequence 1 dropped (only the window attended)
    kz, vz = kc.copy(), vc.copy()
    kz[1, :200 - T] = 0; vz[1, :200 - T] = 0
    nohist, _ = oracle.decode_attn(g, q_rot, kz, vz, p.seq_lens, n_query=T)
    assert not gates.out_ok(nohist, ref, "prefill")
    # GQA mapping h -> h mod G
    perm = np.array([(h % G) * (H // G) + h // G for h in range(H)])
    wrong, _ = oracle.decode_attn(g, np.ascontiguousarray(q_rot[:, :, perm]), kc, vc, p.seq_lens,
                                  n_query=T)
    assert not gates.out_ok(wrong[:, :, np.argsort(perm)], ref, "prefill")


@pytest.mark.parametrize("T", [1, 2, 5, 17])
def test_window_key_count_brute_force(T):
    lens = np.array([0, 1, T - 1, T, T + 1, 40, 300], np.int64).clip(0)
    brute = sum(max(0, min(int(L), int(L) - T + 1 + t)) for L in lens for t in range(T))
    assert sizing.window_key_count(lens, T) == brute
    # a prompt from empty: the causal triangle
    assert sizing.window_key_count([T], T) == T * (T + 1) // 2
    assert sizing.window_attention_flops([T], T, 32, 128) == 4 * 128 * 32 * T * (T + 1) // 2
