"""Shared pieces of the GPU parity tests: run one decode step through the
C ABI and the same step through the oracle, on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import workloads as W


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    return torch.device("cuda", 0)


def geom(s: W.Spec) -> oracle.Geometry:
    return oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                           max_seq_len=s.max_seq_len, block_size=s.block_size,
                           num_blocks=s.num_blocks, max_blocks_per_seq=s.max_blocks_per_seq)


def upload(p: W.Problem, dev):
    t = {k: W.as_torch(getattr(p, k), dev) for k in
         ("q", "k_new", "v_new", "k_cache", "v_cache", "positions", "seq_lens")}
    t["block_table"] = None if p.block_table is None else W.as_torch(p.block_table, dev)
    for k in ("k_scale", "v_scale"):
        a = getattr(p, k)
        t[k] = None if a is None else W.as_torch(a, dev)
    return t


def opts(kernel=None, split=0, tail=(0, -1), order=None, events=None):
    """Per-call options of the attention calls (None when all automatic)."""
    if kernel is None and split == 0 and tail[0] == 0 and order is None and events is None:
        return None
    return kvd.Options(kernel=kernel, split_tokens=split, tail_split_tokens=tail[0],
                       tail_span_tokens=max(tail[1], 0), dispatch_order=order, events=events)


def gpu_step(t, s: W.Spec, max_len: int, style="interleaved", scale=None, sync=True,
             options=None):
    if s.dtype == "i8":
        q_rot = kvd.rope_append_kv_int8(t["q"], t["k_new"], t["v_new"], t["k_cache"],
                                        t["v_cache"], t["k_scale"], t["v_scale"], t["positions"],
                                        t["block_table"], base=s.rope_base, style=style)
        out, lse = kvd.gqa_decode_attn_int8(q_rot, t["k_cache"], t["v_cache"], t["k_scale"],
                                            t["v_scale"], t["seq_lens"], t["block_table"],
                                            scale=scale, max_seq_len=max_len, options=options)
        if sync:
            torch.cuda.synchronize()
        return q_rot, out, lse
    q_rot = kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                               t["positions"], t["block_table"], base=s.rope_base, style=style)
    out, lse = kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                   t["block_table"], scale=scale, max_seq_len=max_len,
                                   options=options)
    if sync:
        torch.cuda.synchronize()
    return q_rot, out, lse


def oracle_step(p: W.Problem, style="interleaved", units=None, scale=None):
    """Returns (q_rot fp64, out, lse, k_cache, v_cache) computed by the oracle
    on host copies of the inputs.  With ``units`` only those (b, h) rows."""
    s = p.spec
    g = geom(s)
    kc, vc = p.k_cache.copy(), p.v_cache.copy()
    sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if s.dtype == "i8" else {}
    q_rot = oracle.rope_append(g, p.q, p.k_new, p.v_new, kc, vc, p.positions, p.block_table,
                               base=s.rope_base, style=style, **sc)
    if units is None:
        out, lse = oracle.decode_attn(g, q_rot, kc, vc, p.seq_lens, p.block_table, scale=scale,
                                      **sc)
    else:
        out, lse = oracle.decode_attn_units(g, q_rot, kc, vc, p.seq_lens, units, p.block_table,
                                            scale=scale, **sc)
    return q_rot, out, lse, kc, vc


def appended_rows(p: W.Problem):
    """Index tuples (leading two indices) of the appended token rows in the
    bf16 / fp32 cache arrays: (b, position) when contiguous, (block, row in
    block) in a paged pool of p.spec.block_size-token blocks."""
    s = p.spec
    rows = []
    for b in range(s.batch):
        pos = int(p.positions[b])
        if s.block_size:
            bs = s.block_size
            rows.append((int(p.block_table[b, pos // bs]), pos % bs))
        else:
            rows.append((b, pos))
    return rows


def assert_q_rot(got, ref, what=""):
    """q_rot against the oracle's fp64 rotation.  Both sides rotate in fp64
    and round once to fp32, so they agree to 1 ulp -- except where the
    rotated value nearly cancels (|a cos - c sin| << |a|): there the fp64
    rounding of the angle itself (P * theta, up to ~1e-11 rad at positions
    near 131072, and the 1-ulp freedom of libm's pow / sin / cos) is no
    longer small against the result.  Such elements must still agree to
    1e-9 of their row's largest element, far below any effect on the
    attention and far above a wrong angle or pair."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float64)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.astype(np.float32).view(np.int32))
    near = np.abs(got.astype(np.float64) - ref) <= 1e-9 * np.abs(ref).max(axis=-1, keepdims=True)
    ok = (ulp <= 1) | near
    assert ok.all(), (f"{what}: q_rot differs at {(~ok).sum()} elements "
                      f"(max {ulp[~ok].max()} ulp)")
    return int((ulp > 1).sum())


def bits(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.int8:
        return a
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)
