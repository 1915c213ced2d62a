"""The decode step in one call (gqa_decode_step) against the two calls it
stands for (rope_append_kv, then gqa_decode_attn_multi over positions + 1
tokens) and against the oracle.

The fused split kernel rotates q with the same fp64 arithmetic as the append
kernel, and its last split's workgroup writes the new key and value before
it reads any tile, so the two paths must agree bit for bit: q_rot, both
caches, out and lse.  The oracle holds the fused step to the same gates as
the two calls (caches bit for bit, q_rot to 1 ulp, outputs to the bf16
gates).  Cases: head dims 64 and 128, n_rep 1-16, both RoPE styles,
contiguous and paged (16- and 32-token blocks) caches, one and many splits
(the direct write and the merge), every decode dispatch order, positions 0
and at split and tile boundaries, a negative position, and the c3 batch at
full size.

Several new tokens (gqa_decode_step_multi, bf16): against
rope_append_kv_multi + gqa_decode_attn_multi bit for bit and the oracle's
window step, for T = 2-16 with 2-32 query rows per KV head, both RoPE
styles, paged caches, windows that straddle splits, a host bound inside the
window, every dispatch order, 65 sequences, and c3 with T = 5 at full size.
"""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import assert_q_rot, bits, device, oracle_step, upload

pytestmark = pytest.mark.gpu

LENS = np.array([1, 2, 16, 17, 32, 33, 128, 129, 300, 511, 512, 1000], np.int32)


def _spec(B, H, G, D, S, block_size=0, q_gain=2.0):
    if block_size:
        nb = S // block_size
        return W.spec("c4", batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                      num_blocks=B * nb + 5, max_blocks_per_seq=nb, block_size=block_size,
                      q_gain=q_gain)
    return W.spec("c3", batch=B, n_heads=H, n_kv_heads=G, head_dim=D, max_seq_len=S,
                  q_gain=q_gain)


def _scales(t, s):
    return dict(k_scale=t["k_scale"], v_scale=t["v_scale"]) if s.dtype == "i8" else {}


def two_calls(p: W.Problem, style, options, positions=None):
    dev = device()
    t = upload(p, dev)
    pos = t["positions"] if positions is None else positions
    if p.spec.dtype == "i8":
        q_rot = kvd.rope_append_kv_int8(t["q"], t["k_new"], t["v_new"], t["k_cache"],
                                        t["v_cache"], t["k_scale"], t["v_scale"], pos,
                                        t["block_table"], base=p.spec.rope_base, style=style)
    else:
        q_rot = kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                   pos, t["block_table"], base=p.spec.rope_base, style=style)
    lens = (pos + 1).contiguous()
    out, lse = kvd.gqa_decode_attn_multi(q_rot[:, None], t["k_cache"], t["v_cache"], lens,
                                         t["block_table"], max_seq_len=p.max_len,
                                         options=options, **_scales(t, p.spec))
    torch.cuda.synchronize()
    return q_rot, out[:, 0], lse[:, 0], t


def fused(p: W.Problem, style, options, positions=None):
    dev = device()
    t = upload(p, dev)
    pos = t["positions"] if positions is None else positions
    q_rot = torch.full(tuple(p.q.shape), float("nan"), dtype=torch.float32, device=dev)
    out, lse = kvd.gqa_decode_step(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                   pos, t["block_table"], base=p.spec.rope_base, style=style,
                                   max_seq_len=p.max_len, q_rot=q_rot, options=options,
                                   **_scales(t, p.spec))
    torch.cuda.synchronize()
    return q_rot, out, lse, t


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32 if a.element_size() == 4 else torch.int16),
                       b.contiguous().view(torch.int32 if b.element_size() == 4 else torch.int16))


def check(p: W.Problem, style="interleaved", options=None, what=""):
    print(f"[step] {what}", flush=True)
    qa, oa, la, ta = two_calls(p, style, options)
    qb, ob, lb, tb = fused(p, style, options)
    assert same(qa, qb), f"{what}: q_rot differs from the two calls"
    assert same(ta["k_cache"], tb["k_cache"]), f"{what}: K cache differs from the two calls"
    assert same(ta["v_cache"], tb["v_cache"]), f"{what}: V cache differs from the two calls"
    assert same(oa, ob), f"{what}: out differs from the two calls"
    assert same(la, lb), f"{what}: lse differs from the two calls"
    oq, oo, ol, okc, ovc = oracle_step(p, style=style)
    assert np.array_equal(bits(W.from_torch(tb["k_cache"])), bits(okc)), f"{what}: K cache"
    assert np.array_equal(bits(W.from_torch(tb["v_cache"])), bits(ovc)), f"{what}: V cache"
    assert_q_rot(qb.cpu().numpy(), oq, what)
    gates.assert_out(ob.cpu().numpy(), oo, p.spec.dtype, what)
    gates.assert_lse(lb.cpu().numpy(), ol, p.spec.dtype, what)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_rep", [1, 2, 4, 8, 16, 20, 32])
def test_head_shapes(D, n_rep):
    G = 2
    s = _spec(LENS.size, G * n_rep, G, D, 1024)
    check(W.make_problem(s, lengths=LENS), what=f"D={D} n_rep={n_rep}")


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("block_size", [0, 16, 32])
@pytest.mark.parametrize("split", [0, 16, 64, 256])
def test_layouts_and_splits(style, block_size, split):
    s = _spec(LENS.size, 8, 2, 128, 1024, block_size)
    opts = kvd.Options(split_tokens=split) if split else None
    check(W.make_problem(s, lengths=LENS), style=style, options=opts,
          what=f"{style} block {block_size} split {split}")


@pytest.mark.parametrize("order", [0, 1, 2, 3, 4])
def test_dispatch_orders(order):
    s = _spec(LENS.size, 16, 4, 128, 1024, q_gain=8.0)
    check(W.make_problem(s, lengths=LENS), options=kvd.Options(split_tokens=64, dispatch_order=order),
          what=f"order {order}")


def test_many_sequences_and_a_negative_position():
    """65 sequences (the work list built by its own launch, dispatch order
    3) with the positions given by hand: sequence 3 has none (position -1:
    no append, out = 0, lse = -inf), the others match the two calls."""
    B = 65
    lens = np.resize(LENS, B)
    s = _spec(B, 8, 2, 64, 1024)
    p = W.make_problem(s, lengths=lens)
    dev = device()
    pos = torch.tensor(lens - 1, dtype=torch.int32, device=dev)
    pos[3] = -1
    qa, oa, la, ta = two_calls(p, "interleaved", None, positions=pos)
    qb, ob, lb, tb = fused(p, "interleaved", None, positions=pos)
    keep = [b for b in range(B) if b != 3]
    assert same(qa[keep], qb[keep])
    assert same(ta["k_cache"], tb["k_cache"]) and same(ta["v_cache"], tb["v_cache"])
    assert same(oa, ob) and same(la, lb)
    assert (ob[3] == 0).all() and torch.isinf(lb[3]).all()


def test_c3_full_size():
    """The batched workload (64 sequences up to 8K tokens): the two paths
    bit for bit, every row against the oracle."""
    check(W.make_problem(W.spec("c3")), what="c3 full")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("block_size,split", [(0, 0), (0, 64), (16, 0), (32, 128)])
def test_int8_cache(D, style, block_size, split):
    """gqa_decode_step_int8: the quantising append inside the INT8 split
    kernel, against rope_append_kv_int8 + the attention call."""
    s = _spec(LENS.size, 8, 2, D, 1024, block_size).replace(dtype="i8")
    opts = kvd.Options(split_tokens=split) if split else None
    check(W.make_problem(s, lengths=LENS), style=style, options=opts,
          what=f"INT8 D={D} {style} block {block_size} split {split}")


def test_int8_c3_full_size():
    check(W.make_problem(W.spec("c3").replace(dtype="i8")), what="INT8 c3 full")


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("block_size", [0, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_two_column_blocks(style, block_size, D):
    """17-32 query heads per KV head (the kernel with two column blocks,
    its q rows staged through LDS): MQA with 32 heads and a 24-head group."""
    for H, G in ((32, 1), (48, 2)):
        s = _spec(LENS.size, H, G, D, 1024, block_size, q_gain=4.0)
        check(W.make_problem(s, lengths=LENS), style=style, options=kvd.Options(split_tokens=64),
              what=f"two blocks H={H} G={G} D={D} {style} block {block_size}")


def test_mqa_128k():
    """The 128K MQA sequence at full size (32 heads on one KV head)."""
    check(W.make_problem(W.spec("c5", n_kv_heads=1)), what="c5 MQA full")


def test_unsupported_shapes_raise():
    """More query heads per KV head than the kernels take (64, or 32 on an
    INT8 cache), or an fp32 cache: the two calls, not this one."""
    for s in (_spec(2, 128, 2, 64, 64), _spec(2, 8, 2, 64, 64).replace(dtype="f32"),
              _spec(2, 64, 2, 64, 64).replace(dtype="i8")):
        p = W.make_problem(s, lengths=np.array([3, 64], np.int32))
        t = upload(p, device())
        with pytest.raises((kvd.KvdError, ValueError)):
            kvd.gqa_decode_step(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                t["positions"])


# ---- several new tokens per sequence (gqa_decode_step_multi) ----

def _window_spec(B, H, G, D, S, block_size=0):
    if block_size:
        nb = S // block_size
        return W.spec("c4", batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                      num_blocks=B * nb + 5, max_blocks_per_seq=nb, block_size=block_size,
                      q_gain=4.0)
    return W.spec("c3", batch=B, n_heads=H, n_kv_heads=G, head_dim=D, max_seq_len=S, q_gain=4.0)


def check_window_step(p: W.Problem, style="interleaved", options=None, what="", max_len=None):
    """rope_append_kv_multi + gqa_decode_attn_multi against the fused step
    bit for bit, then the fused step against the oracle's window step (its
    caches only when a host bound ``max_len`` below the lengths cuts the
    attention)."""
    from tests.test_gpu_multi import oracle_window
    print(f"[step T] {what}", flush=True)
    dev = device()
    msl = p.max_len if max_len is None else max_len
    ta = upload(p, dev)
    qa = kvd.rope_append_kv_multi(ta["q"], ta["k_new"], ta["v_new"], ta["k_cache"],
                                  ta["v_cache"], ta["positions"], ta["block_table"],
                                  base=p.spec.rope_base, style=style)
    oa, la = kvd.gqa_decode_attn_multi(qa, ta["k_cache"], ta["v_cache"],
                                       (ta["positions"] + p.n_query).contiguous(),
                                       ta["block_table"], max_seq_len=msl, options=options)
    tb = upload(p, dev)
    qb = torch.full(tuple(p.q.shape), float("nan"), dtype=torch.float32, device=dev)
    ob, lb = kvd.gqa_decode_step(tb["q"], tb["k_new"], tb["v_new"], tb["k_cache"],
                                 tb["v_cache"], tb["positions"], tb["block_table"],
                                 base=p.spec.rope_base, style=style, max_seq_len=msl,
                                 q_rot=qb, options=options)
    torch.cuda.synchronize()
    assert ob.shape == oa.shape and lb.shape == la.shape
    assert same(qa, qb), f"{what}: q_rot differs from the two calls"
    assert same(ta["k_cache"], tb["k_cache"]), f"{what}: K cache differs from the two calls"
    assert same(ta["v_cache"], tb["v_cache"]), f"{what}: V cache differs from the two calls"
    assert same(oa, ob), f"{what}: out differs from the two calls"
    assert same(la, lb), f"{what}: lse differs from the two calls"
    oq, oo, ol, okc, ovc = oracle_window(p, style=style)
    assert np.array_equal(bits(W.from_torch(tb["k_cache"])), bits(okc)), f"{what}: K cache"
    assert np.array_equal(bits(W.from_torch(tb["v_cache"])), bits(ovc)), f"{what}: V cache"
    assert_q_rot(qb.cpu().numpy(), oq, what)
    if msl < p.max_len:
        return
    gates.assert_out(ob.cpu().numpy(), oo, "bf16", what)
    gates.assert_lse(lb.cpu().numpy(), ol, "bf16", what)


@pytest.mark.parametrize("T,H,G", [(2, 8, 2), (5, 8, 2), (8, 8, 2), (16, 2, 2), (5, 24, 4),
                                   (8, 32, 8), (16, 4, 2)])
@pytest.mark.parametrize("D", [64, 128])
def test_several_tokens_head_shapes(T, H, G, D):
    """T new tokens with T x n_rep query rows from 2 to 32 (one and two
    column blocks), windows that straddle 16- and 64-token splits."""
    s = _window_spec(LENS.size, H, G, D, 1024)
    p = W.make_window(s, T, lengths=np.maximum(LENS, T))
    check_window_step(p, options=kvd.Options(split_tokens=64),
                      what=f"T={T} H={H} G={G} D={D}")


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("block_size", [0, 16, 32])
@pytest.mark.parametrize("split", [0, 16, 48])
def test_several_tokens_layouts(style, block_size, split):
    s = _window_spec(LENS.size, 8, 2, 128, 1024, block_size)
    p = W.make_window(s, 5, lengths=np.maximum(LENS, 5))
    opts = kvd.Options(split_tokens=split) if split else None
    check_window_step(p, style=style, options=opts,
                      what=f"T=5 {style} block {block_size} split {split}")


def test_several_tokens_past_the_host_bound():
    """max_seq_len below the window's end: the tokens past it are still
    appended (by the last split's workgroup) and not attended."""
    s = _window_spec(3, 8, 2, 64, 256)
    p = W.make_window(s, 6, lengths=np.array([6, 153, 200], np.int32))
    check_window_step(p, options=kvd.Options(split_tokens=32), what="T=6 host bound 150",
                      max_len=150)


def test_several_tokens_c3_full_size():
    """The batched workload (64 sequences up to 8K tokens, 32 heads on 8 KV
    heads) verifying 5 draft tokens: 20 query rows per KV head."""
    s = W.spec("c3")
    p = W.make_window(s, 5)
    check_window_step(p, what="c3 T=5 full")


def test_several_tokens_unsupported():
    """More than 16 new tokens, more than 32 query rows per KV head, or an
    INT8 cache: the two calls, not this one."""
    for (T, H, G, dt) in ((17, 2, 2, "bf16"), (9, 8, 2, "bf16"), (2, 8, 2, "i8")):
        s = _window_spec(2, H, G, 64, 64).replace(dtype=dt)
        p = W.make_window(s, T, lengths=np.array([T, 64], np.int32))
        t = upload(p, device())
        with pytest.raises((kvd.KvdError, ValueError)):
            kvd.gqa_decode_step(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                t["positions"], t["block_table"])


@pytest.mark.parametrize("order", [0, 1, 2, 3, 4])
def test_several_tokens_dispatch_orders(order):
    """Every decode dispatch order with T = 5: the work lists (orders 3 and
    4) read the lengths as positions + T."""
    s = _window_spec(LENS.size, 16, 4, 128, 1024)
    p = W.make_window(s, 5, lengths=np.maximum(LENS, 5))
    check_window_step(p, options=kvd.Options(split_tokens=64, dispatch_order=order),
                      what=f"T=5 order {order}")


def test_several_tokens_many_sequences():
    """65 sequences (the work list built by its own launch) with 3 new
    tokens each, on a paged cache."""
    lens = np.maximum(np.resize(LENS, 65), 3)
    s = _window_spec(65, 8, 2, 64, 1024, block_size=16)
    check_window_step(W.make_window(s, 3, lengths=lens), what="T=3 B=65 paged")
