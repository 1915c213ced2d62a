"""The append (RoPE + cache write) has two kernels: a vector form for
16-byte-aligned buffers and 128 tokens or more, which moves runs of 4
elements, and the scalar form otherwise, one rotation pair per thread.
Both compute each element the same way, so for the same inputs they must
write the same bits: q_rot, the caches and the rings are compared bit for
bit, with a q one element off 16-byte alignment sending the second call to
the scalar form.
The aligned result is also held to the oracle (caches bit for bit, q_rot to
1 ulp).

Shapes cover the slice layouts of both kernels: a decode step of 130
sequences (pair and value workgroups per token), a few tokens per sequence,
and 4096 tokens (one workgroup per token).
"""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
import oracle
from kv_cache_gqa_decode_amd import workloads as W
from tests.gpu_helpers import assert_q_rot, bits, device, geom, upload

pytestmark = pytest.mark.gpu


def off_alignment(x: torch.Tensor) -> torch.Tensor:
    """A copy of x whose data starts one element past a 16-byte boundary."""
    buf = torch.empty(x.numel() + 16, dtype=x.dtype, device=x.device)
    y = buf[1:1 + x.numel()].view(x.shape)
    y.copy_(x)
    assert y.data_ptr() % 16 != 0
    return y


def _append(t, s, q, style, multi):
    sc = dict(k_scale=t["k_scale"], v_scale=t["v_scale"]) if s.dtype == "i8" else {}
    if multi:
        return kvd.rope_append_kv_multi(q, t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                        t["positions"], t["block_table"], base=s.rope_base,
                                        style=style, **sc)
    if s.dtype == "i8":
        return kvd.rope_append_kv_int8(q, t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                       t["k_scale"], t["v_scale"], t["positions"],
                                       t["block_table"], base=s.rope_base, style=style)
    return kvd.rope_append_kv(q, t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                              t["positions"], t["block_table"], base=s.rope_base, style=style)


def _both(p: W.Problem, style: str, multi: bool):
    """(q_rot, K cache, V cache) of the aligned call and of the call with q
    off alignment, as host arrays."""
    dev = device()
    s = p.spec
    res = []
    for shift in (False, True):
        t = upload(p, dev)
        q = off_alignment(t["q"]) if shift else t["q"]
        q_rot = _append(t, s, q, style, multi)
        torch.cuda.synchronize()
        res.append((q_rot.cpu().numpy(), W.from_torch(t["k_cache"]), W.from_torch(t["v_cache"])))
    (qa, ka, va), (qb, kb, vb) = res
    assert np.array_equal(qa.view(np.uint32), qb.view(np.uint32)), "q_rot differs"
    assert np.array_equal(bits(ka), bits(kb)), "K cache differs"
    assert np.array_equal(bits(va), bits(vb)), "V cache differs"
    return qa, ka, va


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("block_size", [0, 16, 32])
@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_step_both_kernels(dtype, block_size, style, D):
    B, H, G, S = 130, 12, 4, 128
    if block_size:
        nb = S // block_size
        s = W.spec("c4", dtype=dtype, batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                   num_blocks=B * nb + 3, max_blocks_per_seq=nb, block_size=block_size)
    else:
        s = W.spec("c3", dtype=dtype, batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                   max_seq_len=S)
    p = W.make_problem(s, lengths=np.resize(np.array([1, 2, 17, 64, 100, 128], np.int32), B))
    qa, ka, va = _both(p, style, multi=False)
    g = geom(s)
    kc, vc = p.k_cache.copy(), p.v_cache.copy()
    sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if dtype == "i8" else {}
    oq = oracle.rope_append(g, p.q, p.k_new, p.v_new, kc, vc, p.positions, p.block_table,
                            base=s.rope_base, style=style, **sc)
    assert np.array_equal(bits(ka), bits(kc)), "K cache differs from the oracle's"
    assert np.array_equal(bits(va), bits(vc)), "V cache differs from the oracle's"
    assert_q_rot(qa, oq, f"{dtype} block {block_size} {style} D={D}")


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("B,T,S", [(17, 8, 256), (9, 40, 256), (1, 4096, 4096)])
@pytest.mark.parametrize("block_size", [0, 32])
def test_several_tokens_both_kernels(dtype, B, T, S, block_size):
    """From 16 tokens per sequence INT8 caches take v by 16-token groups:
    chunks that start and end inside a group (byte stores) and whole groups
    (16-byte stores); 8 tokens keep the per-token v items."""
    if block_size:
        nb = S // block_size
        s = W.spec("c4", dtype=dtype, batch=B, n_heads=8, n_kv_heads=2, head_dim=64,
                   num_blocks=B * nb + 3, max_blocks_per_seq=nb, block_size=block_size)
    else:
        s = W.spec("c3", dtype=dtype, batch=B, n_heads=8, n_kv_heads=2, head_dim=64,
                   max_seq_len=S)
    lens = np.resize(np.array([T, T + 100, S, T + 7], np.int32), B)
    p = W.make_window(s, T, lengths=lens)
    qa, ka, va = _both(p, "half", multi=True)
    g = geom(s)
    kc, vc = p.k_cache.copy(), p.v_cache.copy()
    sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if dtype == "i8" else {}
    oq = oracle.rope_append(g, p.q, p.k_new, p.v_new, kc, vc, p.positions, p.block_table,
                            base=s.rope_base, style="half", n_query=T, **sc)
    assert np.array_equal(bits(ka), bits(kc)), "K cache differs from the oracle's"
    assert np.array_equal(bits(va), bits(vc)), "V cache differs from the oracle's"
    assert_q_rot(qa, oq, f"{dtype} B={B} T={T} block {block_size}")


@pytest.mark.parametrize("block_size", [0, 16])
def test_mixed_step_both_kernels(block_size):
    """The mixed-precision append (the token leaving the bf16 ring is
    quantised into the INT8 history): both kernels, rings and caches bit for
    bit."""
    dev = device()
    B, H, G, D, S, Wn = 130, 8, 2, 128, 128, 16
    if block_size:
        nb = S // block_size
        s = W.spec("c4", dtype="i8", batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                   num_blocks=B * nb + 3, max_blocks_per_seq=nb, block_size=block_size)
    else:
        s = W.spec("c3", dtype="i8", batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                   max_seq_len=S)
    p = W.make_mixed(s, Wn, lengths=np.resize(np.array([1, 15, 16, 17, 100, 128], np.int32), B))
    res = []
    for shift in (False, True):
        t = upload(p, dev)
        kr, vr = W.as_torch(p.k_recent, dev), W.as_torch(p.v_recent, dev)
        q = off_alignment(t["q"]) if shift else t["q"]
        q_rot = kvd.rope_append_kv_mixed(q, t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                         t["k_scale"], t["v_scale"], kr, vr, t["positions"],
                                         t["block_table"], base=s.rope_base)
        torch.cuda.synchronize()
        res.append([q_rot.cpu().numpy()] + [W.from_torch(x) for x in
                                            (t["k_cache"], t["v_cache"], kr, vr)])
    for name, a, b in zip(("q_rot", "K cache", "V cache", "K ring", "V ring"), *res):
        assert np.array_equal(bits(a), bits(b)), f"{name} differs"
    g = geom(s)
    okc, ovc = p.k_cache.copy(), p.v_cache.copy()
    okr, ovr = p.k_recent.copy(), p.v_recent.copy()
    oq = oracle.rope_append_mixed(g, Wn, p.q, p.k_new, p.v_new, okc, ovc, okr, ovr, p.positions,
                                  p.block_table, base=s.rope_base, k_scale=p.k_scale,
                                  v_scale=p.v_scale)
    q_rot, kc, vc, kr, vr = res[0]
    for name, a, b in (("K cache", kc, okc), ("V cache", vc, ovc), ("K ring", kr, okr),
                       ("V ring", vr, ovr)):
        assert np.array_equal(bits(a), bits(b)), f"{name} differs from the oracle's"
    assert_q_rot(q_rot, oq, f"mixed block {block_size}")
