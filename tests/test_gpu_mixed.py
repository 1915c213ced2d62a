"""GPU parity of the mixed-precision cache (rope_append_kv_mixed +
gqa_decode_attn_mixed) against the oracle on the same seeded inputs.

"Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §4.3: the W newest tokens of
a sequence stay in bf16 rings, the older history is INT8 with per-head
scales.  The appended ring rows and the codes of the token that leaves the
ring must match bit for bit (the whole INT8 cache and both rings are
compared); outputs and lse pass the bf16 gates (both sides read the same
codes and bf16 values, fp32 accumulation).  Every slot the step must not
read holds poison (INT8 code 127, bf16 NaN).
"""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
import oracle
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import assert_q_rot, device, geom, upload

pytestmark = pytest.mark.gpu


def _spec(B, H, G, D, S, block_size=0, q_gain=1.0):
    if block_size:
        nbps = S // block_size
        return W.spec("c4", dtype="i8", batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                      num_blocks=B * nbps + 8, max_blocks_per_seq=nbps, block_size=block_size,
                      q_gain=q_gain)
    return W.spec("c3", dtype="i8", batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                  max_seq_len=S, q_gain=q_gain)


def run_mixed(p: W.Problem, what="", max_len=None, options=None, units=None):
    dev = device()
    s = p.spec
    Wn = p.window
    msl = p.max_len if max_len is None else max_len
    print(f"[mixed] {what} W={Wn} lens={p.seq_lens[:8].tolist()}", flush=True)
    t = upload(p, dev)
    kr = W.as_torch(p.k_recent, dev)
    vr = W.as_torch(p.v_recent, dev)
    q_rot = kvd.rope_append_kv_mixed(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["k_scale"], t["v_scale"], kr, vr, t["positions"],
                                     t["block_table"], base=s.rope_base)
    out, lse = kvd.gqa_decode_attn_mixed(q_rot, t["k_cache"], t["v_cache"], t["k_scale"],
                                         t["v_scale"], kr, vr, t["seq_lens"], t["block_table"],
                                         max_seq_len=msl, options=options)
    torch.cuda.synchronize()
    g = geom(s)
    okc, ovc = p.k_cache.copy(), p.v_cache.copy()
    okr, ovr = p.k_recent.copy(), p.v_recent.copy()
    oq = oracle.rope_append_mixed(g, Wn, p.q, p.k_new, p.v_new, okc, ovc, okr, ovr, p.positions,
                                  p.block_table, base=s.rope_base, k_scale=p.k_scale,
                                  v_scale=p.v_scale)
    lens = np.minimum(p.seq_lens, msl).astype(np.int32)
    oo, ol = oracle.decode_attn_mixed(g, Wn, oq, okc, ovc, okr, ovr, lens, p.block_table,
                                      k_scale=p.k_scale, v_scale=p.v_scale, units=units)
    assert np.array_equal(W.from_torch(t["k_cache"]), okc), f"{what}: INT8 K cache"
    assert np.array_equal(W.from_torch(t["v_cache"]), ovc), f"{what}: INT8 V cache"
    assert np.array_equal(W.from_torch(kr), okr), f"{what}: K ring"
    assert np.array_equal(W.from_torch(vr), ovr), f"{what}: V ring"
    assert_q_rot(q_rot.cpu().numpy(), oq, what)
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    if units is not None:
        ub, uh = (np.array([u[i] for u in units]) for i in range(2))
        go, gl = go[ub, uh], gl[ub, uh]
    e = gates.assert_out(go, oo, "i8", what)
    gates.assert_lse(gl, ol, "i8", what)
    print(f"[mixed] {what}: {e}", flush=True)
    return e


@pytest.mark.parametrize("window", [16, 100, 256])
@pytest.mark.parametrize("block_size", [0, 16, 32])
def test_ragged_batch(window, block_size):
    """Sequences shorter than, equal to, one past and far beyond the window
    (the token leaving the ring is quantised into the INT8 cache)."""
    lens = np.array([1, 5, window, window + 1, window + 2, 700, 1024, 333], np.int32)
    s = _spec(lens.size, 32, 8, 128, 1024, block_size)
    run_mixed(W.make_mixed(s, window, lengths=lens), what=f"ragged bs={block_size}")


@pytest.mark.parametrize("H,G,D", [(32, 32, 128), (32, 1, 128), (16, 2, 64), (24, 8, 64)])
def test_head_shapes(H, G, D):
    """n_rep 1, 32 (both kernels' wide forms), 8 and 3; D 64 and 128."""
    lens = np.array([40, 300, 520], np.int32)
    s = _spec(lens.size, H, G, D, 528)
    run_mixed(W.make_mixed(s, 128, lengths=lens), what=f"H={H} G={G} D={D}")


@pytest.mark.parametrize("split,order", [(16, None), (64, 0), (128, 1), (256, 2), (512, 3),
                                         (0, 4)])
def test_split_layouts_and_orders(split, order):
    lens = np.array([17, 900, 1500, 2048, 64, 1200], np.int32)
    s = _spec(lens.size, 32, 8, 128, 2048)
    run_mixed(W.make_mixed(s, 192, lengths=lens), what=f"split {split} order {order}",
              options=kvd.Options(split_tokens=split, dispatch_order=order))


def test_peaked_scores():
    """q x 32: the running max moves inside the history and the ring."""
    lens = np.array([600, 1024], np.int32)
    s = _spec(lens.size, 32, 8, 128, 1024, q_gain=32.0)
    run_mixed(W.make_mixed(s, 160, lengths=lens), what="peaked")


def test_host_bound_below_the_window():
    """max_seq_len below the window: no history part; the attended tokens are
    clamped to the bound on both sides."""
    lens = np.array([50, 300, 400], np.int32)
    s = _spec(lens.size, 32, 8, 128, 512)
    p = W.make_mixed(s, 256, lengths=lens)
    run_mixed(p, what="bound 200 < window", max_len=200)


def test_full_size_batched():
    """The batched workload's shape (B 64, H 32, G 8, D 128, lengths
    U[512, 8192]) on a mixed cache with a 256-token window: every row."""
    s = W.spec("c3", dtype="i8")
    run_mixed(W.make_mixed(s, 256), what="c3 mixed W=256, all rows")


def test_full_size_long_context():
    """One 128K sequence with 8 KV heads and a 1024-token window: every row."""
    s = W.spec("c5", n_kv_heads=8, dtype="i8")
    run_mixed(W.make_mixed(s, 1024), what="c5 G=8 mixed W=1024, all rows")
