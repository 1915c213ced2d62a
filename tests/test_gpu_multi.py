"""GPU parity of the multi-token step (rope_append_kv_multi and
gqa_decode_attn_multi, T = n_query new tokens per sequence) through the C ABI
against the oracle's multi-token step on the same seeded inputs.

"Transformer架构优化实战2026" §五: the target model checks the gamma draft
tokens of speculative decoding in one forward (gamma = 4 there, T = 5); each
of the T queries attends the cache and the new tokens up to its own position
([KVGR] §5.1 b.v).  Caches must match bit for bit, q_rot to 1 ulp (gpu_helpers.assert_q_rot), outputs
and lse within the bf16 gates (INT8 caches use them too: both sides read the
same codes).  Every case compares every output row and lse, and the caches
in full.
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import assert_q_rot, device, geom, opts, upload

pytestmark = pytest.mark.gpu

RAGGED = np.array([5, 6, 15, 16, 17, 20, 63, 64, 65, 300, 1000, 1024], np.int32)


def _scales(t, s):
    return dict(k_scale=t["k_scale"], v_scale=t["v_scale"]) if s.dtype == "i8" else {}


def gpu_window(t, s: W.Spec, max_len: int, style="interleaved", options=None):
    q_rot = kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["positions"], t["block_table"], base=s.rope_base,
                                     style=style, **_scales(t, s))
    out, lse = kvd.gqa_decode_attn_multi(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                         t["block_table"], max_seq_len=max_len, options=options,
                                         **_scales(t, s))
    torch.cuda.synchronize()
    return q_rot, out, lse


def oracle_window(p: W.Problem, style="interleaved", units=None):
    """The oracle's step on a window problem; arrays keep the T axis (also
    for T = 1, which the oracle takes in the single-token layout)."""
    s = p.spec
    g = geom(s)
    T = p.n_query
    one = T == 1 and p.q.ndim == 4
    sq = (lambda a: np.ascontiguousarray(a[:, 0])) if one else (lambda a: a)
    kc, vc = p.k_cache.copy(), p.v_cache.copy()
    sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if s.dtype == "i8" else {}
    q_rot = oracle.rope_append(g, sq(p.q), sq(p.k_new), sq(p.v_new), kc, vc, p.positions,
                               p.block_table, base=s.rope_base, style=style, n_query=T, **sc)
    if units is None:
        out, lse = oracle.decode_attn(g, q_rot, kc, vc, p.seq_lens, p.block_table, n_query=T,
                                      **sc)
        if one:
            out, lse = out[:, None], lse[:, None]
    else:
        u = [(b, h) for b, _, h in units] if one else units
        out, lse = oracle.decode_attn_units(g, q_rot, kc, vc, p.seq_lens, u, p.block_table,
                                            n_query=T, **sc)
    return (q_rot[:, None] if one else q_rot), out, lse, kc, vc


def check_window(p: W.Problem, split=0, style="interleaved", what=""):
    dev = device()
    s = p.spec
    print(f"[window] {what}", flush=True)
    t = upload(p, dev)
    q_rot, out, lse = gpu_window(t, s, p.max_len, style=style, options=opts(None, split))
    oq, oo, ol, okc, ovc = oracle_window(p, style=style)
    assert np.array_equal(W.from_torch(t["k_cache"]), okc), f"{what}: K cache differs"
    assert np.array_equal(W.from_torch(t["v_cache"]), ovc), f"{what}: V cache differs"
    qr = q_rot.cpu().numpy()
    assert_q_rot(qr, oq, what)
    gd = "i8" if s.dtype == "i8" else "bf16"
    gates.assert_out(out.cpu().numpy(), oo, gd, what)
    gates.assert_lse(lse.cpu().numpy(), ol, gd, what)


def _spec(dtype, paged, block_size=16, **kw):
    if paged:
        s = W.spec("c4", batch=RAGGED.size, num_blocks=16000 // block_size,
                   max_blocks_per_seq=1024 // block_size, block_size=block_size, q_gain=8.0, **kw)
    else:
        s = W.spec("c3", batch=RAGGED.size, max_seq_len=1024, q_gain=8.0, **kw)
    return s.replace(dtype=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("T", [2, 5])
@pytest.mark.parametrize("split", [0, 16, 48])
def test_window_contiguous(dtype, T, split):
    p = W.make_window(_spec(dtype, False), T, lengths=RAGGED)
    check_window(p, split=split, what=f"{dtype} contiguous T={T} split={split}")


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("split", [0, 32])
def test_window_paged(dtype, block_size, split):
    p = W.make_window(_spec(dtype, True, block_size), 5, lengths=RAGGED)
    check_window(p, split=split, what=f"{dtype} paged{block_size} T=5 split={split}")


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("n_rep,T", [(1, 5), (1, 32), (2, 16), (4, 5), (8, 2), (8, 4), (16, 2)])
def test_window_gqa_ratios(dtype, n_rep, T):
    H = 32
    s = W.spec("c3", batch=3, n_heads=H, n_kv_heads=H // n_rep, max_seq_len=768,
               q_gain=4.0).replace(dtype=dtype)
    p = W.make_window(s, T, lengths=np.array([700, 129, T], np.int32))
    check_window(p, what=f"{dtype} n_rep={n_rep} T={T}")


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_window_rope_styles(style):
    s = W.spec("c3", batch=3, max_seq_len=256, q_gain=4.0)
    p = W.make_window(s, 4, lengths=np.array([4, 100, 256], np.int32))
    check_window(p, style=style, what=f"rope {style}")


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_single_token_equals_single_calls(dtype):
    """n_query = 1 through the multi calls = the single-token calls, bit for bit."""
    dev = device()
    s = _spec(dtype, False)
    p = W.make_problem(s, lengths=RAGGED)
    pw = W.make_window(s, 1, lengths=RAGGED)
    res = []
    for prob, multi in ((p, False), (pw, True)):
        t = upload(prob, dev)
        if multi:
            q_rot, out, lse = gpu_window(t, s, prob.max_len)
            res.append([q_rot[:, 0], out[:, 0], lse[:, 0], t["k_cache"], t["v_cache"]])
            continue
        t["q"], t["k_new"], t["v_new"] = (
            W.as_torch(np.ascontiguousarray(getattr(pw, k)[:, 0]), dev)
            for k in ("q", "k_new", "v_new"))
        from tests.gpu_helpers import gpu_step
        q_rot, out, lse = gpu_step(t, s, prob.max_len)
        res.append([q_rot, out, lse, t["k_cache"], t["v_cache"]])
    for a, b in zip(res[0], res[1]):      # bit patterns (the poisoned cache slots hold NaN)
        assert torch.equal(_bits(a), _bits(b))


def _bits(x):
    x = x.contiguous()
    return x.view({torch.bfloat16: torch.int16, torch.float32: torch.int32}.get(x.dtype, x.dtype))


def test_rejected_shapes():
    dev = device()
    k = torch.empty((2, 64, 2, 128), dtype=torch.bfloat16, device=dev)    # G = 2
    lens = torch.full((2,), 10, dtype=torch.int32, device=dev)
    q = torch.empty((2, 3, 32, 128), dtype=torch.float32, device=dev)    # n_rep 16, T 3: 48 rows
    with pytest.raises(kvd.KvdError):
        kvd.gqa_decode_attn_multi(q, k, k, lens, max_seq_len=64)
    kf = torch.empty((2, 64, 2, 128), dtype=torch.float32, device=dev)
    q2 = torch.empty((2, 2, 4, 128), dtype=torch.float32, device=dev)
    with pytest.raises(kvd.KvdError):                                    # fp32 cache, T > 1
        kvd.gqa_decode_attn_multi(q2, kf, kf, lens, max_seq_len=64)


def test_full_batched_window():
    """The batched workload (B 64, H 32, G 8, D 128, contexts U[512, 8192])
    with T = 5 new tokens per sequence: every row against the oracle, the
    caches in full."""
    dev = device()
    s = W.spec("c3")
    p = W.make_window(s, 5)
    print(f"[window full] B={s.batch} max_len={p.max_len}", flush=True)
    t = upload(p, dev)
    q_rot, out, lse = gpu_window(t, s, p.max_len)
    oq, oo, ol, okc, ovc = oracle_window(p)
    gates.assert_out(out.cpu().numpy(), oo, "bf16", "window full, all rows")
    gates.assert_lse(lse.cpu().numpy(), ol, "bf16", "window full, all rows lse")
    assert torch.equal(_bits(t["k_cache"]), _bits(W.as_torch(okc, dev)))
    assert torch.equal(_bits(t["v_cache"]), _bits(W.as_torch(ovc, dev)))
