"""GPU parity of the causal prefill (gqa_prefill_attn after
rope_append_kv_multi) against the oracle's multi-token step on the same
seeded inputs.

A prompt is the window of T new tokens on an empty history; a chunk of a
prompt is the same window after a cached history.  Query t attends the
tokens j < L_b - T + 1 + t ([KVGR] §5.1 b.v inside the window; the tiled
attention of [KVGR] §4.2).  The caches must match bit for bit; outputs and
lse pass the prefill gates (bf16 q and probabilities on the matrix cores:
max abs <= 1e-2, normwise <= 1e-2, lse <= 5e-3 relative).  Every case up to
a 2048-token prompt compares every element; the 8192-token prompt compares
4096 sampled (b, t, h) rows (the oracle takes each row's causal bound).
"""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import assert_q_rot, device, upload
from tests.test_gpu_multi import oracle_window, _bits

pytestmark = pytest.mark.gpu


def gpu_prefill(t, s: W.Spec, max_len: int, style="interleaved", options=None):
    sc = dict(k_scale=t["k_scale"], v_scale=t["v_scale"]) if s.dtype == "i8" else {}
    q_rot = kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["positions"], t["block_table"], base=s.rope_base,
                                     style=style, **sc)
    out, lse = kvd.gqa_prefill_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                    t["block_table"], max_seq_len=max_len, options=options, **sc)
    torch.cuda.synchronize()
    return q_rot, out, lse


def check_prefill(p: W.Problem, what="", units=None, style="interleaved", options=None):
    dev = device()
    s = p.spec
    print(f"[prefill] {what}", flush=True)
    t = upload(p, dev)
    q_rot, out, lse = gpu_prefill(t, s, p.max_len, style=style, options=options)
    oq, oo, ol, okc, ovc = oracle_window(p, style=style, units=units)
    assert torch.equal(_bits(t["k_cache"]), _bits(W.as_torch(okc, dev))), f"{what}: K cache"
    assert torch.equal(_bits(t["v_cache"]), _bits(W.as_torch(ovc, dev))), f"{what}: V cache"
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    if units is not None:
        ub, ut, uh = ([u[i] for u in units] for i in range(3))
        go, gl = go[ub, ut, uh], gl[ub, ut, uh]
    else:
        qr = q_rot.cpu().numpy()
        assert_q_rot(qr, oq, what)
    e = gates.assert_out(go, oo, "prefill", what)
    gates.assert_lse(gl, ol, "prefill", what)
    print(f"[prefill] {what}: {e}", flush=True)
    return e


def _spec(B, H, G, D, S, paged=False, block_size=16, q_gain=2.0, dtype="bf16"):
    if paged:
        s = W.spec("c4", batch=B, n_heads=H, n_kv_heads=G, head_dim=D,
                   num_blocks=B * (S // block_size) + 8, max_blocks_per_seq=S // block_size,
                   block_size=block_size, q_gain=q_gain, dtype=dtype)
    else:
        s = W.spec("c3", batch=B, n_heads=H, n_kv_heads=G, head_dim=D, max_seq_len=S,
                   q_gain=q_gain, dtype=dtype)
    return s


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 7, 32, 33, 100, 257])
def test_prompt_from_empty(D, T):
    """A whole prompt: no history, query t sees tokens 0 .. t."""
    s = _spec(2, 8, 2, D, 512)
    p = W.make_window(s, T, lengths=np.array([T, T], np.int32))
    check_prefill(p, what=f"prompt D={D} T={T}")


@pytest.mark.parametrize("T", [16, 64, 100])
@pytest.mark.parametrize("paged,block_size", [(False, 16), (True, 16), (True, 32)])
def test_chunk_after_history(T, paged, block_size):
    """A chunk of T tokens after ragged cached histories (the shortest has
    none)."""
    lens = np.array([T, T + 1, T + 15, T + 300, 900, 1024], np.int32)
    s = _spec(lens.size, 32, 8, 128, 1024, paged, block_size)
    p = W.make_window(s, T, lengths=lens)
    check_prefill(p, what=f"chunk T={T} paged={paged}/{block_size}")


@pytest.mark.parametrize("n_rep", [1, 2, 4, 8, 16, 32])
def test_gqa_ratios(n_rep):
    H = 32
    s = _spec(2, H, H // n_rep, 128, 640)
    p = W.make_window(s, 150, lengths=np.array([150, 600], np.int32))
    check_prefill(p, what=f"n_rep={n_rep}")


ORDERS = [kvd.PREFILL_PAIRS_FASTEST, kvd.PREFILL_TILES_FASTEST, kvd.PREFILL_XCD_RUNS]


@pytest.mark.parametrize("split", [0, 64])
@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("B,G,T,paged", [(3, 3, 300, False), (1, 1, 300, True),
                                         (1, 2, 40, False), (5, 8, 64, True)])
def test_dispatch_orders(order, B, G, T, paged, split):
    """Every workgroup order computes the same rows, with and without key
    splits: unit counts that are not a multiple of the XCD count, one pair,
    fewer workgroups than XCDs."""
    H = 4 * G
    lens = np.array([T + 37 * i for i in range(B)], np.int32)
    s = _spec(B, H, G, 128, 512, paged)
    p = W.make_window(s, T, lengths=lens)
    check_prefill(p, what=f"order {order} split {split} B={B} G={G} T={T} paged={paged}",
                  options=kvd.Options(dispatch_order=order, split_tokens=split))


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("split", [0, 64])
@pytest.mark.parametrize("B", [8, 64])
def test_xcd_runs_balanced_by_length(dtype, split, B):
    """Contiguous runs per XCD with the batch a multiple of the XCD count:
    the unit list takes the sequences in an order dealt by length, so the
    runs carry equal work.  Lengths in no particular order, with ties and
    chunks on an empty history; every row against the oracle, and the same
    bits as the order that deals a pair's tiles round-robin."""
    T = 40
    rng = np.random.default_rng(B + split)
    lens = rng.integers(T, 400, B).astype(np.int32)
    lens[: B // 4] = lens[B // 4: B // 2]
    lens[-1] = T
    rng.shuffle(lens)
    s = _spec(B, 8, 2, 128, 512, dtype=dtype)
    p = W.make_window(s, T, lengths=lens)
    what = f"{dtype} B={B} split {split}"
    check_prefill(p, what=f"XCD runs {what}",
                  options=kvd.Options(dispatch_order=kvd.PREFILL_XCD_RUNS, split_tokens=split))
    dev = device()
    res = []
    for order in (kvd.PREFILL_TILES_FASTEST, kvd.PREFILL_XCD_RUNS):
        t = upload(p, dev)
        _, out, lse = gpu_prefill(t, s, p.max_len,
                                  options=kvd.Options(dispatch_order=order, split_tokens=split))
        res.append((out.cpu(), lse.cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), what


@pytest.mark.parametrize("split", [32, 96, 2048])
@pytest.mark.parametrize("paged,block_size", [(False, 16), (True, 32)])
def test_key_split_forced(split, paged, block_size):
    """Key splits of `split` tokens merged by their log-sum-exp: rows whose
    bound lies before a split's start (empty partials), sequences that end
    before the longest (splits past their end are never read), a sequence
    with no history, split boundaries inside the window."""
    T = 100
    lens = np.array([T, T + 31, T + 500, 1024, 1200], np.int32)
    s = _spec(lens.size, 32, 8, 128, 1280, paged, block_size)
    p = W.make_window(s, T, lengths=lens)
    check_prefill(p, what=f"split {split} paged={paged}/{block_size}",
                  options=kvd.Options(split_tokens=split))


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("paged,block_size,split", [(False, 16, 64), (True, 16, 0), (True, 32, 96)])
def test_head_dim_64_chunks(dtype, paged, block_size, split):
    """D = 64 (its own LDS layouts: 128-byte rows, another swizzle) on chunks
    after ragged histories, contiguous and paged, with and without key
    splits, on both cache dtypes."""
    T = 100
    lens = np.array([T, T + 17, T + 400, 1000], np.int32)
    s = _spec(lens.size, 16, 4, 64, 1024, paged, block_size, dtype=dtype)
    p = W.make_window(s, T, lengths=lens)
    check_prefill(p, what=f"D=64 {dtype} paged={paged}/{block_size} split={split}",
                  options=kvd.Options(split_tokens=split))


def test_key_split_automatic_long_history():
    """A 64-token chunk after a 20K history, one sequence and two KV heads:
    four query tiles cannot fill the device, so the library splits the keys
    (it asks for a workspace); every row against the oracle."""
    T, L = 64, 20480
    s = _spec(1, 8, 2, 128, L)
    p = W.make_window(s, T, lengths=np.array([L], np.int32))
    k = torch.empty((1, L, 2, 128), dtype=torch.bfloat16, device=device())
    assert kvd.prefill_workspace_size(1, 8, T, k, max_seq_len=L) > 0
    check_prefill(p, what="chunk 64 after 20K, automatic split")


def test_key_split_128k_history_sampled():
    """A 512-token chunk after a 128K history at the 128K workload's head
    shape (H 32, G 8, D 128), split automatically: 1024 sampled rows (the
    first and last tokens of every query tile among them) against the
    oracle, caches in full."""
    s = W.spec("c5", q_gain=2.0)
    T, L = 512, s.max_seq_len
    p = W.make_window(s, T, lengths=np.array([L], np.int32))
    rng = np.random.default_rng(72)
    edges = np.r_[np.arange(0, T, 128 // 4), np.arange(31, T, 128 // 4)]
    ts = np.r_[edges, rng.integers(0, T, 1024 - edges.size)]
    units = [(0, int(t), int(h)) for t, h in zip(ts, rng.integers(0, s.n_heads, ts.size))]
    check_prefill(p, units=units, what="chunk 512 after 128K, 1024 rows")


@pytest.mark.parametrize("q_gain", [1.0, 8.0, 32.0])
def test_peaked_scores(q_gain):
    s = _spec(2, 32, 8, 128, 1024, q_gain=q_gain)
    p = W.make_window(s, 200, lengths=np.array([200, 1000], np.int32))
    check_prefill(p, what=f"q_gain={q_gain}")


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_rope_styles(style):
    s = _spec(2, 16, 4, 128, 256)
    p = W.make_window(s, 64, lengths=np.array([64, 256], np.int32))
    check_prefill(p, style=style, what=f"rope {style}")


def test_matches_decode_multi_within_gates():
    """For windows the decode kernels take (n_rep * T <= 32) the prefill and
    the decode kernel agree within the prefill gate."""
    dev = device()
    s = _spec(4, 32, 8, 128, 1024)
    p = W.make_window(s, 5, lengths=np.array([5, 100, 640, 1024], np.int32))
    t = upload(p, dev)
    q_rot = kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["positions"])
    o1, l1 = kvd.gqa_prefill_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"])
    o2, l2 = kvd.gqa_decode_attn_multi(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"])
    torch.cuda.synchronize()
    gates.assert_out(o1.cpu().numpy(), o2.cpu().numpy(), "prefill", "prefill vs decode")
    gates.assert_lse(l1.cpu().numpy(), l2.cpu().numpy(), "prefill", "prefill vs decode lse")


def test_zero_and_short_lengths():
    """seq_lens below T (queries that see nothing) give out = 0, lse = -inf
    for those queries, and the others match the oracle's bounds."""
    dev = device()
    s = _spec(3, 8, 2, 64, 128)
    T = 10
    p = W.make_window(s, T, lengths=np.array([T, 50, 128], np.int32))
    t = upload(p, dev)
    q_rot = kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["positions"])
    lens = torch.tensor([0, 4, 128], dtype=torch.int32, device=dev)
    out, lse = kvd.gqa_prefill_attn(q_rot, t["k_cache"], t["v_cache"], lens, max_seq_len=128)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert (o[0] == 0).all() and np.isneginf(l[0]).all()
    # length 4 with T = 10: queries 0 .. 5 see nothing, query t >= 6 sees t - 5 tokens
    assert (o[1, :6] == 0).all() and np.isneginf(l[1, :6]).all()
    assert np.isfinite(l[1, 6:]).all() and np.isfinite(o[2]).all()


def test_prompt_2048_every_row():
    """A 2048-token prompt at the 128K workload's head shape (H 32, G 8,
    D 128): every output row and lse against the oracle, caches in full."""
    T = 2048
    s = W.spec("c5", max_seq_len=T, q_gain=2.0)
    p = W.make_window(s, T, lengths=np.array([T], np.int32))
    check_prefill(p, what="prompt 2048, all rows")


def test_long_prompt_sampled():
    """An 8192-token prompt at the same head shape: 4096 sampled rows (the
    first and last tokens of every 128-row query tile among them) against the
    oracle, caches in full."""
    T = 8192
    s = W.spec("c5", max_seq_len=T, q_gain=2.0)
    p = W.make_window(s, T, lengths=np.array([T], np.int32))
    rng = np.random.default_rng(71)
    edges = np.r_[np.arange(0, T, 128), np.arange(127, T, 128)]
    ts = np.r_[edges, rng.integers(0, T, 4096 - edges.size)]
    units = [(0, int(t), int(h)) for t, h in zip(ts, rng.integers(0, s.n_heads, ts.size))]
    check_prefill(p, units=units, what="prompt 8192, 4096 rows")


# INT8 caches ([KVGR] §4.3): codes with per-head scales, converted once per
# tile to exact fp16; q and P rounded to fp16 (finer than the bf16 prefill's
# bf16), so the prefill gates apply.  The caches (codes of the appended
# window) must match bit for bit.

@pytest.mark.parametrize("D,T", [(64, 1), (64, 100), (128, 33), (128, 257)])
def test_int8_prompt_from_empty(D, T):
    s = _spec(2, 8, 2, D, 512, dtype="i8")
    p = W.make_window(s, T, lengths=np.array([T, T], np.int32))
    check_prefill(p, what=f"INT8 prompt D={D} T={T}")


@pytest.mark.parametrize("paged,block_size", [(False, 16), (True, 16), (True, 32)])
@pytest.mark.parametrize("split", [0, 64])
def test_int8_chunk_after_history(paged, block_size, split):
    T = 100
    lens = np.array([T, T + 1, T + 15, T + 300, 900, 1024], np.int32)
    s = _spec(lens.size, 32, 8, 128, 1024, paged, block_size, dtype="i8")
    p = W.make_window(s, T, lengths=lens)
    check_prefill(p, what=f"INT8 chunk paged={paged}/{block_size} split={split}",
                  options=kvd.Options(split_tokens=split))


@pytest.mark.parametrize("n_rep", [1, 4, 32])
def test_int8_gqa_ratios_and_orders(n_rep):
    H = 32
    s = _spec(2, H, H // n_rep, 128, 640, dtype="i8")
    p = W.make_window(s, 150, lengths=np.array([150, 600], np.int32))
    for order in ORDERS:
        check_prefill(p, what=f"INT8 n_rep={n_rep} order {order}",
                      options=kvd.Options(dispatch_order=order))


def test_int8_peaked_scores():
    s = _spec(2, 32, 8, 128, 1024, q_gain=16.0, dtype="i8")
    p = W.make_window(s, 200, lengths=np.array([400, 1024], np.int32))
    check_prefill(p, what="INT8 peaked")


def test_int8_prompt_2048_every_row():
    T = 2048
    s = W.spec("c5", max_seq_len=T, q_gain=2.0, dtype="i8")
    p = W.make_window(s, T, lengths=np.array([T], np.int32))
    check_prefill(p, what="INT8 prompt 2048, all rows")


def test_int8_key_split_after_long_history():
    """A 64-token chunk after a 20K history: split automatically."""
    T, L = 64, 20480
    s = _spec(1, 8, 2, 128, L, dtype="i8")
    p = W.make_window(s, T, lengths=np.array([L], np.int32))
    check_prefill(p, what="INT8 chunk 64 after 20K, automatic split")
